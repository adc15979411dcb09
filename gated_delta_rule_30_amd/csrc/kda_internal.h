// Internal host-side declarations of the KDA library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int CHUNK = 64;     // tokens per chunk
constexpr int SUBBLK = 16;    // sub-block edge = MFMA tile edge
constexpr int NSUB = CHUNK / SUBBLK;
constexpr int NTHREADS = 256;  // threads per workgroup of every chunk kernel

// Input option bits (the KDA_OPT_* values of the C ABI).
constexpr uint32_t OPT_SCALAR_GATE = 1u, OPT_GATE_LOGITS = 2u, OPT_BETA_LOGITS = 4u,
                   OPT_L2NORM_QK = 8u;
// Added to the sum of squares before the L2 normalisation of q and k.
constexpr float L2NORM_EPS = 1e-6f;

// Target number of (chunk, head) records per segment: the segment's record buffer (66 KB per
// record at K=V=128 bf16, 135 MB) then stays resident in the 256 MB Infinity Cache.
constexpr int64_t SEG_CHUNK_HEADS = 2048;

struct DecodeArgs {
  const void *q, *k, *v, *g, *beta;
  float* state;
  void* o;
  int num_seqs, num_heads, dk, dv;
  bool dtype_bf16;
  uint32_t options;  // KDA_OPT_* bits
  void* stream;
};

// One entry of the device chunk table (32 bytes).
struct Entry {
  int32_t seq;    // sequence index
  int32_t tok;    // first token (packed index)
  int32_t len;    // tokens in this chunk, 1..CHUNK
  int32_t depth;  // chunk index inside its sequence
  int32_t prev;   // entry index of the previous chunk of the sequence, -1 if none
  int32_t next;   // entry index of the next chunk of the sequence, -1 if none
  int32_t end;    // one past the last token of the sequence (packed index)
  int32_t pad;
};

// Host-side launch plan of one kda_chunk_fwd call; a pure function of the shape.
struct ChunkPlan {
  int64_t ub_entries;   // upper bound of the number of chunks over all sequences
  int64_t seg_entries;  // E: chunks per segment
  int64_t num_segs;
  int64_t slots;        // max distinct sequences in one segment = min(N, E)
  int64_t rec_bytes;    // bytes of one (chunk, head) record
  int n_slices;         // V split into n_slices slices of vs columns
  int vs;
  // workspace offsets (bytes)
  size_t off_header, off_entries, off_basetab, off_seg_first, off_seg_count, off_state,
      off_rec, rec_buf_bytes;
  size_t total_bytes;
};

bool make_chunk_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                     bool bf16, ChunkPlan* p);

struct ChunkArgs {
  const void *q, *k, *v, *g, *beta;
  const float* init_state;
  const int32_t* cu_seqlens;
  int num_seqs;
  int64_t total_tokens;
  int num_heads, dk, dv;
  bool dtype_bf16;
  uint32_t options;  // KDA_OPT_* bits
  void* o;
  float* final_state;
  void* workspace;
  void* stream;
};

hipError_t launch_decode(const DecodeArgs& a);
// Where a chunked pass keeps its (chunk, head) records when the caller wants them to outlive
// it: base holds one slot of seg_entries * num_heads * rec_bytes per segment; prep = false
// skips the record-building kernel because an earlier pass over the same chunks (with at
// least as many value columns) left them there.
struct RecordRegion {
  char* base;
  int64_t rec_bytes;
  bool prep;
};
hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkPlan& p,
                            const RecordRegion* records = nullptr);

// Chunk-parallel scan over equal-length sequences split into G groups of whole chunks: a pass
// over the groups with V + K state columns, a combine, and a pass from the groups' initial
// states that reuses the first pass's records. Workspace: the chunk workspace of the larger
// pass with every segment's records, [v | 0], its scratch output, [0 | I], the groups'
// [B | M], their initial states and the group boundaries.
struct ScanPlan {
  int64_t L, Lg;       // tokens per sequence and per group
  ChunkPlan p1, p3;    // the two chunk passes (N * G sequences; V + K and V columns)
  size_t rec_region_bytes;  // every segment's records of the first pass, kept for the second
  size_t off_ws, off_vaug, off_oaug, off_init1, off_fin1, off_sin, off_cu, off_dummy,
      total_bytes;
};
bool make_scan_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv, bool bf16,
                    int groups, ScanPlan* p);
hipError_t launch_chunk_fwd_scan(const ChunkArgs& a, int groups, const ScanPlan& p);

// One chunk of the fp32 chunk machinery's table: its sequence, first token and length.
struct ChunkRow {
  int32_t seq, tok, len, pad;
};
// seq_first[n] = the first chunk of sequence n (seq_first[N] = the number of chunks) and the
// rows of every chunk, for N sequences (cu_seqlens, or equal lengths T / N when cu is null).
hipError_t launch_chunk_rows(const int32_t* cu, int N, int64_t T, int64_t ub, int32_t* seq_first,
                             ChunkRow* rows, hipStream_t st);

// Chunked forward at 256 key channels (kda_wide.hip): fp32 records for every chunk at once.
struct WidePlan {
  int64_t ub;  // upper bound of the number of chunks over all sequences
  size_t off_seq, off_rows, off_rec, total_bytes;
};
bool make_wide_plan(int num_seqs, int64_t total_tokens, int num_heads, int dv, WidePlan* p);
hipError_t launch_chunk_fwd_wide(const ChunkArgs& a, const WidePlan& p);

// Training backward (kda_bwd.hip): per chunk and head an fp32 record, the chunk-start states,
// the chunk-end state gradients, Delta, dDelta and the gradient kernels' scratch, for every
// chunk at once.
struct BwdPlan {
  int64_t ub;  // upper bound of the number of chunks over all sequences
  size_t off_seq, off_chunks, off_rec, off_ckS, off_ckX, off_D, off_dD, off_scr, total_bytes;
};
bool make_bwd_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv, BwdPlan* p);

struct BwdArgs {
  const void *q, *k, *v, *g, *beta;
  const float* init_state;
  const int32_t* cu_seqlens;
  int num_seqs;
  int64_t total_tokens;
  int num_heads, dk, dv;
  bool dtype_bf16;
  const void* dO;
  const float* dfinal;
  float *grad_q, *grad_k, *grad_v, *grad_g, *grad_beta, *grad_init;
  void* workspace;
  void* stream;
};
hipError_t launch_chunk_bwd(const BwdArgs& a, const BwdPlan& p);

}  // namespace kda
