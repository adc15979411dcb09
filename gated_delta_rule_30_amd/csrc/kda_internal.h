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
  int seq_major;        // chunk table order: 1 sequence-major (token order), 0 depth-major
  // workspace offsets (bytes)
  size_t off_header, off_entries, off_basetab, off_seg_first, off_seg_count, off_state,
      off_rec, rec_buf_bytes;
  size_t total_bytes;
};

// max_rec_buf_bytes > 0 caps the record buffer (fewer chunks per segment; false if not even
// one chunk of every head fits); running_state = false leaves out the running state, which a
// call with a final_state buffer does not use.
bool make_chunk_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                     bool bf16, ChunkPlan* p, size_t max_rec_buf_bytes = 0,
                     bool running_state = true);

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
  // with a sequence-major chunk table: per segment boundary s + 1 (entry (s + 1) E, E chunks per
  // segment) the state before that chunk of the sequence it belongs to, [s][H][K][V], when the
  // chunk is not the sequence's first (no slot is written otherwise); nullptr: none
  float* ckpt = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a);
// Compute units of the current device (queried once per device, then cached).
int device_cu_count();
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

// The chunk records at 256 key channels (bf16 inputs, no input options), for entries
// [seg_begin, seg_begin + E) of the chunk table, written by an fp32 record kernel
// (kda_wide.hip) in the layout the state kernel reads.
struct Rec256Params {
  const void *q, *k, *v, *g, *beta;
  const Entry* entries;
  const int32_t* header;
  int H, V;
  int64_t seg_begin, E;
  char* rec;
  int64_t rec_bytes;
  uint32_t opts;  // input option bits (OPT_*)
};
void launch_rec256(const Rec256Params& p, hipStream_t st);

}  // namespace kda
