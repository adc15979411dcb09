// Internal host-side declarations of the library's other chunked paths (not part of the C
// ABI): the chunk-parallel scan, the fp32 chunk table, the wide-key forward and the training
// backward. Kept apart from kda_internal.h, which describes the main forward and decode.
#pragma once

#include "../../include/kda.h"
#include "kda_internal.h"

namespace kda {

// The argument checks of kda_chunk_fwd_ex that do not involve the workspace; on success *a
// holds the launch arguments with workspace = nullptr.
kda_status prepare_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* init_state, const int32_t* cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                             int32_t dv, kda_dtype dtype, uint32_t options, void* o,
                             float* final_state, void* stream, ChunkArgs* a);
// Whether kda_chunk_fwd_ex runs this head dim, dtype and options on the wide-key path
// (kda_wide.hip).
bool is_wide_path(int32_t dk, kda_dtype dtype, uint32_t options);

// Chunk-parallel scan over equal-length sequences split into G groups of whole chunks: a pass
// over the groups with V + K state columns, a combine, and a pass from the groups' initial
// states that reuses the first pass's records. Workspace: the chunk workspace of the larger
// pass with every segment's records, [v | 0], its scratch output, [0 | I], the groups'
// [B | M], their initial states and the group boundaries.
struct ScanPlan {
  int64_t L, Lg;       // tokens per sequence and per group
  int W;               // value columns of the first pass: V + K, rounded up to a power of two
  ChunkPlan p1, p3;    // the two chunk passes (N * G sequences; W and V columns)
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

// Input options as a pass of their own (kda_prologue.hip), for the paths whose kernels read
// plain inputs. launch_prologue writes the processed q, k, log alpha ([rows][H][K]) and beta
// ([rows][H]) in fp32: every token of the call at its own row (chunks = nullptr), or the
// tokens of chunks [cb, ce) from row 0 (max_rows bounds their number, for the grid).
// launch_bwd_epilogue turns gradients with respect to the processed inputs into gradients
// with respect to the raw ones (grad_q, grad_k, grad_beta in place; dg [T][H][K] into grad_g,
// which is [T][H] with the scalar gate).
struct OptInputs {
  const void *q, *k, *g, *beta;
};
struct OptBuffers {
  float *q, *k, *g, *beta;
};
void launch_prologue(const OptInputs& in, bool bf16, int64_t T, int H, int K, uint32_t options,
                     const ChunkRow* chunks, const int32_t* ntot, int cb, int ce,
                     const OptBuffers& out, hipStream_t st, int64_t max_rows);
void launch_bwd_epilogue(const OptInputs& in, bool bf16, int64_t T, int H, int K,
                         uint32_t options, float* grad_q, float* grad_k, const float* dg,
                         float* grad_g, float* grad_beta, hipStream_t st);

// Chunked forward at 256 key channels (kda_wide.hip): fp32 records for one segment of chunks
// at a time (segments run in order, the state carried between them), and the input-option
// pass's output for one segment's tokens.
struct WidePlan {
  int64_t ub;    // upper bound of the number of chunks over all sequences
  int64_t seg;   // chunks per segment
  int64_t nseg;  // segments (at least one)
  size_t off_seq, off_rows, off_rec, off_opt_q, off_opt_k, off_opt_g, off_opt_b, off_run,
      total_bytes;
};
// Record bytes per segment.
constexpr size_t WIDE_SEGMENT_BYTES = (size_t)512 << 20;
bool make_wide_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                    WidePlan* p);
hipError_t launch_chunk_fwd_wide(const ChunkArgs& a, const WidePlan& p);

// Training backward (kda_bwd.hip): per chunk and head of a segment an fp32 record, the
// chunk-start state, the chunk-end state gradient, Delta, dDelta and the gradient kernels'
// scratch, plus one [H][K][V] state per segment boundary. Segments of `seg` chunks run
// backwards; with more than one, a forward pass over the records first leaves the state at
// every boundary.
struct BwdPlan {
  int64_t ub;    // upper bound of the number of chunks over all sequences
  int64_t seg;   // chunks per segment
  int64_t nseg;  // segments (at least one)
  size_t off_opt_q, off_opt_k, off_opt_g, off_opt_b, off_opt_dg;  // input options only
  size_t off_seq, off_chunks, off_ck, off_rec, off_ckS, off_ckX, off_D, off_dD, off_scr,
      total_bytes;
};
// Per-segment bytes of the default plan (kda_chunk_bwd_workspace_size).
constexpr size_t BWD_SEGMENT_BYTES = (size_t)4 << 30;
// seg_chunks <= 0 (or >= the chunk count): one segment
bool make_bwd_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                   uint32_t options, int64_t seg_chunks, BwdPlan* p);
// The plan with the longest segments whose workspace fits in `bytes` (false if none does).
// The longest segments that fit in bytes; with step > 1, several segments are each a multiple
// of step chunks long.
bool fit_bwd_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                  uint32_t options, size_t bytes, BwdPlan* p, int64_t step = 1);
// Chunks per segment of the default plan.
int64_t default_bwd_segment(int num_heads, int dk, int dv);

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
  uint32_t options;  // KDA_OPT_* bits
  void* workspace;
  void* stream;
  // the forward's checkpoint states (ChunkArgs::ckpt, every ckpt_interval chunks); the plan's
  // segments are then multiples of ckpt_interval and no boundary pass runs. nullptr: none
  const float* ckpt = nullptr;
  int64_t ckpt_interval = 0;
};
hipError_t launch_chunk_bwd(const BwdArgs& a, const BwdPlan& p);

}  // namespace kda
