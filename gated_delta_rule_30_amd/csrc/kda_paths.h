// Internal host-side declarations of the library's other chunked paths (not part of the C
// ABI): the chunk-parallel scan, the fp32 chunk table, the wide-key forward and the training
// backward. Kept apart from kda_internal.h, which describes the main forward and decode.
#pragma once

#include "kda_internal.h"

namespace kda {

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
bool make_wide_plan(int num_seqs, int64_t total_tokens, int num_heads, int dk, int dv,
                    WidePlan* p);
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
