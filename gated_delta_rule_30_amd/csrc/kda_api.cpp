// C ABI of libkda.so: argument validation, workspace planning and launch.
// Every check here runs on the host before anything is enqueued.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include "kda_paths.h"

namespace {

bool supported_dim(int32_t d) { return d == 32 || d == 64 || d == 128 || d == 256; }
// the chunk path's prep kernel holds K-wide operand tiles in LDS: K <= 128 (K = 256 runs an
// fp32 record kernel with the key channels in parts of 64 instead)
bool supported_chunk_dk(int32_t d) { return d == 32 || d == 64 || d == 128; }
constexpr int32_t kWideDk = 256;
// the fp32 wide-key path: fp32 inputs at K >= 128 (bf16 inputs at K = 256, with or without
// input options, run the chunk path: an fp32 record kernel and the bf16 chain)
bool wide_path(int32_t dk, kda_dtype dtype, uint32_t) {
  return dtype == KDA_DTYPE_F32 && (dk == kWideDk || dk == 128);
}
constexpr uint32_t kAllOptions =
    KDA_OPT_SCALAR_GATE | KDA_OPT_GATE_LOGITS | KDA_OPT_BETA_LOGITS | KDA_OPT_L2NORM_QK;
static_assert(KDA_OPT_SCALAR_GATE == kda::OPT_SCALAR_GATE && KDA_OPT_GATE_LOGITS == kda::OPT_GATE_LOGITS &&
                  KDA_OPT_BETA_LOGITS == kda::OPT_BETA_LOGITS && KDA_OPT_L2NORM_QK == kda::OPT_L2NORM_QK,
              "option bits of the ABI and the kernels");
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_dtype(kda_dtype t) { return t == KDA_DTYPE_F32 || t == KDA_DTYPE_BF16; }
size_t esize(kda_dtype t) { return t == KDA_DTYPE_BF16 ? 2 : 4; }

// [a, a+na) and [b, b+nb) overlap
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Largest packed token count the 32-bit chunk table indexes.
constexpr int64_t kMaxTokens = (int64_t)1 << 30;

}  // namespace

extern "C" const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
    case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
    case KDA_ERROR_WORKSPACE_TOO_SMALL: return "KDA_ERROR_WORKSPACE_TOO_SMALL";
    case KDA_ERROR_LAUNCH: return "KDA_ERROR_LAUNCH";
  }
  return "KDA_ERROR_UNKNOWN";
}

static kda_status check_chunk_shape(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype) {
  if (num_seqs <= 0 || num_heads <= 0 || total_tokens < 0 || total_tokens > kMaxTokens)
    return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(dtype) || !(supported_chunk_dk(dk) || dk == kWideDk) || !supported_dim(dv))
    return KDA_ERROR_NOT_SUPPORTED;
  return KDA_SUCCESS;
}

extern "C" size_t kda_chunk_fwd_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                               int32_t num_heads, int32_t dk, int32_t dv,
                                               kda_dtype dtype) {
  if (check_chunk_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype) != KDA_SUCCESS) return 0;
  size_t need = 0;
  if (wide_path(dk, dtype, 0u)) {
    kda::WidePlan wp;
    if (!kda::make_wide_plan(num_seqs, total_tokens, num_heads, dk, dv, &wp)) return 0;
    need = wp.total_bytes;
  }
  if (!wide_path(dk, dtype, 0u)) {
    kda::ChunkPlan pl;
    if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_DTYPE_BF16, &pl))
      return 0;
    need = pl.total_bytes > need ? pl.total_bytes : need;
  }
  return need;
}

// Everything kda_chunk_fwd_ex checks before it looks at the workspace; fills the launch
// arguments (all but the workspace).
kda_status kda::prepare_chunk_fwd(const void* q, const void* k, const void* v,
                                  const void* log_alpha, const void* beta,
                                  const float* init_state, const int32_t* cu_seqlens,
                                  int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype, uint32_t options,
                                  void* o, float* final_state, void* stream, ChunkArgs* a) {
  kda_status st = check_chunk_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (st != KDA_SUCCESS) return st;
  if (options & ~kAllOptions) return KDA_ERROR_NOT_SUPPORTED;
  const int32_t gdim = (options & KDA_OPT_SCALAR_GATE) ? 1 : dk;  // gate values per token and head
  if (cu_seqlens == nullptr && total_tokens % num_seqs != 0) return KDA_ERROR_INVALID_VALUE;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERROR_INVALID_VALUE;
  // vectors of K or V elements need 16 bytes; per-token scalars (beta, a scalar gate) their element
  const bool scalar_gate = (options & KDA_OPT_SCALAR_GATE) != 0;
  const void* ptrs[] = {q, k, v, scalar_gate ? nullptr : log_alpha, init_state, o, final_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
  if ((beta && !aligned_to(beta, esize(dtype))) || (cu_seqlens && !aligned_to(cu_seqlens, 4)) ||
      (log_alpha && !aligned_to(log_alpha, esize(dtype))))
    return KDA_ERROR_INVALID_VALUE;
  const size_t sbytes = (size_t)num_seqs * num_heads * dk * dv * sizeof(float);
  if (init_state && final_state && init_state != final_state &&
      overlap(init_state, sbytes, final_state, sbytes))
    return KDA_ERROR_INVALID_VALUE;
  if (total_tokens > 0) {
    const size_t obytes = (size_t)total_tokens * num_heads * dv * esize(dtype);
    const size_t ibytes = (size_t)total_tokens * num_heads * dk * esize(dtype);
    const size_t gbytes = (size_t)total_tokens * num_heads * gdim * esize(dtype);
    if (overlap(o, obytes, q, ibytes) || overlap(o, obytes, k, ibytes) ||
        overlap(o, obytes, log_alpha, gbytes) || overlap(o, obytes, v, obytes))
      return KDA_ERROR_INVALID_VALUE;
  }
  a->q = q;
  a->k = k;
  a->v = v;
  a->g = log_alpha;
  a->beta = beta;
  a->init_state = init_state;
  a->cu_seqlens = cu_seqlens;
  a->num_seqs = num_seqs;
  a->total_tokens = total_tokens;
  a->num_heads = num_heads;
  a->dk = dk;
  a->dv = dv;
  a->dtype_bf16 = dtype == KDA_DTYPE_BF16;
  a->options = options;
  a->o = o;
  a->final_state = final_state;
  a->workspace = nullptr;
  a->stream = stream;
  return KDA_SUCCESS;
}

bool kda::is_wide_path(int32_t dk, kda_dtype dtype, uint32_t options) {
  return wide_path(dk, dtype, options);
}

extern "C" kda_status kda_chunk_fwd_ex(const void* q, const void* k, const void* v,
                                       const void* log_alpha, const void* beta,
                                       const float* init_state, const int32_t* cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                       int32_t dk, int32_t dv, kda_dtype dtype, uint32_t options,
                                       void* o, float* final_state, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  kda::ChunkArgs a;
  kda_status st = kda::prepare_chunk_fwd(q, k, v, log_alpha, beta, init_state, cu_seqlens,
                                         num_seqs, total_tokens, num_heads, dk, dv, dtype, options,
                                         o, final_state, stream, &a);
  if (st != KDA_SUCCESS) return st;
  if (!workspace) return KDA_ERROR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERROR_INVALID_VALUE;
  kda::ChunkPlan pl;
  kda::WidePlan wp;
  const bool wide = wide_path(dk, dtype, options);
  if (wide) {
    if (!kda::make_wide_plan(num_seqs, total_tokens, num_heads, dk, dv, &wp)) return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes < wp.total_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  } else {
    if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_DTYPE_BF16, &pl))
      return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes < pl.total_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  }
  a.workspace = workspace;
  hipError_t e = wide ? kda::launch_chunk_fwd_wide(a, wp) : kda::launch_chunk_fwd(a, pl);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}

// Chunks between the forward's checkpoints: its segment length (entries of the chunk table).
static int64_t ckpt_interval(int32_t num_seqs, int64_t total_tokens, int32_t num_heads) {
  kda::ChunkPlan pl;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, 32, 32, true, &pl)) return 0;
  return pl.seg_entries;
}
static size_t ckpt_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                         int32_t dv) {
  kda::ChunkPlan pl;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, 32, 32, true, &pl)) return 0;
  const int64_t slots = pl.num_segs > 1 ? pl.num_segs - 1 : 0;
  return (size_t)slots * num_heads * dk * dv * sizeof(float);
}

extern "C" kda_status kda_chunk_fwd_ckpt(const void* q, const void* k, const void* v,
                                         const void* log_alpha, const void* beta,
                                         const float* init_state, const int32_t* cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens,
                                         int32_t num_heads, int32_t dk, int32_t dv,
                                         kda_dtype dtype, uint32_t options, void* o,
                                         float* final_state, float* checkpoints, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  kda::ChunkArgs a;
  kda_status st = kda::prepare_chunk_fwd(q, k, v, log_alpha, beta, init_state, cu_seqlens,
                                         num_seqs, total_tokens, num_heads, dk, dv, dtype, options,
                                         o, final_state, stream, &a);
  if (st != KDA_SUCCESS) return st;
  // the shapes the training backward takes, on the chunk path
  if (!supported_chunk_dk(dk) || !(supported_chunk_dk(dv) || dv == 256) ||
      wide_path(dk, dtype, options))
    return KDA_ERROR_NOT_SUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return KDA_ERROR_INVALID_VALUE;
  const size_t cb = ckpt_bytes(num_seqs, total_tokens, num_heads, dk, dv);
  if (cb > 0) {
    if (!checkpoints || !aligned16(checkpoints)) return KDA_ERROR_INVALID_VALUE;
    const size_t es = esize(dtype), T = (size_t)total_tokens, H = (size_t)num_heads;
    const size_t gd = (options & KDA_OPT_SCALAR_GATE) ? 1 : (size_t)dk;
    const size_t sbytes = (size_t)num_seqs * H * dk * dv * sizeof(float);
    const void* bp[] = {q, k, v, log_alpha, beta, o, init_state, final_state};
    const size_t bn[] = {T * H * dk * es, T * H * dk * es, T * H * dv * es, T * H * gd * es,
                         T * H * es, T * H * dv * es, sbytes, sbytes};
    for (int i = 0; i < 8; ++i)
      if (bp[i] && bn[i] && overlap(checkpoints, cb, bp[i], bn[i])) return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes && overlap(checkpoints, cb, workspace, workspace_bytes))
      return KDA_ERROR_INVALID_VALUE;
  }
  kda::ChunkPlan pl;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_DTYPE_BF16, &pl))
    return KDA_ERROR_INVALID_VALUE;
  if (workspace_bytes < pl.total_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  // segments along token order, so that each segment boundary is a chunk of one sequence
  pl.seq_major = 1;
  a.workspace = workspace;
  a.ckpt = cb > 0 ? checkpoints : nullptr;
  hipError_t e = kda::launch_chunk_fwd(a, pl);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}

extern "C" kda_status kda_chunk_fwd(const void* q, const void* k, const void* v,
                                    const void* log_alpha, const void* beta,
                                    const float* init_state, const int32_t* cu_seqlens,
                                    int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype, void* o,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return kda_chunk_fwd_ex(q, k, v, log_alpha, beta, init_state, cu_seqlens, num_seqs,
                          total_tokens, num_heads, dk, dv, dtype, 0u, o, final_state, workspace,
                          workspace_bytes, stream);
}

// ---------------------------------------------------------------- training backward
static kda_status check_bwd_shape(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype) {
  if (num_seqs <= 0 || num_heads <= 0 || total_tokens < 0 || total_tokens > kMaxTokens)
    return KDA_ERROR_INVALID_VALUE;
  // K <= 128 (the record kernel's and gradient kernels' channel parts); V up to 256 (value
  // columns in parts of 64)
  if (!valid_dtype(dtype) || !supported_chunk_dk(dk) || !(supported_chunk_dk(dv) || dv == 256))
    return KDA_ERROR_NOT_SUPPORTED;
  return KDA_SUCCESS;
}

extern "C" size_t kda_chunk_bwd_workspace_size_ex(int32_t num_seqs, int64_t total_tokens,
                                                  int32_t num_heads, int32_t dk, int32_t dv,
                                                  kda_dtype dtype, uint32_t options,
                                                  int64_t segment_tokens) {
  if (check_bwd_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype) != KDA_SUCCESS) return 0;
  if (options & ~kAllOptions) return 0;
  kda::BwdPlan p;
  const int64_t seg = segment_tokens < 0    ? kda::default_bwd_segment(num_heads, dk, dv)
                      : segment_tokens == 0 ? 0
                                            : (segment_tokens + kda::CHUNK - 1) / kda::CHUNK;
  if (!kda::make_bwd_plan(num_seqs, total_tokens, num_heads, dk, dv, options, seg, &p)) return 0;
  return p.total_bytes;
}

extern "C" size_t kda_chunk_bwd_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                               int32_t num_heads, int32_t dk, int32_t dv,
                                               kda_dtype dtype) {
  if (check_bwd_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype) != KDA_SUCCESS) return 0;
  kda::BwdPlan p;
  if (!kda::make_bwd_plan(num_seqs, total_tokens, num_heads, dk, dv, 0u,
                          kda::default_bwd_segment(num_heads, dk, dv), &p))
    return 0;
  return p.total_bytes;
}

static kda_status chunk_bwd_impl(const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta,
                                 const float* init_state, const int32_t* cu_seqlens,
                                 int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                 int32_t dk, int32_t dv, kda_dtype dtype, uint32_t options,
                                 const void* d_o, const float* d_final_state,
                                 const float* checkpoints, float* grad_q, float* grad_k,
                                 float* grad_v, float* grad_log_alpha, float* grad_beta,
                                 float* grad_init_state, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  kda_status st = check_bwd_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (st != KDA_SUCCESS) return st;
  if (options & ~kAllOptions) return KDA_ERROR_NOT_SUPPORTED;
  const bool scalar = (options & KDA_OPT_SCALAR_GATE) != 0;
  if (cu_seqlens == nullptr && total_tokens % num_seqs != 0) return KDA_ERROR_INVALID_VALUE;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !grad_q || !grad_k ||
                           !grad_v || !grad_log_alpha || !grad_beta))
    return KDA_ERROR_INVALID_VALUE;
  if (!workspace) return KDA_ERROR_INVALID_VALUE;
  // the scalar gate and its gradient ([rows][H]) need only their element alignment
  const void* vec[] = {q, k, v, d_o, init_state, d_final_state, grad_q, grad_k, grad_v,
                       grad_init_state, scalar ? nullptr : log_alpha,
                       scalar ? nullptr : grad_log_alpha};
  for (const void* p : vec)
    if (p && !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
  if ((beta && !aligned_to(beta, esize(dtype))) || (grad_beta && !aligned_to(grad_beta, 4)) ||
      (cu_seqlens && !aligned_to(cu_seqlens, 4)) ||
      (scalar && log_alpha && !aligned_to(log_alpha, esize(dtype))) ||
      (scalar && grad_log_alpha && !aligned_to(grad_log_alpha, 4)))
    return KDA_ERROR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERROR_INVALID_VALUE;
  // every gradient buffer is written while the inputs are still read: none may overlap them
  const size_t T = (size_t)total_tokens, H = (size_t)num_heads, es = esize(dtype);
  const size_t sbytes = (size_t)num_seqs * H * dk * dv * sizeof(float);
  const void* in_p[] = {q, k, v, log_alpha, beta, d_o, init_state, d_final_state};
  const size_t gd = scalar ? 1 : (size_t)dk;  // gate values per token and head
  const size_t in_n[] = {T * H * dk * es, T * H * dk * es, T * H * dv * es, T * H * gd * es,
                         T * H * es, T * H * dv * es, sbytes, sbytes};
  const void* out_p[] = {grad_q, grad_k, grad_v, grad_log_alpha, grad_beta, grad_init_state};
  const size_t out_n[] = {T * H * dk * 4, T * H * dk * 4, T * H * dv * 4, T * H * gd * 4, T * H * 4,
                          sbytes};
  for (int o = 0; o < 6; ++o) {
    if (!out_p[o] || out_n[o] == 0) continue;
    for (int i = 0; i < 8; ++i)
      if (in_p[i] && in_n[i] && overlap(out_p[o], out_n[o], in_p[i], in_n[i])) return KDA_ERROR_INVALID_VALUE;
    for (int o2 = o + 1; o2 < 6; ++o2)
      if (out_p[o2] && out_n[o2] && overlap(out_p[o], out_n[o], out_p[o2], out_n[o2]))
        return KDA_ERROR_INVALID_VALUE;
  }
  // with checkpoints: segments that start where the forward kept a state
  int64_t step = 1;
  const size_t cb = ckpt_bytes(num_seqs, total_tokens, num_heads, dk, dv);
  if (cb == 0) checkpoints = nullptr;  // one forward segment: no boundary to start from
  if (checkpoints != nullptr) {
    if (!aligned16(checkpoints)) return KDA_ERROR_INVALID_VALUE;
    for (int o = 0; o < 6; ++o)
      if (out_p[o] && out_n[o] && overlap(out_p[o], out_n[o], checkpoints, cb))
        return KDA_ERROR_INVALID_VALUE;
    if (workspace_bytes && overlap(workspace, workspace_bytes, checkpoints, cb))
      return KDA_ERROR_INVALID_VALUE;
    step = ckpt_interval(num_seqs, total_tokens, num_heads);
    if (step < 1) return KDA_ERROR_INVALID_VALUE;
  }
  // the longest segments the caller's workspace holds (one segment when it holds them all)
  kda::BwdPlan p;
  if (!kda::make_bwd_plan(num_seqs, total_tokens, num_heads, dk, dv, options, 0, &p))
    return KDA_ERROR_INVALID_VALUE;
  if (!kda::fit_bwd_plan(num_seqs, total_tokens, num_heads, dk, dv, options, workspace_bytes, &p,
                         step))
    return KDA_ERROR_WORKSPACE_TOO_SMALL;
  kda::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_alpha;
  a.beta = beta;
  a.init_state = init_state;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.num_heads = num_heads;
  a.dk = dk;
  a.dv = dv;
  a.dtype_bf16 = dtype == KDA_DTYPE_BF16;
  a.dO = d_o;
  a.dfinal = d_final_state;
  a.grad_q = grad_q;
  a.grad_k = grad_k;
  a.grad_v = grad_v;
  a.grad_g = grad_log_alpha;
  a.grad_beta = grad_beta;
  a.grad_init = grad_init_state;
  a.options = options;
  a.workspace = workspace;
  a.stream = stream;
  a.ckpt = checkpoints;
  a.ckpt_interval = step;
  hipError_t e = kda::launch_chunk_bwd(a, p);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}

extern "C" kda_status kda_chunk_bwd_ex(const void* q, const void* k, const void* v,
                                       const void* log_alpha, const void* beta,
                                       const float* init_state, const int32_t* cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                       int32_t dk, int32_t dv, kda_dtype dtype, uint32_t options,
                                       const void* d_o, const float* d_final_state, float* grad_q,
                                       float* grad_k, float* grad_v, float* grad_log_alpha,
                                       float* grad_beta, float* grad_init_state, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, num_seqs, total_tokens,
                        num_heads, dk, dv, dtype, options, d_o, d_final_state, nullptr, grad_q,
                        grad_k, grad_v, grad_log_alpha, grad_beta, grad_init_state, workspace,
                        workspace_bytes, stream);
}

extern "C" kda_status kda_chunk_bwd_ckpt(const void* q, const void* k, const void* v,
                                         const void* log_alpha, const void* beta,
                                         const float* init_state, const int32_t* cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens,
                                         int32_t num_heads, int32_t dk, int32_t dv,
                                         kda_dtype dtype, uint32_t options, const void* d_o,
                                         const float* d_final_state, const float* checkpoints,
                                         float* grad_q, float* grad_k, float* grad_v,
                                         float* grad_log_alpha, float* grad_beta,
                                         float* grad_init_state, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (checkpoints == nullptr && ckpt_bytes(num_seqs, total_tokens, num_heads, dk, dv) > 0)
    return KDA_ERROR_INVALID_VALUE;
  return chunk_bwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, num_seqs, total_tokens,
                        num_heads, dk, dv, dtype, options, d_o, d_final_state, checkpoints,
                        grad_q, grad_k, grad_v, grad_log_alpha, grad_beta, grad_init_state,
                        workspace, workspace_bytes, stream);
}

extern "C" int64_t kda_chunk_fwd_ckpt_interval(int32_t num_seqs, int64_t total_tokens,
                                               int32_t num_heads) {
  if (num_seqs <= 0 || num_heads <= 0 || total_tokens < 0 || total_tokens > kMaxTokens) return 0;
  return ckpt_interval(num_seqs, total_tokens, num_heads);
}

extern "C" size_t kda_chunk_fwd_ckpt_bytes(int32_t num_seqs, int64_t total_tokens,
                                           int32_t num_heads, int32_t dk, int32_t dv) {
  if (num_seqs <= 0 || num_heads <= 0 || total_tokens < 0 || total_tokens > kMaxTokens ||
      !supported_chunk_dk(dk) || !(supported_chunk_dk(dv) || dv == 256))
    return 0;
  return ckpt_bytes(num_seqs, total_tokens, num_heads, dk, dv);
}

extern "C" kda_status kda_chunk_bwd(const void* q, const void* k, const void* v,
                                    const void* log_alpha, const void* beta,
                                    const float* init_state, const int32_t* cu_seqlens,
                                    int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype, const void* d_o,
                                    const float* d_final_state, float* grad_q, float* grad_k,
                                    float* grad_v, float* grad_log_alpha, float* grad_beta,
                                    float* grad_init_state, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return kda_chunk_bwd_ex(q, k, v, log_alpha, beta, init_state, cu_seqlens, num_seqs,
                          total_tokens, num_heads, dk, dv, dtype, 0u, d_o, d_final_state, grad_q,
                          grad_k, grad_v, grad_log_alpha, grad_beta, grad_init_state, workspace,
                          workspace_bytes, stream);
}

static kda_status check_scan_shape(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                   int32_t dk, int32_t dv, kda_dtype dtype, int32_t num_groups) {
  kda_status st = check_chunk_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (st != KDA_SUCCESS) return st;
  // the first pass needs V + K columns (<= 256) and the chunk path (K <= 128; fp32 at K <= 64)
  if (dk + dv > 256 || dk > 128 || wide_path(dk, dtype, 0u)) return KDA_ERROR_NOT_SUPPORTED;
  if (num_groups <= 0) return KDA_ERROR_INVALID_VALUE;
  return KDA_SUCCESS;
}

extern "C" size_t kda_chunk_fwd_scan_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                                    int32_t num_heads, int32_t dk, int32_t dv,
                                                    kda_dtype dtype, int32_t num_groups) {
  if (check_scan_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype, num_groups) != KDA_SUCCESS)
    return 0;
  kda::ScanPlan sp;
  if (!kda::make_scan_plan(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_DTYPE_BF16,
                           num_groups, &sp))
    return 0;
  return sp.total_bytes;
}

extern "C" kda_status kda_chunk_fwd_scan_ex(const void* q, const void* k, const void* v,
                                            const void* log_alpha, const void* beta,
                                            const float* init_state, const int32_t* cu_seqlens,
                                            int32_t num_seqs, int64_t total_tokens,
                                            int32_t num_heads, int32_t dk, int32_t dv,
                                            kda_dtype dtype, uint32_t options, int32_t num_groups,
                                            void* o, float* final_state, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  kda_status st = check_scan_shape(num_seqs, total_tokens, num_heads, dk, dv, dtype, num_groups);
  if (st != KDA_SUCCESS) return st;
  if (cu_seqlens == nullptr && total_tokens % num_seqs != 0) return KDA_ERROR_INVALID_VALUE;
  if (cu_seqlens && !aligned_to(cu_seqlens, 4)) return KDA_ERROR_INVALID_VALUE;
  if (options & ~kAllOptions) return KDA_ERROR_NOT_SUPPORTED;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERROR_INVALID_VALUE;
  if (!workspace) return KDA_ERROR_INVALID_VALUE;
  const bool scalar_gate = (options & KDA_OPT_SCALAR_GATE) != 0;
  const void* ptrs[] = {q, k, v, scalar_gate ? nullptr : log_alpha, init_state, o, final_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
  if ((beta && !aligned_to(beta, esize(dtype))) || (log_alpha && !aligned_to(log_alpha, esize(dtype))))
    return KDA_ERROR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERROR_INVALID_VALUE;
  const size_t sbytes = (size_t)num_seqs * num_heads * dk * dv * sizeof(float);
  if (init_state && final_state && init_state != final_state &&
      overlap(init_state, sbytes, final_state, sbytes))
    return KDA_ERROR_INVALID_VALUE;
  if (total_tokens > 0) {
    const int32_t gdim = scalar_gate ? 1 : dk;
    const size_t obytes = (size_t)total_tokens * num_heads * dv * esize(dtype);
    const size_t ibytes = (size_t)total_tokens * num_heads * dk * esize(dtype);
    const size_t gbytes = (size_t)total_tokens * num_heads * gdim * esize(dtype);
    if (overlap(o, obytes, q, ibytes) || overlap(o, obytes, k, ibytes) ||
        overlap(o, obytes, log_alpha, gbytes) || overlap(o, obytes, v, obytes))
      return KDA_ERROR_INVALID_VALUE;
  }
  kda::ScanPlan sp;
  if (!kda::make_scan_plan(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_DTYPE_BF16,
                           num_groups, &sp))
    return KDA_ERROR_INVALID_VALUE;
  if (workspace_bytes < sp.total_bytes) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  kda::ChunkArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_alpha;
  a.beta = beta;
  a.init_state = init_state;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.num_heads = num_heads;
  a.dk = dk;
  a.dv = dv;
  a.dtype_bf16 = dtype == KDA_DTYPE_BF16;
  a.options = options;
  a.o = o;
  a.final_state = final_state;
  a.workspace = workspace;
  a.stream = stream;
  hipError_t e = kda::launch_chunk_fwd_scan(a, num_groups, sp);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}

extern "C" kda_status kda_chunk_fwd_scan(const void* q, const void* k, const void* v,
                                         const void* log_alpha, const void* beta,
                                         const float* init_state, int32_t num_seqs,
                                         int64_t total_tokens, int32_t num_heads, int32_t dk,
                                         int32_t dv, kda_dtype dtype, uint32_t options,
                                         int32_t num_groups, void* o, float* final_state,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return kda_chunk_fwd_scan_ex(q, k, v, log_alpha, beta, init_state, nullptr, num_seqs,
                               total_tokens, num_heads, dk, dv, dtype, options, num_groups, o,
                               final_state, workspace, workspace_bytes, stream);
}

extern "C" kda_status kda_decode_step_ex(const void* q, const void* k, const void* v,
                                         const void* log_alpha, const void* beta, float* state,
                                         void* o, int32_t num_seqs, int32_t num_heads,
                                         int32_t dk, int32_t dv, kda_dtype dtype,
                                         uint32_t options, void* stream) {
  if (num_seqs <= 0 || num_heads <= 0) return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(dtype) || !supported_dim(dk) || !supported_dim(dv)) return KDA_ERROR_NOT_SUPPORTED;
  if (options & ~kAllOptions) return KDA_ERROR_NOT_SUPPORTED;
  const int32_t gdim = (options & KDA_OPT_SCALAR_GATE) ? 1 : dk;
  if (!q || !k || !v || !log_alpha || !beta || !state || !o) return KDA_ERROR_INVALID_VALUE;
  const bool scalar_gate = (options & KDA_OPT_SCALAR_GATE) != 0;
  const void* ptrs[] = {q, k, v, scalar_gate ? state : log_alpha, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned_to(beta, esize(dtype)) || !aligned_to(log_alpha, esize(dtype)))
    return KDA_ERROR_INVALID_VALUE;
  const size_t heads = (size_t)num_seqs * num_heads;
  const size_t obytes = heads * dv * esize(dtype);
  if (overlap(o, obytes, state, heads * dk * dv * sizeof(float)) ||
      overlap(o, obytes, q, heads * dk * esize(dtype)) || overlap(o, obytes, k, heads * dk * esize(dtype)) ||
      overlap(o, obytes, v, obytes) || overlap(o, obytes, log_alpha, heads * gdim * esize(dtype)))
    return KDA_ERROR_INVALID_VALUE;
  kda::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_alpha;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.dk = dk;
  a.dv = dv;
  a.dtype_bf16 = dtype == KDA_DTYPE_BF16;
  a.options = options;
  a.stream = stream;
  hipError_t e = kda::launch_decode(a);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}

extern "C" kda_status kda_decode_step(const void* q, const void* k, const void* v,
                                      const void* log_alpha, const void* beta, float* state,
                                      void* o, int32_t num_seqs, int32_t num_heads, int32_t dk,
                                      int32_t dv, kda_dtype dtype, void* stream) {
  return kda_decode_step_ex(q, k, v, log_alpha, beta, state, o, num_seqs, num_heads, dk, dv,
                            dtype, 0u, stream);
}
