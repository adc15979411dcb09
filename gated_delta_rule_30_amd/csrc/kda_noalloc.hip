// kda_chunk_fwd_noalloc: the chunkwise forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// It runs the same kernels as kda_chunk_fwd_ex, with the workspace taken from one file-scope
// device array instead of a caller buffer. The array's address is obtained once per device
// with hipGetSymbolAddress (with that device current) and cached; host code uses only that
// address, never the array's name, which in host code is not a device address.
//
// The array holds the chunk table and one record buffer, which this entry point caps so that
// everything fits: a call runs in more, shorter segments than kda_chunk_fwd_ex's. Every call on
// a device shares that device's array; calls that overlap in time on one device race (order
// them on one stream, or serialise them). Nothing in the array needs to start at zero: each call
// writes every part it reads.
#include <mutex>

#include "kda_paths.h"

namespace kda {

// Fixed size of the no-allocation scratch (bytes), held on every device the library runs on
// until the process ends.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)128 << 20;

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of this device's scratch array (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace kda

extern "C" kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const void* log_alpha, const void* beta,
                                            const float* init_state, const int32_t* cu_seqlens,
                                            int32_t num_seqs, int64_t total_tokens,
                                            int32_t num_heads, int32_t dk, int32_t dv,
                                            kda_dtype dtype, uint32_t options, void* o,
                                            float* final_state, void* stream) {
  kda::ChunkArgs a;
  kda_status st = kda::prepare_chunk_fwd(q, k, v, log_alpha, beta, init_state, cu_seqlens,
                                         num_seqs, total_tokens, num_heads, dk, dv, dtype, options,
                                         o, final_state, stream, &a);
  if (st != KDA_SUCCESS) return st;
  // the running state lives in the caller's final_state; the wide-key path's records grow
  // with the sequence length and are not served from the fixed scratch
  if (final_state == nullptr) return KDA_ERROR_INVALID_VALUE;
  if (kda::is_wide_path(dk, dtype, options)) return KDA_ERROR_NOT_SUPPORTED;
  // plan with the record buffer capped to what the scratch leaves after the tables; the
  // tables are largest with one chunk per segment, so that plan bounds them
  kda::ChunkPlan pl;
  const bool bf16 = dtype == KDA_DTYPE_BF16;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, bf16, &pl, 0, false))
    return KDA_ERROR_INVALID_VALUE;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, bf16, &pl,
                            (size_t)num_heads * pl.rec_bytes, false))
    return KDA_ERROR_INVALID_VALUE;
  const size_t tables = pl.off_rec;
  if (tables >= kda::NOALLOC_SCRATCH_BYTES) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  if (!kda::make_chunk_plan(num_seqs, total_tokens, num_heads, dk, dv, bf16, &pl,
                            kda::NOALLOC_SCRATCH_BYTES - tables, false))
    return KDA_ERROR_WORKSPACE_TOO_SMALL;
  if (pl.total_bytes > kda::NOALLOC_SCRATCH_BYTES) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (kda::scratch_address(&ws) != hipSuccess) return KDA_ERROR_LAUNCH;
  a.workspace = ws;
  const hipError_t e = kda::launch_chunk_fwd(a, pl);
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH;
}
