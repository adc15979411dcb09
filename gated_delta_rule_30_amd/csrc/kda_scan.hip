// Chunk-parallel scan over long sequences: the sequence splits into G groups of whole chunks,
// and the groups' state transitions compose, so the sequential part shrinks from the whole
// sequence to G small matrix products ("Kimi Linear" explainer, "DPLR Chunked Parallel": the
// chunk transitions are diagonal-plus-low-rank matrices whose products are formed in
// parallel and combined; "A Technical Breakdown", section 4, state passing between chunks).
//
// With the state S (K x V) of a group's start, the group's end state is M_g S + B_g, where
// M_g (K x K) is the product of the group's per-token transitions (I - beta k k^T) Diag(alpha)
// and B_g (K x V) is the end state from S = 0. Since the columns of S evolve independently,
// one chunked pass over the groups with the values [v | 0] and the initial state [0 | I]
// (K x (V + K) per group) yields [B_g | M_g] at every group's end. Then, per sequence,
//   S_in(0) = initial state,   S_in(g + 1) = M_g S_in(g) + B_g      (a few K x K x V products)
// and a second chunked pass runs all groups at once from S_in(g), writing the outputs and the
// groups' end states; the last group's end state is the sequence's final state.
//
// Both passes are the chunk path of kda_chunk.hip on the packed groups (a group is a sequence
// of the pass); this file holds the glue: the group boundaries, [v | 0] and [0 | I], the
// combine and the final copy. It pays a second pass and K more state columns in the first, so
// it helps when few (sequence, head) chains leave most CUs idle (e.g. one sequence, 4 heads).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// group g of sequence n: tokens [n L + min(g Lg, L), n L + min((g + 1) Lg, L))
__global__ void scan_cu_kernel(int32_t* cu, int N, int G, int64_t L, int64_t Lg) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i > (int64_t)N * G) return;
  const int64_t n = i / G, g = i % G;
  cu[i] = (int32_t)(n * L + min(g * Lg, L));
}

// v' = [v | 0]: rows of V + K values, 16-byte pieces
template <typename MT>
__global__ void scan_vaug_kernel(const MT* __restrict__ v, MT* __restrict__ vaug, int64_t rows,
                                 int V, int K) {
  const int64_t ppr = (int64_t)(V + K) * sizeof(MT) / 16, vp = (int64_t)V * sizeof(MT) / 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < rows * ppr;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ppr, c = i - r * ppr;
    v4u32 x = {0u, 0u, 0u, 0u};
    if (c < vp) x = reinterpret_cast<const v4u32*>(v + r * V)[c];
    reinterpret_cast<v4u32*>(vaug + r * (V + K))[c] = x;
  }
}

// init' = [0 | I]: [groups * H][K][V + K] fp32
__global__ void scan_init_kernel(float* __restrict__ init, int64_t heads, int K, int V) {
  const int W = V + K;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < heads * K * W;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(i % W);
    const int c = (int)((i / W) % K);
    init[i] = (j == V + c) ? 1.f : 0.f;
  }
}

// S_in of every group. One workgroup per (sequence, head, 16 value columns): the column block
// of S (K x 16) and, per group, M_g (read once, coalesced) sit in LDS; thread (r, half) owns
// row r and 8 of the 16 columns of S, and forms them as K outer-product steps
// acc += M_g[r][c] * S[c][cols] (one LDS read of M, two 16-byte reads of S, 8 FMAs per step),
// plus B_g. fin1 rows are V + K wide.
constexpr int SCAN_THREADS = 256;
__global__ __launch_bounds__(SCAN_THREADS) void scan_combine_kernel(
    const float* __restrict__ fin1, const float* __restrict__ init, float* __restrict__ sin,
    int G, int H, int K, int V) {
  __shared__ __align__(16) float sS[128 * 16];        // K <= 128
  __shared__ __align__(16) float sM[128 * (128 + 4)];  // M_g, rows padded by 4
  const int blocks = V / 16;
  const int cb = blockIdx.x % blocks;
  const int nh = blockIdx.x / blocks;
  const int n = nh / H, h = nh % H;
  const int W = V + K, c0 = 16 * cb, LM = K + 4;
  const int tid = threadIdx.x;
  const int r = tid >> 1, half = tid & 1;  // threads past 2K idle in the product
  for (int e = tid; e < K * 16; e += SCAN_THREADS) {
    const int rr = e >> 4, j = e & 15;
    sS[e] = init ? init[((size_t)nh * K + rr) * V + c0 + j] : 0.f;
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const size_t gi = ((size_t)n * G + g) * H + h;
    for (int e = tid; e < K * 16; e += SCAN_THREADS)
      sin[(gi * K + (e >> 4)) * V + c0 + (e & 15)] = sS[e];
    if (g == G - 1) break;
    const float* F = fin1 + gi * (size_t)K * W;
    // M_g: K * K / 4 16-byte pieces, at most 16 per thread, all loads issued before the stores
    {
      constexpr int MAXP = 128 * 128 / 4 / SCAN_THREADS;
      const int ppr = K / 4, np = K * ppr;  // pieces per row, pieces
      f32x4 mp[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int e = tid + SCAN_THREADS * i;
        if (e < np) mp[i] = *reinterpret_cast<const f32x4*>(F + (size_t)(e / ppr) * W + V + 4 * (e % ppr));
      }
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int e = tid + SCAN_THREADS * i;
        if (e < np) *reinterpret_cast<f32x4*>(sM + (e / ppr) * LM + 4 * (e % ppr)) = mp[i];
      }
    }
    __syncthreads();
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    if (r < K) {
      const float* brow = F + (size_t)r * W + c0 + 8 * half;
      a0 = *reinterpret_cast<const f32x4*>(brow);
      a1 = *reinterpret_cast<const f32x4*>(brow + 4);
      const float* mrow = sM + r * LM;
      for (int c = 0; c < K; ++c) {
        const float mv = mrow[c];
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sS + c * 16 + 8 * half);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(sS + c * 16 + 8 * half + 4);
        a0 += mv * s0;
        a1 += mv * s1;
      }
    }
    __syncthreads();
    if (r < K) {
      *reinterpret_cast<f32x4*>(sS + r * 16 + 8 * half) = a0;
      *reinterpret_cast<f32x4*>(sS + r * 16 + 8 * half + 4) = a1;
    }
    __syncthreads();
  }
}

// final_state[n, h] = the last group's end state
__global__ void scan_final_kernel(const float* __restrict__ sin, float* __restrict__ fin, int N,
                                  int G, int H, int KV) {
  const int64_t total = (int64_t)N * H * KV;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t nh = i / KV, e = i - nh * KV;
    const int64_t n = nh / H, h = nh - n * H;
    fin[i] = sin[((n * G + G - 1) * H + h) * KV + e];
  }
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

bool make_scan_plan(int N, int64_t T, int H, int K, int V, bool bf16, int G, ScanPlan* sp) {
  if (N <= 0 || G <= 0 || T < 0 || T % N != 0 || K != V || K > 128) return false;
  const int64_t N1 = (int64_t)N * G;
  if (N1 > (1 << 30)) return false;
  const size_t es = bf16 ? 2 : 4;
  const int64_t L = T / N;
  sp->L = L;
  sp->Lg = ((L + G - 1) / G + CHUNK - 1) / CHUNK * CHUNK;
  if (!make_chunk_plan((int)N1, T, H, K, V + K, bf16, &sp->p1)) return false;
  if (!make_chunk_plan((int)N1, T, H, K, V, bf16, &sp->p3)) return false;
  size_t off = 0;
  sp->off_ws = off;
  off += al256(sp->p1.total_bytes > sp->p3.total_bytes ? sp->p1.total_bytes : sp->p3.total_bytes);
  sp->off_vaug = off;
  off += al256((size_t)T * H * (V + K) * es);
  sp->off_oaug = off;
  off += al256((size_t)T * H * (V + K) * es);
  sp->off_init1 = off;
  off += al256((size_t)N1 * H * K * (V + K) * 4);
  sp->off_fin1 = off;
  off += al256((size_t)N1 * H * K * (V + K) * 4);
  sp->off_sin = off;
  off += al256((size_t)N1 * H * K * V * 4);
  sp->off_cu = off;
  off += al256((size_t)(N1 + 1) * 4);
  sp->total_bytes = off;
  return true;
}

hipError_t launch_chunk_fwd_scan(const ChunkArgs& a, int G, const ScanPlan& sp) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  const int N = a.num_seqs, H = a.num_heads, K = a.dk, V = a.dv;
  const int64_t T = a.total_tokens, N1 = (int64_t)N * G;
  int32_t* cu = reinterpret_cast<int32_t*>(ws + sp.off_cu);
  void* vaug = ws + sp.off_vaug;
  void* oaug = ws + sp.off_oaug;
  float* init1 = reinterpret_cast<float*>(ws + sp.off_init1);
  float* fin1 = reinterpret_cast<float*>(ws + sp.off_fin1);
  float* sin = reinterpret_cast<float*>(ws + sp.off_sin);
  const int64_t cu_n = N1 + 1;
  hipLaunchKernelGGL(scan_cu_kernel, dim3((unsigned)((cu_n + 255) / 256)), dim3(256), 0, st, cu, N,
                     G, sp.L, sp.Lg);
  const unsigned fill_blocks = 1024;
  if (T > 0) {
    if (a.dtype_bf16)
      hipLaunchKernelGGL(scan_vaug_kernel<bf16>, dim3(fill_blocks), dim3(256), 0, st,
                         (const bf16*)a.v, (bf16*)vaug, T * H, V, K);
    else
      hipLaunchKernelGGL(scan_vaug_kernel<float>, dim3(fill_blocks), dim3(256), 0, st,
                         (const float*)a.v, (float*)vaug, T * H, V, K);
  }
  hipLaunchKernelGGL(scan_init_kernel, dim3(fill_blocks), dim3(256), 0, st, init1, N1 * H, K, V);
  // pass 1: [B_g | M_g] of every group
  ChunkArgs a1 = a;
  a1.v = vaug;
  a1.init_state = init1;
  a1.cu_seqlens = cu;
  a1.num_seqs = (int)N1;
  a1.dv = V + K;
  a1.o = oaug;
  a1.final_state = fin1;
  a1.workspace = ws + sp.off_ws;
  hipError_t e = launch_chunk_fwd(a1, sp.p1);
  if (e != hipSuccess) return e;
  // the groups' initial states
  hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((int64_t)N * H * (V / 16))),
                     dim3(SCAN_THREADS), 0, st, fin1, a.init_state, sin, G, H, K, V);
  // pass 3: every group from its initial state; the end states overwrite them
  ChunkArgs a3 = a;
  a3.init_state = sin;
  a3.cu_seqlens = cu;
  a3.num_seqs = (int)N1;
  a3.final_state = sin;
  a3.workspace = ws + sp.off_ws;
  e = launch_chunk_fwd(a3, sp.p3);
  if (e != hipSuccess) return e;
  if (a.final_state)
    hipLaunchKernelGGL(scan_final_kernel, dim3(fill_blocks), dim3(256), 0, st, sin, a.final_state,
                       N, G, H, K * V);
  return hipGetLastError();
}

}  // namespace kda
