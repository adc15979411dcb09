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
// (K x (V + K) per group) yields [B_g | M_g] at every group's end. (The first pass takes W
// columns, V + K rounded up to a power of two, the width the chunk path runs; the columns past
// V + K hold zeros in the values and the initial state and are never read.) Then, per sequence,
//   S_in(0) = initial state,   S_in(g + 1) = M_g S_in(g) + B_g      (a few K x K x V products)
// and a second chunked pass runs all groups at once from S_in(g), writing the outputs and the
// groups' end states; the last group's end state is the sequence's final state.
//
// Both passes are the chunk path of kda_chunk.hip on the packed groups (a group is a sequence
// of the pass); the second reuses the (chunk, head) records the first built, so only the
// state recurrence runs twice. This file holds the glue: the group boundaries, [v | 0] and
// [0 | I], the combine and the final copy. It pays a second state sweep and K more state
// columns in the first, so it helps when few (sequence, head) chains leave most CUs idle
// (one long sequence with a few heads).
#include "kda_device.h"
#include "kda_paths.h"

namespace kda {

// group g of sequence n: tokens [s_n + min(g Lg_n, L_n), s_n + min((g + 1) Lg_n, L_n)), with
// s_n, L_n the sequence's start and length (cu_in, or n L and L for equal lengths) and Lg_n
// its length over G rounded up to whole chunks
__global__ void scan_cu_kernel(int32_t* cu, const int32_t* __restrict__ cu_in, int N, int G,
                               int64_t L) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i > (int64_t)N * G) return;
  int64_t n = i / G, g = i % G;
  if (n == N) {  // the end of the last sequence
    n = N - 1;
    g = G;
  }
  const int64_t s0 = cu_in ? cu_in[n] : n * L;
  const int64_t len = cu_in ? cu_in[n + 1] - s0 : L;
  const int64_t lg = ((len + G - 1) / G + CHUNK - 1) / CHUNK * CHUNK;
  cu[i] = (int32_t)(s0 + min(g * lg, len));
}

// v' = [v | 0]: rows of W values, 16-byte pieces
template <typename MT>
__global__ void scan_vaug_kernel(const MT* __restrict__ v, MT* __restrict__ vaug, int64_t rows,
                                 int V, int W) {
  const int64_t ppr = (int64_t)W * sizeof(MT) / 16, vp = (int64_t)V * sizeof(MT) / 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < rows * ppr;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ppr, c = i - r * ppr;
    v4u32 x = {0u, 0u, 0u, 0u};
    if (c < vp) x = reinterpret_cast<const v4u32*>(v + r * V)[c];
    reinterpret_cast<v4u32*>(vaug + r * W)[c] = x;
  }
}

// init' = [0 | I | 0]: [groups * H][K][W] fp32, the identity in columns V .. V + K - 1
__global__ void scan_init_kernel(float* __restrict__ init, int64_t heads, int K, int V, int W) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < heads * K * W;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(i % W);
    const int c = (int)((i / W) % K);
    init[i] = (j == V + c) ? 1.f : 0.f;
  }
}

// S_in of every group. One workgroup of 4K threads per (sequence, head, 4 value columns):
// thread (r, q) holds a quarter of row r of M_g in registers (columns 16 i + 4 q .. + 3, so the
// four threads of a row read 64 contiguous bytes per load) and forms that quarter's share of
// row r of M_g S_in(g) from the K x 4 column block of S_in(g) in LDS (broadcast reads, the
// four quarters in four bank groups); the shares meet through two quad permutes, and the sum
// plus row r of B_g is row r of S_in(g + 1). The half rows and B of the next two groups are in flight
// while the current product runs. fin1 rows are W wide: B_g, then M_g (then unused columns).
constexpr int SCAN_COLS = 4;

__device__ __forceinline__ float quad_xor(float x, int m) {
  // DPP quad_perm: lane i of each 4-lane group reads lane i ^ m (m = 1: [1,0,3,2], 2: [2,3,0,1])
  return m == 1 ? __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, true))
                : __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, true));
}

template <int K>
__global__ __launch_bounds__(4 * K) void scan_combine_kernel(
    const float* __restrict__ fin1, const float* __restrict__ init, float* __restrict__ sin,
    float* __restrict__ dummy, int G, int H, int V, int W) {
  constexpr int KQ = K / 4;  // this thread's share of a row
  __shared__ __align__(16) f32x4 sS[K];  // S_in(g)'s column block
  const int blocks = V / SCAN_COLS;
  const int cb = blockIdx.x % blocks;
  const int nh = blockIdx.x / blocks;
  const int n = nh / H, h = nh % H;
  const int c0 = SCAN_COLS * cb;
  const int tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;
  // three register sets in rotation: the current group's quarter row, the next group's (in
  // flight since the step before) and the one after (issued now)
  f32x4 m0[KQ / 4], m1[KQ / 4], m2[KQ / 4];
  f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0, b2 = b0;
  auto load = [&](int g, f32x4* m, f32x4& bv) {
    const float* F = fin1 + ((((size_t)n * G + g) * H + h) * K + r) * (size_t)W;
#pragma unroll
    for (int i = 0; i < KQ / 4; ++i)
      m[i] = *reinterpret_cast<const f32x4*>(F + V + 16 * i + 4 * q);
    bv = *reinterpret_cast<const f32x4*>(F + c0);
  };
  // The loop body has no branch: the steps run in threes, to a multiple of 3; a group past
  // the last is read as the last (in bounds), and a step past the last group stores its unused
  // values to a dummy slot. The four threads of a row hold the same values; each stores one
  // column. (A branch between a load and its use lets the compiler sink the load to the use,
  // and one around the loads makes it wait for every load in flight at the join.)
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (init) s = *reinterpret_cast<const f32x4*>(init + ((size_t)nh * K + r) * V + c0);
  sS[r] = s;
  load(0, m0, b0);
  load(min(1, G - 1), m1, b1);
  __syncthreads();
  float* srow = sin + ((size_t)n * G * H + h) * K * V + (size_t)r * V + c0 + q;
  const size_t gstride = (size_t)H * K * V;
  // step g: store S_in(g), start loading group g + 2, form S_in(g + 1) = M_g S_in(g) + B_g
  auto step = [&](int g, const f32x4* cur, const f32x4& bcur, f32x4* nxt, f32x4& bnxt) {
    const float mine = q == 0 ? s[0] : q == 1 ? s[1] : q == 2 ? s[2] : s[3];
    *(g < G ? srow + (size_t)g * gstride : dummy) = mine;
    load(min(g + 2, G - 1), nxt, bnxt);
    // the quarter's rows of S_in(g) in batches of up to 16 LDS reads, each batch issued whole
    // before its FMAs (the scheduler would otherwise wait on every read or two)
    constexpr int BI = KQ / 4 < 4 ? KQ / 4 : 4;  // 4-row pieces per batch
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < KQ / 4; b += BI) {
      f32x4 sv[4 * BI];
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[4 * i + j] = sS[16 * (b + i) + 4 * q + j];
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += cur[b + i][j] * sv[4 * i + j];
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * BI, 0);   // the batch's LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 16 * BI, 0);  // then its FMAs
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += quad_xor(acc[j], 1);
      acc[j] += quad_xor(acc[j], 2);
    }
    s = acc + bcur;
    __syncthreads();  // every read of sS done
    sS[r] = s;
    __syncthreads();
  };
  for (int g = 0; g < G; g += 3) {
    step(g, m0, b0, m2, b2);
    step(g + 1, m1, b1, m0, b0);
    step(g + 2, m2, b2, m1, b1);
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
  if (N <= 0 || G <= 0 || T < 0 || K > 128 || V + K > 256) return false;
  const int64_t N1 = (int64_t)N * G;
  if (N1 > (1 << 30)) return false;
  const size_t es = bf16 ? 2 : 4;
  // the sizes hold for any lengths: N G groups over T tokens (L: the equal-length split)
  const int64_t L = T / N;
  sp->L = L;
  sp->Lg = ((L + G - 1) / G + CHUNK - 1) / CHUNK * CHUNK;
  sp->W = 32;
  while (sp->W < V + K) sp->W *= 2;
  if (!make_chunk_plan((int)N1, T, H, K, sp->W, bf16, &sp->p1)) return false;
  if (!make_chunk_plan((int)N1, T, H, K, V, bf16, &sp->p3)) return false;
  size_t off = 0;
  // the first pass keeps every segment's records (one slot each, from its record buffer on)
  // and the second pass reads them: same chunks, and its value columns lead the first's
  sp->off_ws = off;
  sp->rec_region_bytes = (size_t)sp->p1.num_segs * sp->p1.rec_buf_bytes;
  const size_t ws1 = sp->p1.off_rec + sp->rec_region_bytes;
  off += al256(ws1 > sp->p3.total_bytes ? ws1 : sp->p3.total_bytes);
  sp->off_vaug = off;
  off += al256((size_t)T * H * sp->W * es);
  sp->off_oaug = off;
  off += al256((size_t)T * H * sp->W * es);
  sp->off_init1 = off;
  off += al256((size_t)N1 * H * K * sp->W * 4);
  sp->off_fin1 = off;
  off += al256((size_t)N1 * H * K * sp->W * 4);
  sp->off_sin = off;
  off += al256((size_t)N1 * H * K * V * 4);
  sp->off_cu = off;
  off += al256((size_t)(N1 + 1) * 4);
  sp->off_dummy = off;
  off += 256;
  sp->total_bytes = off;
  return true;
}

hipError_t launch_chunk_fwd_scan(const ChunkArgs& a, int G, const ScanPlan& sp) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  const int N = a.num_seqs, H = a.num_heads, K = a.dk, V = a.dv, W = sp.W;
  const int64_t T = a.total_tokens, N1 = (int64_t)N * G;
  int32_t* cu = reinterpret_cast<int32_t*>(ws + sp.off_cu);
  void* vaug = ws + sp.off_vaug;
  void* oaug = ws + sp.off_oaug;
  float* init1 = reinterpret_cast<float*>(ws + sp.off_init1);
  float* fin1 = reinterpret_cast<float*>(ws + sp.off_fin1);
  float* sin = reinterpret_cast<float*>(ws + sp.off_sin);
  float* dummy = reinterpret_cast<float*>(ws + sp.off_dummy);
  const int64_t cu_n = N1 + 1;
  hipLaunchKernelGGL(scan_cu_kernel, dim3((unsigned)((cu_n + 255) / 256)), dim3(256), 0, st, cu,
                     a.cu_seqlens, N, G, sp.L);
  const unsigned fill_blocks = 1024;
  if (T > 0) {
    if (a.dtype_bf16)
      hipLaunchKernelGGL(scan_vaug_kernel<bf16>, dim3(fill_blocks), dim3(256), 0, st,
                         (const bf16*)a.v, (bf16*)vaug, T * H, V, W);
    else
      hipLaunchKernelGGL(scan_vaug_kernel<float>, dim3(fill_blocks), dim3(256), 0, st,
                         (const float*)a.v, (float*)vaug, T * H, V, W);
  }
  hipLaunchKernelGGL(scan_init_kernel, dim3(fill_blocks), dim3(256), 0, st, init1, N1 * H, K, V, W);
  // pass 1: [B_g | M_g] of every group
  ChunkArgs a1 = a;
  a1.v = vaug;
  a1.init_state = init1;
  a1.cu_seqlens = cu;
  a1.num_seqs = (int)N1;
  a1.dv = W;
  a1.o = oaug;
  a1.final_state = fin1;
  a1.workspace = ws + sp.off_ws;
  const RecordRegion rr1{ws + sp.off_ws + sp.p1.off_rec, sp.p1.rec_bytes, true};
  hipError_t e = launch_chunk_fwd(a1, sp.p1, &rr1);
  if (e != hipSuccess) return e;
  // the groups' initial states
  const dim3 cgrid((unsigned)((int64_t)N * H * (V / SCAN_COLS)));
  if (K == 32)
    hipLaunchKernelGGL(scan_combine_kernel<32>, cgrid, dim3(4 * 32), 0, st, fin1, a.init_state, sin, dummy, G, H, V, W);
  else if (K == 64)
    hipLaunchKernelGGL(scan_combine_kernel<64>, cgrid, dim3(4 * 64), 0, st, fin1, a.init_state, sin, dummy, G, H, V, W);
  else
    hipLaunchKernelGGL(scan_combine_kernel<128>, cgrid, dim3(4 * 128), 0, st, fin1, a.init_state, sin, dummy, G, H, V, W);
  // pass 3: every group from its initial state; the end states overwrite them
  ChunkArgs a3 = a;
  a3.init_state = sin;
  a3.cu_seqlens = cu;
  a3.num_seqs = (int)N1;
  a3.final_state = sin;
  a3.workspace = ws + sp.off_ws;
  const RecordRegion rr3{rr1.base, sp.p1.rec_bytes, false};
  e = launch_chunk_fwd(a3, sp.p3, &rr3);
  if (e != hipSuccess) return e;
  if (a.final_state)
    hipLaunchKernelGGL(scan_final_kernel, dim3(fill_blocks), dim3(256), 0, st, sin, a.final_state,
                       N, G, H, K * V);
  return hipGetLastError();
}

}  // namespace kda
