// Chunked forward at 256 key channels (and at 128 for fp32 inputs). The same chunk form as
// kda_chunk.hip ("A Technical Breakdown", section 4; "Kimi Linear" explainer, "WY
// Representation"):
//     Delta = U - W S,   O = Qe S + P Delta,   S' = diag(gamma) S + Kt^T Delta,
// with b = cumsum(log alpha) per key channel, Qe = q e^b, Kt = k e^{b_last - b}, gamma =
// e^{b_last}, A = strict_lower(diag(beta) (k k^T weighted by e^{b_i - b_j})), T = (I + A)^{-1},
// W = T diag(beta) (k e^b), U = T diag(beta) V and P = lower(q k^T weighted by e^{b_i - b_j}).
// kda_chunk.hip's prep kernel keeps K-wide operand tiles in LDS, which at K = 256 (or fp32 at
// K = 128) would not fit; here the per-chunk kernel works over the key channels in parts of 64
// (the sums over channels in A and P add up across the parts, and every other quantity is per
// channel),
// in fp32 on the shared fp32 machinery of the training backward:
//   wide_prep_kernel   per (chunk, head), 512 threads: P, W, Kt, Qe, U, gamma -> fp32 record
//   wide_state_kernel  per (sequence, head, 16 or 32 value columns), 256 threads: the chain
//                      over the sequence's chunks, S (256 x 16 or 32) in LDS, the record
//                      blocks staged through LDS one after another (W, then Qe, then Kt),
//                      matrix-core steps
// Every product that carries in-chunk decay is formed pairwise, e^{b_i - b_j} with j <= i.
#include "kda_fp32.h"

namespace kda {

using namespace fp32;

namespace {

constexpr int KQ = 64;  // key channels per part (the record kernel's LDS tiles)

// per-(chunk, head) fp32 record, row-major blocks
template <int KW, int V>
struct WRec {
  static constexpr int oP = 0;               // P (lower incl.)     [64][64]
  static constexpr int oW = oP + BC * BC;    // W                   [64][256]
  static constexpr int oKt = oW + BC * KW;   // Kt                  [64][256]
  static constexpr int oQe = oKt + BC * KW;  // Qe                  [64][256]
  static constexpr int oU = oQe + BC * KW;   // U                   [64][V]
  static constexpr int oGam = oU + BC * V;   // gamma               [256]
  static constexpr int floats = (oGam + KW + 63) / 64 * 64;
};

}  // namespace

template <int KW, int V, typename MT>
__global__ __launch_bounds__(NTP, 4) void wide_prep_kernel(
    const MT* __restrict__ q, const MT* __restrict__ k, const MT* __restrict__ v,
    const MT* __restrict__ g, const MT* __restrict__ beta, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, float* __restrict__ rec) {
  using R = WRec<KW, V>;
  constexpr int LK = KQ + 4;                 // rows of a channel quarter
  constexpr int VH = V > KQ ? KQ : V, LV = VH + 4;
  // 70 KB in all and at most 128 VGPRs (4 waves per SIMD), so that two workgroups share a CU
  __shared__ __align__(16) float sQ[BC * LK];  // q (quarter), then beta v (quarter)
  __shared__ __align__(16) float sK[BC * LK];  // k (quarter)
  __shared__ __align__(16) float sB[BC * LK];  // b log2 e (quarter), then beta k e^b (quarter)
  __shared__ __align__(16) float sA[BC * 68];  // A (strict lower), then T = (I + A)^{-1}
  float* sT = sA;
  __shared__ float sBeta[BC];
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  float* rc = rec + ((size_t)c * H + h) * R::floats;
  if (threadIdx.x < BC)
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
  // A and P, summed over the four quarters: rows pi and 63 - pi form a pair with 65 entries j <= i;
  // TPP threads share a pair, thread jq taking v = jq + TPP u (v <= pi: row pi, j = v; else
  // row 63 - pi, j = v - pi - 1), so every thread has the same work
  constexpr int TPP = NTP / (BC / 2), VPT = (BC + 1 + TPP - 1) / TPP;
  const int pi = threadIdx.x / TPP, jq = threadIdx.x % TPP, i2 = BC - 1 - pi;
  float a[VPT], p[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) a[u] = p[u] = 0.f;
  for (int hh = 0; hh < KW / KQ; ++hh) {
    const int c0 = hh * KQ;
    load_rows<KQ, LK, NTP, MT, KW>(sQ, q, ch.tok, ch.len, H, h, c0);
    load_rows<KQ, LK, NTP, MT, KW>(sK, k, ch.tok, ch.len, H, h, c0);
    load_rows<KQ, LK, NTP, MT, KW>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KQ, LK, NTP>(sB);
    lds_barrier();
    // Qe, Kt, gamma of the quarter (rows past len hold q = k = 0, and b stays at its last value)
    for (int e = threadIdx.x; e < BC * KQ; e += NTP) {
      const int r = e / KQ, cc = e % KQ;
      const float br = sB[r * LK + cc], bl = sB[(BC - 1) * LK + cc];
      rc[R::oQe + r * KW + c0 + cc] = sQ[r * LK + cc] * exp2_f(br);
      rc[R::oKt + r * KW + c0 + cc] = sK[r * LK + cc] * exp2_f(bl - br);
    }
    if (threadIdx.x < KQ) rc[R::oGam + c0 + threadIdx.x] = exp2_f(sB[(BC - 1) * LK + threadIdx.x]);
    for (int c4 = 0; c4 < KQ; c4 += 4) {
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(sQ + pi * LK + c4);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(sK + pi * LK + c4);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(sB + pi * LK + c4);
      const f32x4 q2 = *reinterpret_cast<const f32x4*>(sQ + i2 * LK + c4);
      const f32x4 k2 = *reinterpret_cast<const f32x4*>(sK + i2 * LK + c4);
      const f32x4 b2 = *reinterpret_cast<const f32x4*>(sB + i2 * LK + c4);
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int v = jq + TPP * u;
        if (v <= BC) {
          const bool lo = v <= pi;
          const int j = lo ? v : v - pi - 1;
          const f32x4 qi = lo ? q1 : q2, ki = lo ? k1 : k2, bi = lo ? b1 : b2;
          const f32x4 kj = *reinterpret_cast<const f32x4*>(sK + j * LK + c4);
          const f32x4 bj = *reinterpret_cast<const f32x4*>(sB + j * LK + c4);
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = kj[e] * exp2_f(bi[e] - bj[e]);
          a[u] += dot4(ki, w);
          p[u] += dot4(qi, w);
        }
      }
    }
    lds_barrier();  // the quarter's reads done before the next quarter overwrites it
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int v = jq + TPP * u;
    if (v <= BC) {
      const bool lo = v <= pi;
      const int i = lo ? pi : i2, j = lo ? v : v - pi - 1;
      sA[i * 68 + j] = j < i ? sBeta[i] * a[u] : 0.f;
      rc[R::oP + i * BC + j] = p[u];
    }
  }
  for (int e = threadIdx.x; e < BC * BC; e += NTP)  // P's upper triangle
    if (e % BC > e / BC) rc[R::oP + e] = 0.f;
  lds_barrier();
  // T = (I + A)^{-1} by forward substitution, one column per thread of wave 0; T overwrites A
  // after the wave's last read of it (a wave's LDS accesses take effect in program order)
  if (threadIdx.x < BC) {
    const int m = threadIdx.x;
    float x[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      // four partial sums: the row's dot product is not one chain of dependent FMAs
      float ps[4] = {r == m ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < r; ++j) ps[j & 3] -= sA[r * 68 + j] * x[j];
      x[r] = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
#pragma unroll
    for (int r = 0; r < BC; ++r) sT[r * 68 + m] = x[r];
  }
  lds_barrier();
  // W = T diag(beta) (k e^b), quarter by quarter
  for (int hh = 0; hh < KW / KQ; ++hh) {
    const int c0 = hh * KQ;
    load_rows<KQ, LK, NTP, MT, KW>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KQ, LK, NTP>(sB);
    lds_barrier();
    mul_rows_exp2<KQ, LK, NTP, MT, KW>(sB, k, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    for (int e = threadIdx.x; e < BC * KQ; e += NTP) sB[(e / KQ) * LK + e % KQ] *= sBeta[e / KQ];
    lds_barrier();
    mmf<KQ, BC, false, false, 68, LK, NTP>(sT, sB, [&](int r, int cc, float x) {
      rc[R::oW + r * KW + c0 + cc] = x;
    });
    lds_barrier();
  }
  // U = T diag(beta) V, VH columns at a time
  for (int c0 = 0; c0 < V; c0 += VH) {
    load_rows<VH, LV, NTP, MT, V>(sQ, v, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    for (int e = threadIdx.x; e < BC * VH; e += NTP) sQ[(e / VH) * LV + e % VH] *= sBeta[e / VH];
    lds_barrier();
    mmf<VH, BC, false, false, 68, LV, NTP>(sT, sQ, [&](int r, int cc, float x) {
      rc[R::oU + r * V + c0 + cc] = x;
    });
    lds_barrier();
  }
}

// The chain of one (sequence, head, CW value columns); blockIdx = slice * chains8 + chain, so
// the slices of a chain share one XCD's L2. Per chunk: W staged, Delta = U - W S (wave w:
// rows 16 w ..); Qe staged, O = Qe S + P Delta (wave w: rows 16 w ..); Kt staged,
// S' = diag(gamma) S + Kt^T Delta (wave w: 16-row tiles w, w + 4, ..), each staged A operand
// read once for the CW / 16 column blocks. The next block's loads are issued before the
// current block's products. CW = 32 at V = 256 keeps the chains to one wave of workgroups.
template <int KW, int V, int CW, typename MT>
__global__ __launch_bounds__(NT) void wide_state_kernel(
    const float* __restrict__ rec, const float* __restrict__ init, const int32_t* __restrict__ cu,
    int64_t T, const int32_t* __restrict__ seq_first, int N, int H, int chains8, MT* __restrict__ o,
    float* __restrict__ fin) {
  using R = WRec<KW, V>;
  static_assert(KW <= NT && KW % 64 == 0, "one thread per key channel for gamma");
  constexpr int NCB = CW / 16;           // 16-column blocks per workgroup
  constexpr int LS = CW == 16 ? 16 : CW + 16;  // S and Delta rows, read down their columns
  constexpr int LR = KW + 4;    // W and Qe: read along rows (A operand rows)
  constexpr int LC = KW + 16;   // Kt: read down columns
  constexpr int PB = BC * KW / 4 / NT;   // 16-byte pieces per thread of a 64 x 256 block
  constexpr int PP = BC * BC / 4 / NT;   // ... of P
  constexpr int TPW = KW / 16 / 4;       // S' row tiles per wave
  __shared__ __align__(16) float sS[KW * LS];
  __shared__ __align__(16) float sOp[BC * LC];  // W, then Qe, then Kt
  __shared__ __align__(16) float sP[BC * 68];
  __shared__ __align__(16) float sD[BC * LS];
  __shared__ float sG[KW];
  const int nh = blockIdx.x % chains8, s = blockIdx.x / chains8;
  if (nh >= N * H) return;
  const int n = nh / H, h = nh % H, c0 = CW * s;
  const int tid = threadIdx.x, w = tid >> 6, lm = tid & 15, lg = (tid >> 4) & 3;
  for (int e = tid; e < KW * CW; e += NT)
    sS[(e / CW) * LS + e % CW] = init ? init[((size_t)nh * KW + e / CW) * V + c0 + e % CW] : 0.f;
  const int first = seq_first[n], last = seq_first[n + 1];
  int64_t s0, s1;
  seq_range(cu, N, T, n, &s0, &s1);
  f32x4 rb[PB];
  auto fetch = [&](const float* src) {
#pragma unroll
    for (int u = 0; u < PB; ++u) rb[u] = reinterpret_cast<const f32x4*>(src)[tid + NT * u];
  };
  auto stage = [&](int ld) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = tid + NT * u;
      *reinterpret_cast<f32x4*>(sOp + (e / (KW / 4)) * ld + 4 * (e % (KW / 4))) = rb[u];
    }
  };
  // W, P, this slice of U and gamma of a chunk; a chunk's are loaded while the chunk before
  // forms S' (the last chunk loads its own again)
  f32x4 pp[PP], d[NCB];
  float rg;
  auto fetch_head = [&](const float* rc) {
    fetch(rc + R::oW);
#pragma unroll
    for (int u = 0; u < PP; ++u) pp[u] = reinterpret_cast<const f32x4*>(rc + R::oP)[tid + NT * u];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) d[cb][r] = rc[R::oU + (16 * w + 4 * lg + r) * V + c0 + 16 * cb + lm];
    rg = tid < KW ? rc[R::oGam + tid] : 0.f;
  };
  if (first < last) fetch_head(rec + ((size_t)first * H + h) * R::floats);
  for (int c = first; c < last; ++c) {
    const float* rc = rec + ((size_t)c * H + h) * R::floats;
    const int64_t tok = s0 + (int64_t)(c - first) * BC;
    const int len = (int)min((int64_t)BC, s1 - tok);
    lds_barrier();  // the previous chunk's reads of LDS are done
    stage(LR);
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int e = tid + NT * u;
      *reinterpret_cast<f32x4*>(sP + (e / (BC / 4)) * 68 + 4 * (e % (BC / 4))) = pp[u];
    }
    if (tid < KW) sG[tid] = rg;
    fetch(rc + R::oQe);  // in flight during Delta
    lds_barrier();
    // Delta rows 16 w .. : U - W S
#pragma unroll 4
    for (int mm = 0; mm < KW; mm += 4) {
      const float a = -sOp[(16 * w + lm) * LR + mm + lg];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) d[cb] = mfma4(a, sS[(mm + lg) * LS + 16 * cb + lm], d[cb]);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sD[(16 * w + 4 * lg + r) * LS + 16 * cb + lm] = d[cb][r];
    lds_barrier();  // Delta complete, W no longer read
    stage(LR);
    fetch(rc + R::oKt);  // in flight during O
    lds_barrier();
    // O rows 16 w .. : Qe S + P Delta (P_ij = 0 for j > i: steps up to row 16 w + 15)
    f32x4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int mm = 0; mm < KW; mm += 4) {
      const float a = sOp[(16 * w + lm) * LR + mm + lg];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma4(a, sS[(mm + lg) * LS + 16 * cb + lm], acc[cb]);
    }
    for (int j = 0; j < 16 * (w + 1); j += 4) {
      const float a = sP[(16 * w + lm) * 68 + j + lg];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma4(a, sD[(j + lg) * LS + 16 * cb + lm], acc[cb]);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * lg + r;
        if (row < len)
          o[((tok + row) * H + h) * (int64_t)V + c0 + 16 * cb + lm] = from_f32<MT>(acc[cb][r]);
      }
    lds_barrier();  // Qe no longer read
    stage(LC);
    fetch_head(rec + ((size_t)(c + 1 < last ? c + 1 : c) * H + h) * R::floats);
    lds_barrier();
    // S' tiles: diag(gamma) S + Kt^T Delta
    f32x4 sn[TPW][NCB];
#pragma unroll
    for (int qq = 0; qq < TPW; ++qq) {
      const int mt = w + 4 * qq;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * lg + r;
          sn[qq][cb][r] = sG[row] * sS[row * LS + 16 * cb + lm];
        }
#pragma unroll 4
      for (int r0 = 0; r0 < BC; r0 += 4) {
        const float a = sOp[(r0 + lg) * LC + 16 * mt + lm];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          sn[qq][cb] = mfma4(a, sD[(r0 + lg) * LS + 16 * cb + lm], sn[qq][cb]);
      }
    }
    lds_barrier();  // every read of S done
#pragma unroll
    for (int qq = 0; qq < TPW; ++qq) {
      const int mt = w + 4 * qq;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(16 * mt + 4 * lg + r) * LS + 16 * cb + lm] = sn[qq][cb][r];
    }
  }
  if (fin) {
    __syncthreads();
    for (int e = tid; e < KW * CW; e += NT)
      fin[((size_t)nh * KW + e / CW) * V + c0 + e % CW] = sS[(e / CW) * LS + e % CW];
  }
}

// ---------------------------------------------------------------- host
static size_t al256w(size_t x) { return (x + 255) / 256 * 256; }

bool make_wide_plan(int N, int64_t T, int H, int K, int V, WidePlan* p) {
  if (N <= 0 || H <= 0 || T < 0) return false;
  size_t rec_floats = 0;
#define KDA_WREC(KK, VV) \
  if (K == KK && V == VV) rec_floats = WRec<KK, VV>::floats;
  KDA_WREC(128, 32) KDA_WREC(128, 64) KDA_WREC(128, 128) KDA_WREC(128, 256)
  KDA_WREC(256, 32) KDA_WREC(256, 64) KDA_WREC(256, 128) KDA_WREC(256, 256)
#undef KDA_WREC
  if (rec_floats == 0) return false;
  int64_t ub = (T + (int64_t)N * (BC - 1)) / BC;
  if (ub > T) ub = T;
  p->ub = ub;
  size_t off = 0;
  p->off_seq = off;
  off += al256w((size_t)(N + 1) * 4);
  p->off_rows = off;
  off += al256w((size_t)ub * sizeof(ChunkRow));
  p->off_rec = off;
  off += al256w((size_t)ub * H * rec_floats * 4);
  p->total_bytes = off;
  return true;
}

template <int K, int V, typename MT>
static hipError_t launch_wide_t(const ChunkArgs& a, const WidePlan& p) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + p.off_seq);
  ChunkRow* rows = reinterpret_cast<ChunkRow*>(ws + p.off_rows);
  float* rec = reinterpret_cast<float*>(ws + p.off_rec);
  const int N = a.num_seqs, H = a.num_heads;
  hipError_t e = launch_chunk_rows(a.cu_seqlens, N, a.total_tokens, p.ub, seq_first, rows, st);
  if (e != hipSuccess) return e;
  if (p.ub > 0)
    hipLaunchKernelGGL((wide_prep_kernel<K, V, MT>), dim3((unsigned)p.ub, (unsigned)H), dim3(NTP), 0,
                       st, (const MT*)a.q, (const MT*)a.k, (const MT*)a.v, (const MT*)a.g,
                       (const MT*)a.beta, H, (const ChunkRow*)rows, (const int32_t*)(seq_first + N),
                       rec);
  const int chains8 = (N * H + 7) / 8 * 8;
  constexpr int CW = V == 256 ? 32 : 16;  // value columns per chain workgroup
  hipLaunchKernelGGL((wide_state_kernel<K, V, CW, MT>), dim3((unsigned)(chains8 * (V / CW))), dim3(NT),
                     0, st, (const float*)rec, a.init_state, a.cu_seqlens, a.total_tokens,
                     (const int32_t*)seq_first, N, H, chains8, (MT*)a.o, a.final_state);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd_wide(const ChunkArgs& a, const WidePlan& p) {
#define KDA_WIDE_CASE(KK, VV)                                                                  \
  if (a.dk == KK && a.dv == VV)                                                                \
    return a.dtype_bf16 ? launch_wide_t<KK, VV, bf16>(a, p) : launch_wide_t<KK, VV, float>(a, p);
  KDA_WIDE_CASE(256, 32) KDA_WIDE_CASE(256, 64) KDA_WIDE_CASE(256, 128) KDA_WIDE_CASE(256, 256)
#undef KDA_WIDE_CASE
  // K = 128 comes here for fp32 inputs only (bf16 takes the chunk path)
#define KDA_WIDE_CASE(VV) \
  if (a.dk == 128 && a.dv == VV && !a.dtype_bf16) return launch_wide_t<128, VV, float>(a, p);
  KDA_WIDE_CASE(32) KDA_WIDE_CASE(64) KDA_WIDE_CASE(128) KDA_WIDE_CASE(256)
#undef KDA_WIDE_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
