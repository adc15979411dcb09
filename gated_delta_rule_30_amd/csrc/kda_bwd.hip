// Training backward of the chunked KDA forward: the gradients of
//     L = sum(dO * o) + sum(dS_final * S_final)
// with respect to q, k, v, log alpha, beta and the initial state, by reverse mode through the
// chunk form ("A Technical Breakdown", section 4: state passing with the in-chunk cumulative
// decay and the U / W matrices; "Kimi Linear" explainer, "WY Representation": the chunk's
// rank-1 updates through a unit lower triangular inverse). With, per chunk of C = 64 tokens,
// b = cumsum(log alpha) (per key channel), Qe = q e^b, Ke = k e^b, Kt = k e^{b_last - b},
// gamma = e^{b_last}, A = strict_lower(diag(beta) (k k^T weighted by e^{b_i - b_j})),
// T = (I + A)^{-1}, W = T diag(beta) Ke, U = T diag(beta) V, P = lower((q k^T weighted)),
// the forward is  Delta = U - W S,  O = Qe S + P Delta,  S' = diag(gamma) S + Kt^T Delta,  and the
// adjoints, with X = dL/dS' carried backwards over the chunks, are
//     dDelta = P^T dO + Kt X,          dS = Qe^T dO + diag(gamma) X - W^T dDelta,
//     dP = lower(dO Delta^T),          dW = -dDelta S^T,   dv = diag(beta) T^T dDelta,
//     dT = dDelta (beta V)^T + dW (beta Ke)^T,              dA = strict_lower(-T^T dT T^T),
// and the per-token gradients of q, k, beta and log alpha follow from dP, dA, T^T dW and
// Delta X^T. Every product that carries in-chunk decay is formed pairwise as e^{b_i - b_j}
// with j <= i (at most 1), so nothing overflows for any decay.
//
// Everything runs in fp32 (the chunk's inputs, bf16 or fp32, are exact in fp32). Kernels:
//   bwd_seq_kernel, bwd_chunk_kernel   the chunk table (sequence boundaries from cu_seqlens)
//   bwd_prep_kernel                    per (chunk, head): T, P, W, Kt, Qe, U, gamma -> record
//   bwd_fstate_kernel                  per (sequence, head, 16 value columns), forward in
//                                      time: S at every chunk start and Delta
//   bwd_rstate_kernel                  the same chains backwards: X at every chunk end, dDelta,
//                                      and the initial state's gradient
//   bwd_ga_kernel, bwd_gb_kernel, bwd_gc_kernel
//                                      per (chunk, head): the products with S and X, then the
//                                      T-side adjoints, then the decay-weighted pairwise sums
//                                      and the per-token gradients
#include "kda_fp32.h"

namespace kda {

using namespace fp32;

namespace {

// per-(chunk, head) fp32 record of the backward, row-major blocks
template <int K, int V>
struct BRec {
  static constexpr int oT = 0;                 // T = (I + A)^{-1}        [64][64]
  static constexpr int oP = oT + BC * BC;      // P (lower incl.)        [64][64]
  static constexpr int oW = oP + BC * BC;      // W                       [64][K]
  static constexpr int oKt = oW + BC * K;      // Kt = k e^{b_last - b}   [64][K]
  static constexpr int oQe = oKt + BC * K;     // Qe = q e^b              [64][K]
  static constexpr int oU = oQe + BC * K;      // U                       [64][V]
  static constexpr int oGam = oU + BC * V;     // gamma = e^{b_last}      [K]
  static constexpr int floats = (oGam + K + 63) / 64 * 64;
};

// per-(chunk, head) fp32 scratch between the three gradient kernels
template <int K>
struct GScr {
  // [i][j] = dP_ij for j <= i (written by the S/X product kernel) and [j][i] = dA_ij for
  // j < i (dA's strict lower triangle, transposed, written by the T-side kernel)
  static constexpr int oDPA = 0;               // dP and dA^T            [64][64]
  static constexpr int oR1 = oDPA + BC * BC;   // dO S^T                 [64][K]
  static constexpr int oDW = oR1 + BC * K;     // dW = -dDelta S^T       [64][K]
  static constexpr int oDKt = oDW + BC * K;    // Delta X^T              [64][K]
  static constexpr int oTDW = oDKt + BC * K;   // T^T dW                 [64][K]
  static constexpr int oDG = oTDW + BC * K;    // rowsum(S * X)          [K]
  static constexpr int floats = (oDG + K + 63) / 64 * 64;
};

}  // namespace

// seq_first[n] = the first chunk of sequence n, seq_first[N] = the number of chunks (one block)
__global__ __launch_bounds__(NT) void bwd_seq_kernel(const int32_t* __restrict__ cu, int N,
                                                     int64_t T, int32_t* __restrict__ seq_first) {
  __shared__ int32_t part[NT];
  int32_t carry = 0;
  for (int base = 0; base < N; base += NT) {
    const int n = base + threadIdx.x;
    int32_t cnt = 0;
    if (n < N) {
      const int64_t a = cu ? cu[n] : (T / N) * n, b = cu ? cu[n + 1] : (T / N) * (n + 1);
      cnt = (int32_t)((b - a + BC - 1) / BC);
    }
    part[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {  // inclusive scan
      const int32_t x = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    if (n < N) seq_first[n] = carry + part[threadIdx.x] - cnt;
    carry += part[NT - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq_first[N] = carry;
}

// chunk c: its sequence (the last n with seq_first[n] <= c), first token and length
__global__ __launch_bounds__(NT) void bwd_chunk_kernel(const int32_t* __restrict__ cu, int N,
                                                       int64_t T, const int32_t* __restrict__ seq_first,
                                                       int64_t ub, ChunkRow* __restrict__ chunks) {
  const int64_t c = blockIdx.x * (int64_t)NT + threadIdx.x;
  if (c >= ub || c >= seq_first[N]) return;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (seq_first[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int64_t s1 = cu ? cu[lo + 1] : (T / N) * (lo + 1);
  const int64_t s0 = cu ? cu[lo] : (T / N) * lo;
  const int64_t tok = s0 + (c - seq_first[lo]) * BC;
  chunks[c] = ChunkRow{lo, (int32_t)tok, (int32_t)min((int64_t)BC, s1 - tok), 0};
}

// ---------------------------------------------------------------- per-chunk record
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTP, 4) void bwd_prep_kernel(
    const MT* __restrict__ q, const MT* __restrict__ k, const MT* __restrict__ v,
    const MT* __restrict__ g, const MT* __restrict__ beta, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, float* __restrict__ rec) {
  using R = BRec<K, V>;
  // The key channels are taken in parts of KC and the value columns in parts of VC (at most
  // 64 each): the sums over channels in A and P add up across the parts, and every other
  // quantity is per channel or per column. With T written over A the LDS stays at 70 KB and
  // the kernel at 128 VGPRs, so two workgroups (16 waves) share a CU.
  constexpr int KC = K > 64 ? 64 : K, VC = V > 64 ? 64 : V;
  constexpr int LK = KC + 4, LV = VC + 4, LQ = LK > LV ? LK : LV;
  __shared__ __align__(16) float sQ[BC * LQ];  // q (part), then beta v (part)
  __shared__ __align__(16) float sK[BC * LK];  // k (part)
  __shared__ __align__(16) float sB[BC * LK];  // b log2 e (part), then beta k e^b (part)
  __shared__ __align__(16) float sA[BC * 68];  // A (strict lower), then T = (I + A)^{-1}
  __shared__ float sBeta[BC];
  float* sT = sA;
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  float* rc = rec + ((size_t)c * H + h) * R::floats;
  if (threadIdx.x < BC)
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
  // A_ij = beta_i sum_c k_ic k_jc e^{b_ic - b_jc} (j < i) and P_ij = sum_c q_ic k_jc e^{..} (j <= i).
  // Rows pi and 63 - pi form a pair with 65 entries j <= i between them; TPP threads share a
  // pair, thread jq taking the entries v = jq + TPP u (v <= pi: row pi, j = v; else row
  // 63 - pi, j = v - pi - 1), so every thread has the same work and no entry is masked off.
  constexpr int TPP = NTP / (BC / 2), VPT = (BC + 1 + TPP - 1) / TPP;
  const int pi = threadIdx.x / TPP, jq = threadIdx.x % TPP, i2 = BC - 1 - pi;
  float a[VPT], p[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) a[u] = p[u] = 0.f;
  for (int c0 = 0; c0 < K; c0 += KC) {
    load_rows<KC, LQ, NTP, MT, K>(sQ, q, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTP, MT, K>(sK, k, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTP, MT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LK, NTP>(sB);
    lds_barrier();
    // Qe, Kt, gamma of the part (rows past len hold q = k = 0, and b stays at its last value)
    for (int e = threadIdx.x; e < BC * KC; e += NTP) {
      const int r = e / KC, cc = e % KC;
      const float br = sB[r * LK + cc], bl = sB[(BC - 1) * LK + cc];
      rc[R::oQe + r * K + c0 + cc] = sQ[r * LQ + cc] * exp2_f(br);
      rc[R::oKt + r * K + c0 + cc] = sK[r * LK + cc] * exp2_f(bl - br);
    }
    if (threadIdx.x < KC) rc[R::oGam + c0 + threadIdx.x] = exp2_f(sB[(BC - 1) * LK + threadIdx.x]);
    for (int c4 = 0; c4 < KC; c4 += 4) {
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(sQ + pi * LQ + c4);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(sK + pi * LK + c4);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(sB + pi * LK + c4);
      const f32x4 q2 = *reinterpret_cast<const f32x4*>(sQ + i2 * LQ + c4);
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
    lds_barrier();  // the part's reads done before the next part overwrites it
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
    for (int i = 0; i < BC; ++i) {
      // four partial sums: the row's dot product is not one chain of dependent FMAs
      float ps[4] = {i == m ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < i; ++j) ps[j & 3] -= sA[i * 68 + j] * x[j];
      x[i] = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      sT[i * 68 + m] = x[i];
      rc[R::oT + i * BC + m] = x[i];
    }
  }
  lds_barrier();
  // W = T diag(beta) (k e^b), part by part
  for (int c0 = 0; c0 < K; c0 += KC) {
    load_rows<KC, LK, NTP, MT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LK, NTP>(sB);
    lds_barrier();
    mul_rows_exp2<KC, LK, NTP, MT, K>(sB, k, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    for (int e = threadIdx.x; e < BC * KC; e += NTP) sB[(e / KC) * LK + e % KC] *= sBeta[e / KC];
    lds_barrier();
    mmf<KC, BC, false, false, 68, LK, NTP>(sT, sB, [&](int r, int cc, float x) {
      rc[R::oW + r * K + c0 + cc] = x;
    });
    lds_barrier();
  }
  // U = T diag(beta) V, part by part
  for (int c0 = 0; c0 < V; c0 += VC) {
    load_rows<VC, LV, NTP, MT, V>(sQ, v, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    for (int e = threadIdx.x; e < BC * VC; e += NTP) sQ[(e / VC) * LV + e % VC] *= sBeta[e / VC];
    lds_barrier();
    mmf<VC, BC, false, false, 68, LV, NTP>(sT, sQ, [&](int r, int cc, float x) {
      rc[R::oU + r * V + c0 + cc] = x;
    });
    lds_barrier();
  }
}

// ---------------------------------------------------------------- the chains
constexpr int NTR = 512;  // threads of a chain workgroup: 8 waves
// One workgroup per (sequence, head, 16 value columns); the slices of one chain share
// blockIdx % 8 (one XCD's L2) with blockIdx = slice * chains8 + chain. A chunk's record
// blocks are loaded whole into registers (16-byte pieces, all in flight) while the chunk
// before is computed, then stored to LDS; the chunk's products read LDS only. The loop body
// has no branch around those loads (the next chunk's index is clamped to the last), so the
// compiler neither sinks them to their use nor waits for them early, and its barriers order
// LDS only (a full __syncthreads would also wait for the loads in flight).


// Forward in time: S_c (chunk start) and Delta = U - W S per chunk, S' = diag(gamma) S + Kt^T
// Delta. NTR threads: waves 0-3 form the four 16-row tiles of Delta, wave w the 16-row tiles
// w, w + 8, .. of S', with matrix-core steps over LDS operands; two register sets hold the
// records of the next two chunks.
template <int K, int V>
__global__ __launch_bounds__(NTR) void bwd_fstate_kernel(
    const float* __restrict__ rec, const float* __restrict__ init, const int32_t* __restrict__ seq_first,
    int N, int H, int chains8, float* __restrict__ ckS, float* __restrict__ Dl) {
  using R = BRec<K, V>;
  // LDS row strides: a block read as the A operand along its rows (lane m takes row m, the
  // four lane groups consecutive columns) is padded by 4 floats, one read along its columns
  // (lane group g takes row g) by 16, so a wave's 64 reads fall in 64 different banks
  constexpr int LW = K + 4, LKT = K + 16;
  constexpr int PB = BC * K / 4 / NTR;  // 16-byte pieces per thread of a 64 x K block
  constexpr int WV = NTR / 64;
  constexpr int TPW = (K / 16 + WV - 1) / WV;  // S' tiles per wave
  __shared__ __align__(16) float sS[K * 16];
  __shared__ __align__(16) float sD[BC * 16];
  __shared__ __align__(16) float sW[BC * LW];
  __shared__ __align__(16) float sKt[BC * LKT];
  __shared__ float sG[K];
  const int nh = blockIdx.x % chains8, s = blockIdx.x / chains8;
  if (nh >= N * H) return;
  const int n = nh / H, h = nh % H, c0 = 16 * s;
  const int tid = threadIdx.x, w = tid >> 6, lm = tid & 15, lg = (tid >> 4) & 3;
  for (int e = tid; e < K * 16; e += NTR)
    sS[e] = init ? init[((size_t)nh * K + e / 16) * V + c0 + e % 16] : 0.f;
  const int first = seq_first[n], last = seq_first[n + 1];
  if (first == last) return;
  struct Regs {
    f32x4 w[PB], k[PB];
    float u[4], g;
  };
  Regs ra, rb;
  auto fetch = [&](Regs& x, int c) {
    const float* rc = rec + ((size_t)c * H + h) * R::floats;
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      x.w[u] = reinterpret_cast<const f32x4*>(rc + R::oW)[tid + NTR * u];
      x.k[u] = reinterpret_cast<const f32x4*>(rc + R::oKt)[tid + NTR * u];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) x.u[r] = rc[R::oU + (16 * (w & 3) + 4 * lg + r) * V + c0 + lm];
    x.g = rc[R::oGam + tid % K];
  };
  // one chunk: stage its registers, start loading chunk c + 2 into them, then its products
  auto step = [&](Regs& x, int c) {
    lds_barrier();  // the previous chunk's reads of LDS are done
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = tid + NTR * u;
      *reinterpret_cast<f32x4*>(sW + (e / (K / 4)) * LW + 4 * (e % (K / 4))) = x.w[u];
      *reinterpret_cast<f32x4*>(sKt + (e / (K / 4)) * LKT + 4 * (e % (K / 4))) = x.k[u];
    }
    if (tid < K) sG[tid] = x.g;
    f32x4 d = {x.u[0], x.u[1], x.u[2], x.u[3]};
    fetch(x, min(c + 2, last - 1));
    lds_barrier();
    for (int e = tid; e < K * 16; e += NTR)
      ckS[(((size_t)c * H + h) * K + e / 16) * V + c0 + e % 16] = sS[e];
    // Delta rows 16 w .. (waves 0-3): U - W S (two chains of dependent steps)
    if (w < 4) {
      f32x4 d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int mm = 0; mm < K; mm += 8) {
        d = mfma4(-sW[(16 * w + lm) * LW + mm + lg], sS[(mm + lg) * 16 + lm], d);
        d1 = mfma4(-sW[(16 * w + lm) * LW + mm + 4 + lg], sS[(mm + 4 + lg) * 16 + lm], d1);
      }
      d += d1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * lg + r;
        sD[row * 16 + lm] = d[r];
        Dl[(((size_t)c * H + h) * BC + row) * V + c0 + lm] = d[r];
      }
    }
    lds_barrier();
    // S' tiles: diag(gamma) S + Kt^T Delta
    f32x4 acc[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int mt = w + WV * q;
      if (mt < K / 16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * lg + r;
          acc[q][r] = sG[row] * sS[row * 16 + lm];
        }
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int r0 = 0; r0 < BC; r0 += 8) {
          acc[q] = mfma4(sKt[(r0 + lg) * LKT + 16 * mt + lm], sD[(r0 + lg) * 16 + lm], acc[q]);
          a1 = mfma4(sKt[(r0 + 4 + lg) * LKT + 16 * mt + lm], sD[(r0 + 4 + lg) * 16 + lm], a1);
        }
        acc[q] += a1;
      }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int mt = w + WV * q;
      if (mt < K / 16)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(16 * mt + 4 * lg + r) * 16 + lm] = acc[q][r];
    }
  };
  fetch(ra, first);
  fetch(rb, min(first + 1, last - 1));
  for (int c = first; c < last; c += 2) {
    step(ra, c);
    if (c + 1 >= last) break;
    step(rb, c + 1);
  }
}

// Backwards in time: X_c (the gradient at the chunk's end), dDelta = P^T dO + Kt X per chunk,
// X_prev = diag(gamma) X + Qe^T dO - W^T dDelta; at the end the initial state's gradient.
// NTR threads: waves 0-3 form the four 16-row tiles of dDelta, and wave w the 16-row tiles
// w, w + 8, .. of X_prev. Two register sets hold the records of the next two chunks, so each
// chunk's loads have two chunks of compute to arrive in.
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTR) void bwd_rstate_kernel(
    const float* __restrict__ rec, const MT* __restrict__ dO, const float* __restrict__ dfin,
    const int32_t* __restrict__ cu, int64_t T, const int32_t* __restrict__ seq_first, int N, int H,
    int chains8, float* __restrict__ ckX, float* __restrict__ dDl, float* __restrict__ dinit) {
  using R = BRec<K, V>;
  // LDS row strides as in the forward chain: Kt is read along its rows (+4), P, Qe and W
  // along their columns (+16)
  constexpr int LKt = K + 4, LC = K + 16, LP = BC + 16;
  constexpr int PB = BC * K / 4 / NTR;   // 16-byte pieces per thread of a 64 x K block
  constexpr int PP = BC * BC / 4 / NTR;  // ... of the 64 x 64 P
  constexpr int PO = BC * 16 / NTR;      // dO values per thread (the chunk's 16 columns)
  constexpr int WV = NTR / 64;           // waves
  constexpr int TPW = (K / 16 + WV - 1) / WV;
  static_assert(PB >= 1 && PP >= 1 && PO >= 1, "pieces per thread");
  __shared__ __align__(16) float sX[K * 16];
  __shared__ __align__(16) float sO[BC * 16];
  __shared__ __align__(16) float sDD[BC * 16];
  __shared__ __align__(16) float sP[BC * LP];
  __shared__ __align__(16) float sKt[BC * LKt];
  __shared__ __align__(16) float sQe[BC * LC];
  __shared__ __align__(16) float sW[BC * LC];
  __shared__ float sG[K];
  const int nh = blockIdx.x % chains8, s = blockIdx.x / chains8;
  if (nh >= N * H) return;
  const int n = nh / H, h = nh % H, c0 = 16 * s;
  const int tid = threadIdx.x, w = tid >> 6, lm = tid & 15, lg = (tid >> 4) & 3;
  for (int e = tid; e < K * 16; e += NTR)
    sX[e] = dfin ? dfin[((size_t)nh * K + e / 16) * V + c0 + e % 16] : 0.f;
  const int first = seq_first[n], last = seq_first[n + 1];
  int64_t s0, s1;
  seq_range(cu, N, T, n, &s0, &s1);
  struct Regs {
    f32x4 p[PP], k[PB], q[PB], w[PB];
    MT o[PO];
    float g;
  };
  Regs ra, rb;
  // chunk c's rows are tokens s0 + 64 (c - first) + r; rows past the sequence read its last
  // token (in bounds) and are zeroed when stored
  auto fetch = [&](Regs& x, int c) {
    const float* rc = rec + ((size_t)c * H + h) * R::floats;
#pragma unroll
    for (int u = 0; u < PP; ++u) x.p[u] = reinterpret_cast<const f32x4*>(rc + R::oP)[tid + NTR * u];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      x.k[u] = reinterpret_cast<const f32x4*>(rc + R::oKt)[tid + NTR * u];
      x.q[u] = reinterpret_cast<const f32x4*>(rc + R::oQe)[tid + NTR * u];
      x.w[u] = reinterpret_cast<const f32x4*>(rc + R::oW)[tid + NTR * u];
    }
    x.g = rc[R::oGam + tid % K];
    const int64_t tok = s0 + (int64_t)(c - first) * BC;
#pragma unroll
    for (int u = 0; u < PO; ++u) {
      const int e = tid + NTR * u;
      const int64_t t = min(tok + e / 16, s1 - 1);
      x.o[u] = dO[(t * H + h) * (int64_t)V + c0 + e % 16];
    }
  };
  // one chunk: stage its registers, start loading chunk c - 2 into them, then its products
  auto step = [&](Regs& x, int c) {
    const int len = (int)min((int64_t)BC, s1 - (s0 + (int64_t)(c - first) * BC));
    lds_barrier();  // the previous chunk's reads of LDS are done
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int e = tid + NTR * u;
      *reinterpret_cast<f32x4*>(sP + (e / (BC / 4)) * LP + 4 * (e % (BC / 4))) = x.p[u];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = tid + NTR * u, o = (e / (K / 4)), q4 = 4 * (e % (K / 4));
      *reinterpret_cast<f32x4*>(sKt + o * LKt + q4) = x.k[u];
      *reinterpret_cast<f32x4*>(sQe + o * LC + q4) = x.q[u];
      *reinterpret_cast<f32x4*>(sW + o * LC + q4) = x.w[u];
    }
#pragma unroll
    for (int u = 0; u < PO; ++u) {
      const int e = tid + NTR * u;
      sO[e] = e / 16 < len ? to_f32(x.o[u]) : 0.f;
    }
    if (tid < K) sG[tid] = x.g;
    fetch(x, max(c - 2, first));
    lds_barrier();
    for (int e = tid; e < K * 16; e += NTR)
      ckX[(((size_t)c * H + h) * K + e / 16) * V + c0 + e % 16] = sX[e];
    // dDelta rows 16 w .. (waves 0-3): P^T dO (P_ri = 0 for r < i, so the steps start at
    // r = 16 w) + Kt X
    if (w < 4) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      for (int r0 = 16 * w; r0 < BC; r0 += 4)
        d = mfma4(sP[(r0 + lg) * LP + 16 * w + lm], sO[(r0 + lg) * 16 + lm], d);
#pragma unroll 8
      for (int mm = 0; mm < K; mm += 4)
        d = mfma4(sKt[(16 * w + lm) * LKt + mm + lg], sX[(mm + lg) * 16 + lm], d);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * lg + r;
        sDD[row * 16 + lm] = d[r];
        dDl[(((size_t)c * H + h) * BC + row) * V + c0 + lm] = d[r];
      }
    }
    lds_barrier();
    // X_prev tiles: diag(gamma) X + Qe^T dO - W^T dDelta
    f32x4 acc[TPW];
#pragma unroll
    for (int qq = 0; qq < TPW; ++qq) {
      const int mt = w + WV * qq;
      if (mt < K / 16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * lg + r;
          acc[qq][r] = sG[row] * sX[row * 16 + lm];
        }
#pragma unroll 8
        for (int r0 = 0; r0 < BC; r0 += 4) {
          acc[qq] = mfma4(sQe[(r0 + lg) * LC + 16 * mt + lm], sO[(r0 + lg) * 16 + lm], acc[qq]);
          acc[qq] = mfma4(-sW[(r0 + lg) * LC + 16 * mt + lm], sDD[(r0 + lg) * 16 + lm], acc[qq]);
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int qq = 0; qq < TPW; ++qq) {
      const int mt = w + WV * qq;
      if (mt < K / 16)
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * mt + 4 * lg + r) * 16 + lm] = acc[qq][r];
    }
  };
  if (first < last) {
    fetch(ra, last - 1);
    fetch(rb, max(last - 2, first));
  }
  for (int c = last - 1; c >= first; c -= 2) {
    step(ra, c);
    if (c - 1 < first) break;
    step(rb, c - 1);
  }
  if (dinit) {
    __syncthreads();
    for (int e = tid; e < K * 16; e += NTR)
      dinit[((size_t)nh * K + e / 16) * V + c0 + e % 16] = sX[e];
  }
}

// ---------------------------------------------------------------- per-chunk gradients
// As in the record kernel, the barriers order LDS only: no kernel here reads global memory that
// it writes itself, so none waits for its stores (or for loads it has in flight) at a barrier.
// (a) dP = lower(dO Delta^T); with S (chunk start) and X (chunk end) streamed from HBM:
//     dO S^T, dW = -dDelta S^T, Delta X^T and rowsum(S * X)
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTGA, 8) void bwd_ga_kernel(
    const MT* __restrict__ dO, const float* __restrict__ ckS, const float* __restrict__ ckX,
    const float* __restrict__ Dl, const float* __restrict__ dDl, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, float* __restrict__ scr) {
  using G = GScr<K>;
  // Every product here sums over the value columns; they run over parts of VC columns with
  // the partial tiles kept in registers, so LDS holds 64 x VC and K x VC blocks (70 KB at
  // K = V = 128) and two workgroups share a CU.
  constexpr int VC = V > 64 ? 64 : V;
  constexpr int L = VC + 4;  // every block here is read along its rows
  constexpr int TK = mmf_tiles<K, NTGA>(), TC = mmf_tiles<BC, NTGA>();
  __shared__ __align__(16) float sO[BC * L];
  __shared__ __align__(16) float sD[BC * L];  // dDelta, then Delta
  __shared__ __align__(16) float sS[K * L];   // S, then X
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)c * H + h;
  float* sc = scr + ch_h * G::floats;
  const float* S = ckS + ch_h * K * V;
  const float* X = ckX + ch_h * K * V;
  // rowsum(S * X): NP neighbouring threads per key channel (K NP is a whole number of waves),
  // then a shuffle reduction among them
  {
    constexpr int NP = NTGA / K < V / 4 ? NTGA / K : V / 4, VP = V / NP;
    if (threadIdx.x < K * NP) {
      const int m = threadIdx.x / NP, part = threadIdx.x % NP;
      float dg = 0.f;
#pragma unroll
      for (int vv = 0; vv < VP; vv += 4)
        dg += dot4(*reinterpret_cast<const f32x4*>(S + m * V + part * VP + vv),
                   *reinterpret_cast<const f32x4*>(X + m * V + part * VP + vv));
#pragma unroll
      for (int o = 1; o < NP; o <<= 1) dg += __shfl_xor(dg, o);
      if (part == 0) sc[G::oDG + m] = dg;
    }
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // dO S^T and dW = -dDelta S^T
  {
    f32x4 r1[TK], dw[TK];
#pragma unroll
    for (int i = 0; i < TK; ++i) r1[i] = dw[i] = z;
    for (int c0 = 0; c0 < V; c0 += VC) {
      load_rows<VC, L, NTGA, MT, V>(sO, dO, ch.tok, ch.len, H, h, c0);
      load_block<VC, L, NTGA, BC, V>(sD, dDl + ch_h * BC * V + c0);
      load_block<VC, L, NTGA, K, V>(sS, S + c0);
      lds_barrier();
      mmf_acc<K, VC, false, true, L, L, NTGA>(sO, sS, r1);
      mmf_acc<K, VC, false, true, L, L, NTGA>(sD, sS, dw);
      lds_barrier();
    }
    mmf_out<K, NTGA>(r1, [&](int r, int m, float x) { sc[G::oR1 + r * K + m] = x; });
    mmf_out<K, NTGA>(dw, [&](int r, int m, float x) { sc[G::oDW + r * K + m] = -x; });
  }
  // Delta X^T and dP = lower(dO Delta^T)
  {
    f32x4 dk[TK], dp[TC];
#pragma unroll
    for (int i = 0; i < TK; ++i) dk[i] = z;
#pragma unroll
    for (int i = 0; i < TC; ++i) dp[i] = z;
    for (int c0 = 0; c0 < V; c0 += VC) {
      if (V > VC) load_rows<VC, L, NTGA, MT, V>(sO, dO, ch.tok, ch.len, H, h, c0);
      load_block<VC, L, NTGA, BC, V>(sD, Dl + ch_h * BC * V + c0);
      load_block<VC, L, NTGA, K, V>(sS, X + c0);
      lds_barrier();
      mmf_acc<K, VC, false, true, L, L, NTGA>(sD, sS, dk);
      mmf_acc<BC, VC, false, true, L, L, NTGA>(sO, sD, dp);
      lds_barrier();
    }
    mmf_out<K, NTGA>(dk, [&](int r, int m, float x) { sc[G::oDKt + r * K + m] = x; });
    mmf_out<BC, NTGA>(dp, [&](int i, int j, float x) {
      if (j <= i) sc[G::oDPA + i * BC + j] = x;
    });
  }
}

// (b) dv = diag(beta) T^T dDelta, T^T dW, dT = dDelta (beta V)^T + dW (beta Ke)^T,
//     dA = strict_lower(-T^T dT T^T), and dbeta's terms rowsum(V * T^T dDelta) and
//     rowsum(Ke * T^T dW)
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTG, 8) void bwd_gb_kernel(
    const MT* __restrict__ k, const MT* __restrict__ v, const MT* __restrict__ g,
    const MT* __restrict__ beta, const float* __restrict__ rec, const float* __restrict__ dDl, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, float* __restrict__ scr,
    float* __restrict__ grad_v, float* __restrict__ grad_beta) {
  using R = BRec<K, V>;
  using G = GScr<K>;
  // The value columns and the key channels run in parts of at most 64; dT's partial tiles stay
  // in registers until both sums are done. 64 KB of LDS and 64 VGPRs: two workgroups per CU.
  constexpr int VC = V > 64 ? 64 : V, KC = K > 64 ? 64 : K;
  // row strides: blocks read both along and down their rows (T, dDelta, dW) 20 more than a
  // multiple of 64 floats (no bank conflict along rows, at most two-way down columns); dT,
  // read down its columns, 80; v and Ke, read along rows, + 4
  constexpr int LT = BC + 20, LDT = BC + 16;
  constexpr int LDD = VC + ((84 - VC) & 63), LDW = KC + ((84 - KC) & 63), LVV = VC + 4, LKE = KC + 4;
  constexpr int LA = (LDD > LDW ? LDD : LDW) > LT ? (LDD > LDW ? LDD : LDW) : LT;
  constexpr int LB0 = LVV > LKE ? LVV : LKE, LB = LB0 > LDT ? LB0 : LDT;
  __shared__ __align__(16) float sT[BC * LT];
  __shared__ __align__(16) float bufA[BC * LA];  // dDelta (part), dW (part), then M1 = T^T dT
  __shared__ __align__(16) float bufB[BC * LB];  // v (part), Ke (part), then dT
  __shared__ float sBeta[BC], sDb[BC];
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)c * H + h;
  const float* rc = rec + ch_h * R::floats;
  float* sc = scr + ch_h * G::floats;
  load_block<BC, LT, NTG>(sT, rc + R::oT);
  if (threadIdx.x < BC) {
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
    sDb[threadIdx.x] = 0.f;
  }
  constexpr int TC = mmf_tiles<BC, NTG>();
  f32x4 dT[TC];
#pragma unroll
  for (int i = 0; i < TC; ++i) dT[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int c0 = 0; c0 < V; c0 += VC) {
    load_block<VC, LDD, NTG, BC, V>(bufA, dDl + ch_h * BC * V + c0);
    load_rows<VC, LVV, NTG, MT, V>(bufB, v, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    // T^T dDelta: dv = beta T^T dDelta, dbeta += rowsum(v * T^T dDelta)
    mmf<VC, BC, true, false, LT, LDD, NTG>(sT, bufA, [&](int r, int cc, float x) {
      if (r < ch.len) grad_v[((ch.tok + r) * (int64_t)H + h) * V + c0 + cc] = sBeta[r] * x;
      const float y = row16_sum(bufB[r * LVV + cc] * x);  // the 16 lanes of a row hold one r
      if ((threadIdx.x & 15) == 0) atomicAdd(&sDb[r], y);
    });
    lds_barrier();
    for (int e = threadIdx.x; e < BC * VC; e += NTG) bufB[(e / VC) * LVV + e % VC] *= sBeta[e / VC];
    lds_barrier();
    // dT += dDelta (beta V)^T over the part's columns
    mmf_acc<BC, VC, false, true, LDD, LVV, NTG>(bufA, bufB, dT);
    lds_barrier();
  }
#pragma unroll 1
  for (int c0 = 0; c0 < K; c0 += KC) {
    // dW and Ke = k e^b (the decay is per channel, so a part's cumulative sum is its own)
    load_block<KC, LDW, NTG, BC, K>(bufA, sc + G::oDW + c0);
    load_rows<KC, LKE, NTG, MT, K>(bufB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LKE, NTG>(bufB);
    lds_barrier();
    mul_rows_exp2<KC, LKE, NTG, MT, K>(bufB, k, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    // T^T dW; dbeta += rowsum(Ke * T^T dW)
    mmf<KC, BC, true, false, LT, LDW, NTG>(sT, bufA, [&](int r, int cc, float x) {
      sc[G::oTDW + r * K + c0 + cc] = x;
      const float y = row16_sum(bufB[r * LKE + cc] * x);
      if ((threadIdx.x & 15) == 0) atomicAdd(&sDb[r], y);
    });
    lds_barrier();
    for (int e = threadIdx.x; e < BC * KC; e += NTG) bufB[(e / KC) * LKE + e % KC] *= sBeta[e / KC];
    lds_barrier();
    // dT += dW (beta Ke)^T over the part's channels
    mmf_acc<BC, KC, false, true, LDW, LKE, NTG>(bufA, bufB, dT);
    lds_barrier();
  }
  mmf_out<BC, NTG>(dT, [&](int i, int j, float x) { bufB[i * LDT + j] = x; });
  lds_barrier();
  // M1 = T^T dT into bufA (row stride LT), then dA = strict_lower(-M1 T^T)
  mmf<BC, BC, true, false, LT, LDT, NTG>(sT, bufB, [&](int r, int cc, float x) { bufA[r * LT + cc] = x; });
  lds_barrier();
  mmf<BC, BC, false, true, LT, LT, NTG>(bufA, sT, [&](int i, int j, float x) {
    if (j < i) sc[G::oDPA + j * BC + i] = -x;  // dA_ij, transposed above dP
  });
  // dbeta's T-side terms; the gradient kernel adds the rest (one part of the key channels
  // per workgroup) with atomics
  if (threadIdx.x < ch.len) grad_beta[(ch.tok + threadIdx.x) * (int64_t)H + h] = sDb[threadIdx.x];
}

// (c) the decay-weighted pairwise sums and the per-token gradients of q, k, log alpha, beta
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTG, 8) void bwd_gc_kernel(
    const MT* __restrict__ q, const MT* __restrict__ k, const MT* __restrict__ g,
    const MT* __restrict__ beta, int H, const ChunkRow* __restrict__ chunks,
    const int32_t* __restrict__ ntot, const float* __restrict__ scr, float* __restrict__ grad_q,
    float* __restrict__ grad_k, float* __restrict__ grad_g, float* __restrict__ grad_beta) {
  using G = GScr<K>;
  // Everything here is per key channel except dbeta's sum over the channels, so each
  // workgroup takes one part of KC channels (blockIdx.z) and adds its share of dbeta to
  // grad_beta atomically. dP and dA share one 64 x 64 block (dP on and below the diagonal,
  // dA transposed above it): 70 KB of LDS, and at 64 VGPRs two workgroups share a CU.
  constexpr int KC = K > 64 ? 64 : K;
  constexpr int LK = KC + 4;
  __shared__ __align__(16) float sQ[BC * LK];  // q (part), then the per-token decay gradient
  __shared__ __align__(16) float sK[BC * LK];
  __shared__ __align__(16) float sB[BC * LK];
  __shared__ __align__(16) float sM[BC * 68];  // [i][j] = dP_ij (j <= i), [j][i] = dA_ij (j < i)
  __shared__ float sBeta[BC], sDb[BC], sRed[KC];
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)c * H + h;
  const float* sc = scr + ch_h * G::floats;
  load_block<BC, 68, NTG>(sM, sc + G::oDPA);
  if (threadIdx.x < BC) {
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
    sDb[threadIdx.x] = 0.f;
  }
  // thread: key channel c0 + m, rows i = i0 + NG u (interleaved; a row's two pairwise sums
  // have 65 terms together, so every thread has the same work)
  constexpr int NG = NTG / KC, RB = BC / NG;
  const int m = threadIdx.x % KC, i0 = threadIdx.x / KC;
  const int c0 = blockIdx.z * KC;
  {
    load_rows<KC, LK, NTG, MT, K>(sQ, q, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTG, MT, K>(sK, k, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTG, MT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    if (threadIdx.x < KC) sRed[threadIdx.x] = 0.f;
    // this thread's rows of dO S^T, T^T dW and Delta X^T, in flight through the scan
    float r1v[RB], tdw[RB], dkv[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int i = i0 + NG * u;
      r1v[u] = sc[G::oR1 + i * K + c0 + m];
      tdw[u] = sc[G::oTDW + i * K + c0 + m];
      dkv[u] = sc[G::oDKt + i * K + c0 + m];
    }
    lds_barrier();
    cumsum_log2<KC, LK, NTG>(sB);
    lds_barrier();  // LDS only: the loads above stay in flight
    const float bl = sB[(BC - 1) * LK + m];
    float db[RB];
    float red = 0.f;
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int i = i0 + NG * u;
      const float bi = sB[i * LK + m], qi = sQ[i * LK + m], ki = sK[i * LK + m];
      const float dpii = sM[i * 68 + i];
      // sum_{j <= i} dP_ij k_j e^{b_i - b_j} and sum_{j < i} dA_ij k_j e^{b_i - b_j}
      float s1 = dpii * ki, s2 = 0.f;
      for (int j = 0; j < i; ++j) {
        const float w = sK[j * LK + m] * exp2_f(bi - sB[j * LK + m]);
        s1 += sM[i * 68 + j] * w;
        s2 += sM[j * 68 + i] * w;
      }
      // sum_{r >= i} (dA_ri beta_r k_r + dP_ri q_r) e^{b_r - b_i}  (dA_ii = 0)
      float s3 = dpii * qi;
      for (int r = i + 1; r < BC; ++r)
        s3 += (sM[i * 68 + r] * sBeta[r] * sK[r * LK + m] + sM[r * 68 + i] * sQ[r * LK + m]) *
              exp2_f(sB[r * LK + m] - bi);
      const float eb = exp2_f(bi);
      const float dq = r1v[u] * eb + s1;
      const float dke = sBeta[i] * (tdw[u] * eb + s2);
      const float dkt = dkv[u] * exp2_f(bl - bi);
      const float dk = dke + s3 + dkt;
      {
        // dbeta's sum over the part's key channels of row i: the lanes sharing i (a whole
        // wave, or 32 lanes at K = 32) reduce first, then one LDS atomic
        float y = row16_sum(ki * s2);
        y += __shfl_xor(y, 16);
        if constexpr (KC >= 64) y += __shfl_xor(y, 32);
        if (threadIdx.x % (KC >= 64 ? 64 : KC) == 0) atomicAdd(&sDb[i], y);
      }
      red += ki * dkt;
      db[u] = qi * dq + ki * (dke - s3 - dkt);
      if (i < ch.len) {
        const int64_t o = ((ch.tok + i) * (int64_t)H + h) * K + c0 + m;
        grad_q[o] = dq;
        grad_k[o] = dk;
      }
    }
    atomicAdd(&sRed[m], red);
    lds_barrier();  // every read of sQ done
#pragma unroll
    for (int u = 0; u < RB; ++u) sQ[(i0 + NG * u) * LK + m] = db[u];
    lds_barrier();
    // log alpha: reverse cumulative sum of db over the chunk, the last token also carrying
    // sum_i k_i * dKt_i and gamma * rowsum(S * X); NTG / KC neighbouring threads per channel,
    // as in cumsum_log2 but from the last row
    {
      constexpr int P = NTG / KC, RP = BC / P;
      const int cm = threadIdx.x / P, part = threadIdx.x % P;
      float x[RP];
      float run = 0.f;
#pragma unroll
      for (int r = RP - 1; r >= 0; --r) {
        run += sQ[(part * RP + r) * LK + cm];
        x[r] = run;
      }
      float post = run;  // rows from this thread's first to the last, after the scan
#pragma unroll
      for (int o = 1; o < P; o <<= 1) {
        const float y = __shfl_down(post, o, P);
        if (part + o < P) post += y;
      }
      post -= run;  // the rows after this thread's
      post += sRed[cm] + sc[G::oDG + c0 + cm] * exp2_f(sB[(BC - 1) * LK + cm]);
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int row = part * RP + r;
        if (row < ch.len) grad_g[((ch.tok + row) * (int64_t)H + h) * K + c0 + cm] = x[r] + post;
      }
    }
  }
  if (threadIdx.x < ch.len) atomicAdd(&grad_beta[(ch.tok + threadIdx.x) * (int64_t)H + h], sDb[threadIdx.x]);
}

// ---------------------------------------------------------------- host
hipError_t launch_chunk_rows(const int32_t* cu, int N, int64_t T, int64_t ub, int32_t* seq_first,
                             ChunkRow* rows, hipStream_t st) {
  hipLaunchKernelGGL(bwd_seq_kernel, dim3(1), dim3(NT), 0, st, cu, N, T, seq_first);
  if (ub > 0)
    hipLaunchKernelGGL(bwd_chunk_kernel, dim3((unsigned)((ub + NT - 1) / NT)), dim3(NT), 0, st, cu,
                       N, T, (const int32_t*)seq_first, ub, rows);
  return hipGetLastError();
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

template <int K, int V>
static void bwd_sizes(int64_t ub, int H, size_t* rec_f, size_t* scr_f) {
  *rec_f = (size_t)ub * H * BRec<K, V>::floats;
  *scr_f = (size_t)ub * H * GScr<K>::floats;
}

bool make_bwd_plan(int N, int64_t T, int H, int K, int V, BwdPlan* p) {
  if (N <= 0 || H <= 0 || T < 0) return false;
  int64_t ub = (T + (int64_t)N * (BC - 1)) / BC;
  if (ub > T) ub = T;
  p->ub = ub;
  size_t rec_f = 0, scr_f = 0;
#define KDA_BWD_SIZES(KK, VV) \
  if (K == KK && V == VV) bwd_sizes<KK, VV>(ub, H, &rec_f, &scr_f);
  KDA_BWD_SIZES(32, 32) KDA_BWD_SIZES(32, 64) KDA_BWD_SIZES(32, 128)
  KDA_BWD_SIZES(64, 32) KDA_BWD_SIZES(64, 64) KDA_BWD_SIZES(64, 128)
  KDA_BWD_SIZES(128, 32) KDA_BWD_SIZES(128, 64) KDA_BWD_SIZES(128, 128)
#undef KDA_BWD_SIZES
  if (rec_f == 0 && ub > 0) return false;
  const size_t chv = (size_t)ub * H;
  size_t off = 0;
  p->off_seq = off;
  off += al256((size_t)(N + 1) * 4);
  p->off_chunks = off;
  off += al256((size_t)ub * sizeof(ChunkRow));
  p->off_rec = off;
  off += al256(rec_f * 4);
  p->off_ckS = off;
  off += al256(chv * K * V * 4);
  p->off_ckX = off;
  off += al256(chv * K * V * 4);
  p->off_D = off;
  off += al256(chv * BC * V * 4);
  p->off_dD = off;
  off += al256(chv * BC * V * 4);
  p->off_scr = off;
  off += al256(scr_f * 4);
  p->total_bytes = off;
  return true;
}

template <int K, int V, typename MT>
static hipError_t launch_bwd_t(const BwdArgs& a, const BwdPlan& p) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + p.off_seq);
  ChunkRow* chunks = reinterpret_cast<ChunkRow*>(ws + p.off_chunks);
  float* rec = reinterpret_cast<float*>(ws + p.off_rec);
  float* ckS = reinterpret_cast<float*>(ws + p.off_ckS);
  float* ckX = reinterpret_cast<float*>(ws + p.off_ckX);
  float* Dl = reinterpret_cast<float*>(ws + p.off_D);
  float* dDl = reinterpret_cast<float*>(ws + p.off_dD);
  float* scr = reinterpret_cast<float*>(ws + p.off_scr);
  const int N = a.num_seqs, H = a.num_heads;
  const int32_t* ntot = seq_first + N;
  const MT *q = (const MT*)a.q, *k = (const MT*)a.k, *v = (const MT*)a.v, *g = (const MT*)a.g,
           *beta = (const MT*)a.beta, *dO = (const MT*)a.dO;
  launch_chunk_rows(a.cu_seqlens, N, a.total_tokens, p.ub, seq_first, chunks, st);
  const dim3 cgrid((unsigned)(p.ub > 0 ? p.ub : 1), (unsigned)H);
  if (p.ub > 0)
    hipLaunchKernelGGL((bwd_prep_kernel<K, V, MT>), cgrid, dim3(NTP), 0, st, q, k, v, g, beta, H,
                       (const ChunkRow*)chunks, ntot, rec);
  const int chains8 = (N * H + 7) / 8 * 8;
  const dim3 sgrid((unsigned)(chains8 * (V / 16)));
  hipLaunchKernelGGL((bwd_fstate_kernel<K, V>), sgrid, dim3(NTR), 0, st, (const float*)rec,
                     a.init_state, (const int32_t*)seq_first, N, H, chains8, ckS, Dl);
  hipLaunchKernelGGL((bwd_rstate_kernel<K, V, MT>), sgrid, dim3(NTR), 0, st, (const float*)rec, dO,
                     a.dfinal, a.cu_seqlens, a.total_tokens, (const int32_t*)seq_first, N, H,
                     chains8, ckX, dDl, a.grad_init);
  if (p.ub > 0) {
    hipLaunchKernelGGL((bwd_ga_kernel<K, V, MT>), cgrid, dim3(NTGA), 0, st, dO, (const float*)ckS,
                       (const float*)ckX, (const float*)Dl, (const float*)dDl, H,
                       (const ChunkRow*)chunks, ntot, scr);
    hipLaunchKernelGGL((bwd_gb_kernel<K, V, MT>), cgrid, dim3(NTG), 0, st, k, v, g, beta,
                       (const float*)rec, (const float*)dDl, H, (const ChunkRow*)chunks, ntot, scr,
                       a.grad_v, a.grad_beta);
    const dim3 pgrid(cgrid.x, cgrid.y, (unsigned)(K > 64 ? K / 64 : 1));  // key-channel parts
    hipLaunchKernelGGL((bwd_gc_kernel<K, V, MT>), pgrid, dim3(NTG), 0, st, q, k, g, beta, H,
                       (const ChunkRow*)chunks, ntot, (const float*)scr, a.grad_q, a.grad_k,
                       a.grad_g, a.grad_beta);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdArgs& a, const BwdPlan& p) {
#define KDA_BWD_CASE(KK, VV)                                                     \
  if (a.dk == KK && a.dv == VV)                                                  \
    return a.dtype_bf16 ? launch_bwd_t<KK, VV, bf16>(a, p) : launch_bwd_t<KK, VV, float>(a, p);
  KDA_BWD_CASE(32, 32) KDA_BWD_CASE(32, 64) KDA_BWD_CASE(32, 128)
  KDA_BWD_CASE(64, 32) KDA_BWD_CASE(64, 64) KDA_BWD_CASE(64, 128)
  KDA_BWD_CASE(128, 32) KDA_BWD_CASE(128, 64) KDA_BWD_CASE(128, 128)
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
