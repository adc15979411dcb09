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
// Every stored value and every sum is fp32 (the chunk's inputs, bf16 or fp32, are exact in
// fp32). The matrix-core products of the two chains and of the S/X product kernel take each
// fp32 operand as two bf16 parts (hi = bf16(x), lo = bf16(x - hi); hi*hi + hi*lo + lo*hi on the
// bf16 matrix cores, about 2^-16 relative error per product); the record kernel, the T-side
// and the gradient kernel use the fp32 matrix cores. Kernels:
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

// Every per-(chunk, head) array of a segment (record, scratch, S_c, X_c, Delta, dDelta) is
// head-major: entry h * (chunks of the segment) + chunk. A chain then walks through adjacent
// entries, so its reads and writes stay within a few pages instead of one new page per chunk.
// per-(chunk, head) fp32 record of the backward, row-major blocks
template <int K, int V>
struct BRec {
  static constexpr int oT = 0;                 // T = (I + A)^{-1}        [64][64]
  static constexpr int oP = oT + BC * BC;      // P^T (upper incl.)      [64][64]
  static constexpr int oW = oP + BC * BC;      // W                       [64][K]
  static constexpr int oKt = oW + BC * K;      // Kt = k e^{b_last - b}   [64][K]
  static constexpr int oQe = oKt + BC * K;     // Qe^T, Qe = q e^b        [K][64]
  static constexpr int oU = oQe + BC * K;      // U^T                     [V][64]
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
  static constexpr int KP = K > 64 ? K / 64 : 1;  // key-channel parts of the gradient kernel
  static constexpr int oDB = oDG + K;          // dbeta per part          [KP][64]
  static constexpr int floats = (oDB + KP * BC + 63) / 64 * 64;
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
// MT: v; GT: q, k, log alpha and beta (fp32 when an input-option pass formed them). LIGHT
// writes only what the boundary pass's chain reads (W, Kt, U, gamma): no P, Qe or T.
template <int K, int V, typename MT, typename GT, bool LIGHT = false>
__global__ __launch_bounds__(NTP, 4) void bwd_prep_kernel(
    const GT* __restrict__ q, const GT* __restrict__ k, const MT* __restrict__ v,
    const GT* __restrict__ g, const GT* __restrict__ beta, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, int cb,
    float* __restrict__ rec) {
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
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;  // chunk of the segment, of the call
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  float* rc = rec + ((size_t)h * gridDim.x + lc) * R::floats;
  if (threadIdx.x < BC)
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
  // A_ij = beta_i sum_c k_ic k_jc e^{b_ic - b_jc} (j < i) and P_ij = sum_c q_ic k_jc e^{..} (j <= i),
  // summed over the parts (off-diagonal 16 x 16 blocks on the fp32 matrix cores)
  PairAcc acc;
  pair_acc_init<NTP>(acc);
  for (int c0 = 0; c0 < K; c0 += KC) {
    if constexpr (!LIGHT) load_rows<KC, LQ, NTP, GT, K>(sQ, q, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTP, GT, K>(sK, k, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTP, GT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LK, NTP>(sB);
    lds_barrier();
    // Qe, Kt, gamma of the part (rows past len hold q = k = 0, and b stays at its last value)
    for (int e = threadIdx.x; e < BC * KC; e += NTP) {
      const int r = e / KC, cc = e % KC;
      const float br = sB[r * LK + cc], bl = sB[(BC - 1) * LK + cc];
      rc[R::oKt + r * K + c0 + cc] = sK[r * LK + cc] * exp2_f(bl - br);
    }
    if constexpr (!LIGHT) {
      for (int e = threadIdx.x; e < BC * KC; e += NTP) {  // transposed: token index fastest
        const int r = e % BC, cc = e / BC;
        const float br = sB[r * LK + cc];
        rc[R::oQe + (c0 + cc) * BC + r] = sQ[r * LQ + cc] * exp2_f(br);
      }
    }
    if (threadIdx.x < KC) rc[R::oGam + c0 + threadIdx.x] = exp2_f(sB[(BC - 1) * LK + threadIdx.x]);
    pair_acc_part<KC, LK, LQ, !LIGHT>(acc, sQ, sK, sB);
    lds_barrier();  // the part's reads done before the next part overwrites it
  }
  // (the solve reads A below the diagonal only)
  pair_acc_out(acc, [&](int i, int j, float x) { sA[i * 68 + j] = sBeta[i] * x; },
               [&](int i, int j, float x) {
                 if constexpr (!LIGHT) rc[R::oP + j * BC + i] = x;
               });
  if constexpr (!LIGHT) {
    for (int e = threadIdx.x; e < BC * BC; e += NTP)  // below P^T's diagonal
      if (e / BC > e % BC) rc[R::oP + e] = 0.f;
  }
  lds_barrier();
  // T = (I + A)^{-1} over A (blocked: diagonal blocks by substitution, the rest on the matrix
  // cores), then to the record
  unit_lower_inverse_blocked<NTP>(sT);
  if constexpr (!LIGHT)
    for (int e = threadIdx.x; e < BC * BC; e += NTP) rc[R::oT + e] = sT[(e / BC) * 68 + e % BC];
  // W = T diag(beta) (k e^b), part by part
  for (int c0 = 0; c0 < K; c0 += KC) {
    load_rows<KC, LK, NTP, GT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LK, NTP>(sB);
    lds_barrier();
    mul_rows_exp2<KC, LK, NTP, GT, K>(sB, k, ch.tok, ch.len, H, h, c0);
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
      rc[R::oU + (c0 + cc) * BC + r] = x;
    });
    lds_barrier();
  }
}

// ---------------------------------------------------------------- the chains
// One workgroup per (sequence, head, 16 value columns); the slices of one chain share
// blockIdx % 8 (one XCD's L2) with blockIdx = slice * chains8 + chain.
// Wave v of the chain_waves<K>() waves holds the key-channel rows [16 v HCT, 16 (v + 1) HCT)
// of the chain's state (S forwards, X backwards) in registers, as 16 x 16 matrix-core result
// tiles: lane (n, g) = (lane % 16, lane / 16) holds rows 16 t + 4 g + r (r = 0..3) of column
// n. Such a tile is, unchanged, the B operand of four 16x16x4 steps in which lane group g
// supplies the reduction index 16 t + 4 g + r at step r; the A operand of those steps for
// output row i is then the four values at those indices: one 16-byte load along a row of a
// row-major block, or four loads along a column. So the state and Delta (or dDelta) stay in
// registers; the only exchange per chunk is that of the Delta partials (each wave sums over
// its own rows of the state) through LDS, with one barrier. A chunk's record values load
// while the chunk before is computed (two register sets, each refilled two chunks ahead).
template <int K>
constexpr int chain_waves() { return K >= 64 ? 4 : 2; }
// A compiler-only fence: memory operations are not moved across it (no wait is issued).
__device__ __forceinline__ void fence_compiler() { asm volatile("" ::: "memory"); }

// Forward in time: S_c (chunk start) and Delta = U - W S per chunk, S' = diag(gamma) S + Kt^T
// Delta. The chunks [cb, ce) of one segment (records, S_c and Delta indexed from cb). A
// sequence that began before the segment starts from ck_in (its state at chunk cb,
// [H][K][V]); one that goes on past it leaves its state at chunk ce in ck_out (when given).
// STORE = false runs the chain for that state alone.
template <int K, int V, bool STORE>
__global__ __launch_bounds__(64 * chain_waves<K>()) void bwd_fstate_kernel(
    const float* rec, const float* __restrict__ init, const int32_t* __restrict__ seq_first,
    int N, int H, int chains8, int cb, int ce, const float* __restrict__ ck_in,
    float* __restrict__ ck_out, float* __restrict__ ckS, float* __restrict__ Dl) {
  using R = BRec<K, V>;
  constexpr int NW = chain_waves<K>(), HCT = K / 16 / NW, NTT = BC / 16, TPW = NTT / NW;
  __shared__ __align__(16) f32x4 sX[2][NW][NTT][64];  // [parity][wave][token tile][lane]
  const int nh = blockIdx.x % chains8, s = blockIdx.x / chains8;
  if (nh >= N * H) return;
  const int n = nh / H, h = nh % H, c0 = 16 * s;
  const int lane = threadIdx.x & 63, v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lm = lane & 15, lg = lane >> 4;
  const int r0 = 16 * v * HCT;  // this wave's first key channel
  const int sfirst = seq_first[n], slast = seq_first[n + 1];
  const int first = max(sfirst, cb), last = min(slast, ce);  // the sequence's chunks here
  if (first >= last) return;
  const float* src = sfirst < cb ? ck_in + (size_t)h * K * V : (init ? init + (size_t)nh * K * V : nullptr);
  f32x4 S[HCT];
#pragma unroll
  for (int j = 0; j < HCT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[j][r] = src ? src[(r0 + 16 * j + 4 * lg + r) * V + c0 + lm] : 0.f;
  struct Frags {
    f32x4 w[NTT][HCT];   // W[16 t + lm][r0 + 16 j + 4 lg .. +3]
    f32x4 kt[HCT][NTT];  // Kt[16 t + 4 lg + r][r0 + 16 j + lm], r = 0..3 (a column of Kt)
    f32x4 u[TPW];        // U^T[c0 + lm][16 (v + NW i) + 4 lg .. +3]: the wave's own tiles of Delta
    f32x4 gam[HCT];      // gamma[r0 + 16 j + 4 lg .. +3]
  };
  // The record pieces of chunk c, each loaded by its own helper so that a step can refill a
  // register as soon as it has used it (the loads then trickle out between the matrix-core
  // steps instead of queueing up at the end of the chunk, where a full memory pipeline would
  // stall the wave). Each refill ends in a compiler fence that keeps it where it is.
  auto rec_of = [&](int c) { return rec + ((size_t)h * (ce - cb) + (c - cb)) * R::floats; };
  auto ld_w = [&](Frags& f, const float* rc, int t) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
      f.w[t][j] = *reinterpret_cast<const f32x4*>(rc + R::oW + (16 * t + lm) * K + r0 + 16 * j + 4 * lg);
  };
  auto ld_kt = [&](Frags& f, const float* rc, int t) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) f.kt[j][t][r] = rc[R::oKt + (16 * t + 4 * lg + r) * K + r0 + 16 * j + lm];
  };
  auto ld_u = [&](Frags& f, const float* rc) {
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      f.u[i] = *reinterpret_cast<const f32x4*>(rc + R::oU + (c0 + lm) * BC + 16 * (v + NW * i) + 4 * lg);
  };
  auto ld_gam = [&](Frags& f, const float* rc) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
      f.gam[j] = *reinterpret_cast<const f32x4*>(rc + R::oGam + r0 + 16 * j + 4 * lg);
  };
  auto fetch = [&](Frags& f, int c) {
    const float* rc = rec_of(c);
#pragma unroll
    for (int t = 0; t < NTT; ++t) ld_w(f, rc, t);
#pragma unroll
    for (int t = 0; t < NTT; ++t) ld_kt(f, rc, t);
    ld_u(f, rc);
    ld_gam(f, rc);
  };
  // live = false (the odd tail's second step) computes but stores nothing and keeps S. The
  // set f is refilled with chunk c + 2 piece by piece.
  auto step = [&](Frags& f, int c, bool live) {
    const int par = (c - first) & 1;
    const size_t ch_h = (size_t)h * (ce - cb) + (c - cb);
    const float* rn = rec_of(min(c + 2, last - 1));
    if (STORE && live) {
#pragma unroll
      for (int j = 0; j < HCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) ckS[(ch_h * K + r0 + 16 * j + 4 * lg + r) * V + c0 + lm] = S[j][r];
    }
    // this wave's part of -Delta: W S over its rows, minus U on its own tiles
    f32x4 D[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) D[t] = (t % NW == v) ? -f.u[t / NW] : f32x4{0.f, 0.f, 0.f, 0.f};
    ld_u(f, rn);
    fence_compiler();
    const X3<HCT> sx = x3_of<HCT>(S);
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      D[t] = x3_mma(x3_of<HCT>(f.w[t]), sx, D[t]);
      ld_w(f, rn, t);
      fence_compiler();
    }
#pragma unroll
    for (int t = 0; t < NTT; ++t) sX[par][v][t][lane] = D[t];
    lds_barrier();
    // Delta, the partials summed in wave order (the same in every wave)
    f32x4 Dd[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 x = sX[par][0][t][lane];
#pragma unroll
      for (int u = 1; u < NW; ++u) x += sX[par][u][t][lane];
      Dd[t] = -x;
    }
    if (STORE && live) {
#pragma unroll
      for (int t = 0; t < NTT; ++t)
        if (t % NW == v)
#pragma unroll
          for (int r = 0; r < 4; ++r) Dl[(ch_h * BC + 16 * t + 4 * lg + r) * V + c0 + lm] = Dd[t][r];
    }
    // S' = diag(gamma) S + Kt^T Delta (two accumulators per tile)
    f32x4 A0[HCT], A1[HCT];
#pragma unroll
    for (int j = 0; j < HCT; ++j) {
      A0[j] = f.gam[j] * S[j];
      A1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ld_gam(f, rn);
    fence_compiler();
    // over the tokens in 32-steps (token tiles 2 s and 2 s + 1), one accumulator per step
    static_assert(NTT == 4, "two 32-token steps per chunk");
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const X3<2> dx = x3_of(Dd[2 * s2], Dd[2 * s2 + 1]);
#pragma unroll
      for (int j = 0; j < HCT; ++j) {
        const X3<2> kx = x3_of(f.kt[j][2 * s2], f.kt[j][2 * s2 + 1]);
        if (s2 == 0) A0[j] = x3_mma(kx, dx, A0[j]);
        else A1[j] = x3_mma(kx, dx, A1[j]);
      }
      ld_kt(f, rn, 2 * s2);
      ld_kt(f, rn, 2 * s2 + 1);
      fence_compiler();
    }
#pragma unroll
    for (int j = 0; j < HCT; ++j) S[j] = live ? A0[j] + A1[j] : S[j];
  };
  // Two chunks per iteration and no branch between them: a branch there would let the compiler
  // sink the second register set's loads to their use, which ends the prefetch.
  Frags fa, fb;
  fetch(fa, first);
  fetch(fb, min(first + 1, last - 1));
  for (int c = first; c < last; c += 2) {
    step(fa, c, true);
    step(fb, c + 1, c + 1 < last);
  }
  if (ck_out != nullptr && slast > ce) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) ck_out[((size_t)h * K + r0 + 16 * j + 4 * lg + r) * V + c0 + lm] = S[j][r];
  }
}

// Backwards in time: X_c (the gradient at the chunk's end), dDelta = P^T dO + Kt X per chunk,
// X_prev = diag(gamma) X + Qe^T dO - W^T dDelta; at the end the initial state's gradient.
// The chunks [cb, ce) of one segment, as in the forward chain: a sequence that goes on past
// the segment starts from x_in (its X at chunk ce - 1, [H][K][V]), and one that began before it
// leaves its X at chunk cb - 1 in x_out instead of writing the initial state's gradient.
// Empty sequences (initial state = final state) are handled by the segment at chunk 0.
template <int K, int V, typename MT>
__global__ __launch_bounds__(64 * chain_waves<K>()) void bwd_rstate_kernel(
    const float* rec, const MT* dO, const float* __restrict__ dfin,
    const int32_t* __restrict__ cu, int64_t T, const int32_t* __restrict__ seq_first, int N, int H,
    int chains8, int cb, int ce, const float* __restrict__ x_in, float* __restrict__ x_out,
    float* __restrict__ ckX, float* __restrict__ dDl, float* __restrict__ dinit) {
  using R = BRec<K, V>;
  constexpr int NW = chain_waves<K>(), HCT = K / 16 / NW, NTT = BC / 16, TPW = NTT / NW;
  __shared__ __align__(16) f32x4 sX[2][NW][NTT][64];  // [parity][wave][token tile][lane]
  const int nh = blockIdx.x % chains8, s = blockIdx.x / chains8;
  if (nh >= N * H) return;
  const int n = nh / H, h = nh % H, c0 = 16 * s;
  const int lane = threadIdx.x & 63, v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lm = lane & 15, lg = lane >> 4;
  const int r0 = 16 * v * HCT;  // this wave's first key channel
  const int sfirst = seq_first[n], slast = seq_first[n + 1];
  const int first = max(sfirst, cb), last = min(slast, ce);  // the sequence's chunks here
  if (sfirst < slast ? first >= last : cb != 0) return;
  const bool carried = sfirst < slast && slast > ce;  // X comes from the next segment
  const float* src = carried ? x_in + (size_t)h * K * V : (dfin ? dfin + (size_t)nh * K * V : nullptr);
  f32x4 X[HCT];
#pragma unroll
  for (int j = 0; j < HCT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) X[j][r] = src ? src[(r0 + 16 * j + 4 * lg + r) * V + c0 + lm] : 0.f;
  int64_t s0, s1;
  seq_range(cu, N, T, n, &s0, &s1);
  struct Frags {
    f32x4 kt[NTT][HCT];  // Kt[16 t + lm][r0 + 16 j + 4 lg .. +3]
    f32x4 wt[HCT][NTT];  // W[16 t + 4 lg + r][r0 + 16 j + lm], r = 0..3 (a column of W)
    f32x4 qt[HCT][NTT];  // Qe^T[r0 + 16 j + lm][16 t + 4 lg .. +3]
    f32x4 pt[TPW][NTT];  // P^T[16 (v + NW i) + lm][16 t + 4 lg .. +3] (zero for t below the tile)
    MT o[NTT][4];        // dO[token 16 t + 4 lg + r][c0 + lm]
    f32x4 gam[HCT];
  };
  // chunk c's rows are tokens s0 + 64 (c - sfirst) + row; rows past the sequence read its last
  // token (in bounds) and are zeroed when used. As in the forward chain, each piece has its own
  // loader, so that a step refills a register right after its last use.
  auto rec_of = [&](int c) { return rec + ((size_t)h * (ce - cb) + (c - cb)) * R::floats; };
  auto ld_kt = [&](Frags& f, const float* rc, int t) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
      f.kt[t][j] = *reinterpret_cast<const f32x4*>(rc + R::oKt + (16 * t + lm) * K + r0 + 16 * j + 4 * lg);
  };
  auto ld_wt = [&](Frags& f, const float* rc, int t) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) f.wt[j][t][r] = rc[R::oW + (16 * t + 4 * lg + r) * K + r0 + 16 * j + lm];
  };
  auto ld_qt = [&](Frags& f, const float* rc, int t) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
      f.qt[j][t] = *reinterpret_cast<const f32x4*>(rc + R::oQe + (r0 + 16 * j + lm) * BC + 16 * t + 4 * lg);
  };
  auto ld_pt = [&](Frags& f, const float* rc) {
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int t = 0; t < NTT; ++t)
        f.pt[i][t] = *reinterpret_cast<const f32x4*>(rc + R::oP + (16 * (v + NW * i) + lm) * BC + 16 * t + 4 * lg);
  };
  auto ld_o = [&](Frags& f, int c) {
    const int64_t tok = s0 + (int64_t)(c - sfirst) * BC;
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tt = min(tok + 16 * t + 4 * lg + r, s1 - 1);
        f.o[t][r] = dO[(tt * H + h) * (int64_t)V + c0 + lm];
      }
  };
  auto ld_gam = [&](Frags& f, const float* rc) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
      f.gam[j] = *reinterpret_cast<const f32x4*>(rc + R::oGam + r0 + 16 * j + 4 * lg);
  };
  auto fetch = [&](Frags& f, int c) {
    const float* rc = rec_of(c);
#pragma unroll
    for (int t = 0; t < NTT; ++t) ld_kt(f, rc, t);
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      ld_wt(f, rc, t);
      ld_qt(f, rc, t);
    }
    ld_pt(f, rc);
    ld_o(f, c);
    ld_gam(f, rc);
  };
  // live = false (the odd tail's second step) computes but stores nothing and keeps X. The
  // set f is refilled with chunk c - 2 piece by piece.
  auto step = [&](Frags& f, int c, bool live) {
    const int par = (last - 1 - c) & 1;
    const size_t ch_h = (size_t)h * (ce - cb) + (c - cb);
    const int len = (int)min((int64_t)BC, s1 - (s0 + (int64_t)(c - sfirst) * BC));
    const int cn = max(c - 2, first);
    const float* rn = rec_of(cn);
    if (live) {
#pragma unroll
      for (int j = 0; j < HCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) ckX[(ch_h * K + r0 + 16 * j + 4 * lg + r) * V + c0 + lm] = X[j][r];
    }
    f32x4 od[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) od[t][r] = 16 * t + 4 * lg + r < len ? to_f32(f.o[t][r]) : 0.f;
    ld_o(f, cn);
    fence_compiler();
    // this wave's part of dDelta: Kt X over its rows, plus P^T dO on its own tiles
    f32x4 D[NTT];
    // dO is exact in bf16 when it comes in bf16: its low part is zero
    constexpr bool OX = sizeof(MT) == 2;
    static_assert(NTT == 4, "two 32-token steps per chunk");
    const X3<2> ox[2] = {x3_of(od[0], od[1]), x3_of(od[2], od[3])};
    const X3<HCT> xx = x3_of<HCT>(X);
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      D[t] = x3_mma(x3_of<HCT>(f.kt[t]), xx, f32x4{0.f, 0.f, 0.f, 0.f});
      ld_kt(f, rn, t);
      fence_compiler();
    }
    // P^T dO on the wave's own tiles, over the 32-token steps at or right of the diagonal
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
      if (tt % NW == v)
#pragma unroll
        for (int s2 = tt / 2; s2 < 2; ++s2)
          D[tt] = x3_mma<OX>(x3_of(f.pt[tt / NW][2 * s2], f.pt[tt / NW][2 * s2 + 1]), ox[s2], D[tt]);
    ld_pt(f, rn);
    fence_compiler();
#pragma unroll
    for (int t = 0; t < NTT; ++t) sX[par][v][t][lane] = D[t];
    // diag(gamma) X + Qe^T dO needs no dDelta: formed while the partials meet
    f32x4 A0[HCT], A1[HCT];
#pragma unroll
    for (int j = 0; j < HCT; ++j) {
      A0[j] = f.gam[j] * X[j];
      A1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ld_gam(f, rn);
    fence_compiler();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int j = 0; j < HCT; ++j)
        A0[j] = x3_mma<OX>(x3_of(f.qt[j][2 * s2], f.qt[j][2 * s2 + 1]), ox[s2], A0[j]);
      ld_qt(f, rn, 2 * s2);
      ld_qt(f, rn, 2 * s2 + 1);
      fence_compiler();
    }
    lds_barrier();
    f32x4 dD[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      f32x4 x = sX[par][0][t][lane];
#pragma unroll
      for (int u = 1; u < NW; ++u) x += sX[par][u][t][lane];
      dD[t] = x;
    }
    if (live) {
#pragma unroll
      for (int t = 0; t < NTT; ++t)
        if (t % NW == v)
#pragma unroll
          for (int r = 0; r < 4; ++r) dDl[(ch_h * BC + 16 * t + 4 * lg + r) * V + c0 + lm] = dD[t][r];
    }
    // X_prev = diag(gamma) X + Qe^T dO - W^T dDelta
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const X3<2> dx = x3_of(dD[2 * s2], dD[2 * s2 + 1]);
#pragma unroll
      for (int j = 0; j < HCT; ++j)
        A1[j] = x3_mma(x3_of(f.wt[j][2 * s2], f.wt[j][2 * s2 + 1]), dx, A1[j]);
      ld_wt(f, rn, 2 * s2);
      ld_wt(f, rn, 2 * s2 + 1);
      fence_compiler();
    }
#pragma unroll
    for (int j = 0; j < HCT; ++j) X[j] = live ? A0[j] - A1[j] : X[j];
  };
  if (first < last) {
    // two chunks per iteration, no branch between them (as in the forward chain)
    Frags fa, fb;
    fetch(fa, last - 1);
    fetch(fb, max(last - 2, first));
    for (int c = last - 1; c >= first; c -= 2) {
      step(fa, c, true);
      step(fb, c - 1, c - 1 >= first);
    }
  }
  float* dst = sfirst < cb ? x_out + (size_t)h * K * V : (dinit ? dinit + (size_t)nh * K * V : nullptr);
  if (dst != nullptr) {
#pragma unroll
    for (int j = 0; j < HCT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(r0 + 16 * j + 4 * lg + r) * V + c0 + lm] = X[j][r];
  }
}

// ---------------------------------------------------------------- per-chunk gradients
// As in the record kernel, the barriers order LDS only: no kernel here reads global memory that
// it writes itself, so none waits for its stores (or for loads it has in flight) at a barrier.
// (a) dP = lower(dO Delta^T); with S (chunk start) and X (chunk end) streamed from HBM:
//     dO S^T, dW = -dDelta S^T, Delta X^T and rowsum(S * X)
template <int K, int V, typename MT>
__global__ __launch_bounds__(NTGA, 2) void bwd_ga_kernel(
    const MT* __restrict__ dO, const float* __restrict__ ckS, const float* __restrict__ ckX,
    const float* __restrict__ Dl, const float* __restrict__ dDl, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, int cb,
    float* __restrict__ scr) {
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
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;  // chunk of the segment, of the call
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)h * gridDim.x + lc;
  float* sc = scr + ch_h * G::floats;
  const float* S = ckS + ch_h * K * V;
  const float* X = ckX + ch_h * K * V;
  // rowsum(S * X) rides along with the products, so that neither state is read twice: while
  // a part of S is in LDS each thread keeps EPT of its values (key channel rm, columns rc ..;
  // TPR neighbouring threads share a channel) and multiplies them with the same part of X in
  // the second loop. With more than two parts (V = 256) the kept values would not fit in
  // registers: a pass of its own over both states forms the sum first instead.
  constexpr int NPART = V / VC, EPT = K * VC / NTGA, TPR = VC / EPT;
  constexpr bool FUSE = NPART <= 2;
  static_assert(EPT >= 1 && K * VC == EPT * NTGA && TPR <= 64, "rowsum split");
  const int rm = threadIdx.x / TPR, rc = (threadIdx.x % TPR) * EPT;
  float keep[FUSE ? NPART : 1][EPT];
  if constexpr (!FUSE) {
    constexpr int NP = NTGA / K < V / 4 ? NTGA / K : V / 4, VP = V / NP;
    if (threadIdx.x < K * NP) {
      const int m = threadIdx.x / NP, part = threadIdx.x % NP;
      float s = 0.f;
#pragma unroll
      for (int vv = 0; vv < VP; vv += 4)
        s += dot4(*reinterpret_cast<const f32x4*>(S + m * V + part * VP + vv),
                  *reinterpret_cast<const f32x4*>(X + m * V + part * VP + vv));
#pragma unroll
      for (int o = 1; o < NP; o <<= 1) s += __shfl_xor(s, o);
      if (part == 0) sc[G::oDG + m] = s;
    }
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // dO S^T and dW = -dDelta S^T
  {
    f32x4 r1[TK], dw[TK];
#pragma unroll
    for (int i = 0; i < TK; ++i) r1[i] = dw[i] = z;
#pragma unroll
    for (int pi = 0; pi < NPART; ++pi) {
      const int c0 = pi * VC;
      load_rows<VC, L, NTGA, MT, V>(sO, dO, ch.tok, ch.len, H, h, c0);
      load_block<VC, L, NTGA, BC, V>(sD, dDl + ch_h * BC * V + c0);
      load_block<VC, L, NTGA, K, V>(sS, S + c0);
      lds_barrier();
      mmx_acc<K, VC, false, true, L, L, NTGA>(sO, sS, r1);
      mmx_acc<K, VC, false, true, L, L, NTGA>(sD, sS, dw);
      if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) keep[pi][e] = sS[rm * L + rc + e];
      }
      lds_barrier();
    }
    mmf_out<K, NTGA>(r1, [&](int r, int m, float x) { sc[G::oR1 + r * K + m] = x; });
    mmf_out<K, NTGA>(dw, [&](int r, int m, float x) { sc[G::oDW + r * K + m] = -x; });
  }
  // Delta X^T, dP = lower(dO Delta^T) and rowsum(S * X)
  {
    f32x4 dk[TK], dp[TC];
#pragma unroll
    for (int i = 0; i < TK; ++i) dk[i] = z;
#pragma unroll
    for (int i = 0; i < TC; ++i) dp[i] = z;
    float dg = 0.f;
#pragma unroll
    for (int pi = 0; pi < NPART; ++pi) {
      const int c0 = pi * VC;
      if (V > VC) load_rows<VC, L, NTGA, MT, V>(sO, dO, ch.tok, ch.len, H, h, c0);
      load_block<VC, L, NTGA, BC, V>(sD, Dl + ch_h * BC * V + c0);
      load_block<VC, L, NTGA, K, V>(sS, X + c0);
      lds_barrier();
      mmx_acc<K, VC, false, true, L, L, NTGA>(sD, sS, dk);
      mmx_acc<BC, VC, false, true, L, L, NTGA>(sO, sD, dp);
      if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) dg += keep[FUSE ? pi : 0][e] * sS[rm * L + rc + e];
      }
      lds_barrier();
    }
    if constexpr (FUSE) {
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) dg += __shfl_xor(dg, o);
      if (threadIdx.x % TPR == 0) sc[G::oDG + rm] = dg;
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
template <int K, int V, typename MT, typename GT>
__global__ __launch_bounds__(NTG, 8) void bwd_gb_kernel(
    const GT* __restrict__ k, const MT* __restrict__ v, const GT* __restrict__ g,
    const GT* __restrict__ beta, const float* __restrict__ rec, const float* __restrict__ dDl, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, int cb,
    float* __restrict__ scr, float* __restrict__ grad_v, float* __restrict__ grad_beta) {
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
  // dbeta's row sums per 16-column tile of a part, added to sDb in tile order (no atomics: the
  // gradients are the same bit for bit on every run)
  __shared__ float sDbp[BC][4];
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;  // chunk of the segment, of the call
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)h * gridDim.x + lc;
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
      if ((threadIdx.x & 15) == 0) sDbp[r][cc >> 4] = y;
    });
    lds_barrier();
    if (threadIdx.x < BC) {
      float y = sDb[threadIdx.x];
#pragma unroll
      for (int t = 0; t < VC / 16; ++t) y += sDbp[threadIdx.x][t];
      sDb[threadIdx.x] = y;
    }
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
    load_rows<KC, LKE, NTG, GT, K>(bufB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LKE, NTG>(bufB);
    lds_barrier();
    mul_rows_exp2<KC, LKE, NTG, GT, K>(bufB, k, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    // T^T dW; dbeta += rowsum(Ke * T^T dW)
    mmf<KC, BC, true, false, LT, LDW, NTG>(sT, bufA, [&](int r, int cc, float x) {
      sc[G::oTDW + r * K + c0 + cc] = x;
      const float y = row16_sum(bufB[r * LKE + cc] * x);
      if ((threadIdx.x & 15) == 0) sDbp[r][cc >> 4] = y;
    });
    lds_barrier();
    if (threadIdx.x < BC) {
      float y = sDb[threadIdx.x];
#pragma unroll
      for (int t = 0; t < KC / 16; ++t) y += sDbp[threadIdx.x][t];
      sDb[threadIdx.x] = y;
    }
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
  // dbeta's T-side terms; the per-part sums of the gradient kernel are added after it
  if (threadIdx.x < ch.len) grad_beta[(ch.tok + threadIdx.x) * (int64_t)H + h] = sDb[threadIdx.x];
}

// (c) the decay-weighted pairwise sums and the per-token gradients of q, k, log alpha, beta
template <int K, int V, typename GT>
__global__ __launch_bounds__(NTG, 8) void bwd_gc_kernel(
    const GT* __restrict__ q, const GT* __restrict__ k, const GT* __restrict__ g,
    const GT* __restrict__ beta, int H, const ChunkRow* __restrict__ chunks,
    const int32_t* __restrict__ ntot, int cb, float* __restrict__ scr, float* __restrict__ grad_q,
    float* __restrict__ grad_k, float* __restrict__ grad_g) {
  using G = GScr<K>;
  // Everything here is per key channel except dbeta's sum over the channels, so each
  // workgroup takes one part of KC channels (blockIdx.z) and leaves its share of dbeta in the
  // scratch (bwd_beta_kernel adds the parts in order). dP and dA share one 64 x 64 block (dP on and below the diagonal,
  // dA transposed above it): 70 KB of LDS, and at 64 VGPRs two workgroups share a CU.
  constexpr int KC = K > 64 ? 64 : K;
  constexpr int LK = KC + 4;
  __shared__ __align__(16) float sQ[BC * LK];  // q (part), then the per-token decay gradient
  __shared__ __align__(16) float sK[BC * LK];
  __shared__ __align__(16) float sB[BC * LK];
  __shared__ __align__(16) float sM[BC * 68];  // [i][j] = dP_ij (j <= i), [j][i] = dA_ij (j < i)
  __shared__ float sBeta[BC], sDb[BC];
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;  // chunk of the segment, of the call
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const size_t ch_h = (size_t)h * gridDim.x + lc;
  float* sc = scr + ch_h * G::floats;
  load_block<BC, 68, NTG>(sM, sc + G::oDPA);
  if (threadIdx.x < BC) {
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(ch.tok + threadIdx.x) * (int64_t)H + h]) : 0.f;
    sDb[threadIdx.x] = 0.f;
  }
  const int c0 = blockIdx.z * KC;
  // sDbp: dbeta's row sums per channel tile, added in tile order (no atomics)
  constexpr int NCT = KC / 16;  // channel tiles of the part
  __shared__ float sDbp[NCT][BC];
  {
    load_rows<KC, LK, NTG, GT, K>(sQ, q, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTG, GT, K>(sK, k, ch.tok, ch.len, H, h, c0);
    load_rows<KC, LK, NTG, GT, K>(sB, g, ch.tok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KC, LK, NTG>(sB);
    lds_barrier();
    // Wave w takes row block X = w / NCT (rows 16 X ..) and channel tile ct = w % NCT; lane
    // (n, lg) holds rows 16 X + 4 lg + r (r = 0..3) of channel m = 16 ct + n, as a matrix-core
    // result tile. With b non-increasing along the chunk, the three decay-weighted sums
    //   s1_i = sum_{j <= i} dP_ij k_j e^{b_i - b_j},  s2_i = sum_{j < i} dA_ij k_j e^{b_i - b_j},
    //   s3_i = sum_{r >= i} (dA_ri beta_r k_r + dP_ri q_r) e^{b_r - b_i}          (dA_ii = 0)
    // split into the blocks before (after) X, on the fp32 matrix cores with the decay split at
    // the block boundary (e^{b_i - b_j} = e^{b_i - b_e} e^{b_e - b_j}, b_e the last token before
    // block X; for s3 the last token of X; both factors at most 1), and the diagonal block X,
    // pairwise. (The NCT * 4 waves cover the part; at 32 key channels the others idle here.)
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, lg = lane >> 4;
    const int X = w / NCT, ct = w % NCT, m = 16 * ct + n;
    const bool active = w < 4 * NCT;
    f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = s1, s3 = s1;
    float bi[4];
    if (active) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bi[r] = sB[(16 * X + 4 * lg + r) * LK + m];
      const int ia = 16 * X + n;  // the A operands' row
      if (X >= 1) {
        const float e = sB[(16 * X - 1) * LK + m];
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll 2
        for (int j0 = 0; j0 < 16 * X; j0 += 4) {
          const int jj = j0 + lg;
          const float kh = sK[jj * LK + m] * exp2_f(e - sB[jj * LK + m]);
          a1 = mfma4(sM[ia * 68 + jj], kh, a1);  // dP_ij
          a2 = mfma4(sM[jj * 68 + ia], kh, a2);  // dA_ij (kept at [j][i])
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float f = exp2_f(bi[r] - e);
          s1[r] = a1[r] * f;
          s2[r] = a2[r] * f;
        }
      }
      if (X <= 2) {
        const float e = sB[(16 * X + 15) * LK + m];
        f32x4 a3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int r0 = 16 * X + 16; r0 < BC; r0 += 4) {
          const int rr = r0 + lg;
          const float f = exp2_f(sB[rr * LK + m] - e);
          a3 = mfma4(sM[ia * 68 + rr], sBeta[rr] * sK[rr * LK + m] * f, a3);  // dA_ri (at [i][r])
          a3 = mfma4(sM[rr * 68 + ia], sQ[rr * LK + m] * f, a3);                // dP_ri
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s3[r] = a3[r] * exp2_f(e - bi[r]);
      }
      // the diagonal block, pairwise: j <= i feeds s1 (and s2 for j < i), j >= i feeds s3
#pragma clang loop unroll(disable)
      for (int jj = 0; jj < 16; ++jj) {
        const int j = 16 * X + jj;
        const float kj = sK[j * LK + m], bj = sB[j * LK + m], qj = sQ[j * LK + m];
        const float kbj = sBeta[j] * kj;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int il = 4 * lg + r, i = 16 * X + il;
          const float xij = sM[i * 68 + j], xji = sM[j * 68 + i];
          const float ex = exp2_f(jj <= il ? bi[r] - bj : bj - bi[r]);
          s1[r] += jj <= il ? xij * kj * ex : 0.f;
          s2[r] += jj < il ? xji * kj * ex : 0.f;
          s3[r] += jj >= il ? ((jj > il ? xij * kbj : 0.f) + xji * qj) * ex : 0.f;
        }
      }
    }
    float db[4];
    float red = 0.f;
    if (active) {
      const float bl = sB[(BC - 1) * LK + m];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * X + 4 * lg + r;
        const float r1v = sc[G::oR1 + i * K + c0 + m], tdw = sc[G::oTDW + i * K + c0 + m];
        const float dkv = sc[G::oDKt + i * K + c0 + m];
        const float qi = sQ[i * LK + m], ki = sK[i * LK + m];
        const float eb = exp2_f(bi[r]);
        const float dq = r1v * eb + s1[r];
        const float dke = sBeta[i] * (tdw * eb + s2[r]);
        const float dkt = dkv * exp2_f(bl - bi[r]);
        const float dk = dke + s3[r] + dkt;
        // dbeta's sum over the tile's 16 channels of row i (the 16 lanes of a lane group)
        const float y = row16_sum(ki * s2[r]);
        if (n == 0) sDbp[ct][i] = y;
        red += ki * dkt;
        db[r] = qi * dq + ki * (dke - s3[r] - dkt);
        if (i < ch.len) {
          const int64_t o = ((ch.tok + i) * (int64_t)H + h) * K + c0 + m;
          grad_q[o] = dq;
          grad_k[o] = dk;
        }
      }
      red += __shfl_xor(red, 16);
      red += __shfl_xor(red, 32);
    }
    lds_barrier();  // every read of sQ and sK done
    if (active) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sQ[(16 * X + 4 * lg + r) * LK + m] = db[r];
      if (lg == 0) sK[X * LK + m] = red;  // this row block's share of sum_i k_i dKt_i
    }
    if (threadIdx.x < BC) {
      float y = 0.f;
#pragma unroll
      for (int t = 0; t < NCT; ++t) y += sDbp[t][threadIdx.x];
      sDb[threadIdx.x] = y;
    }
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
      float red = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) red += sK[u * LK + cm];
      post += red + sc[G::oDG + c0 + cm] * exp2_f(sB[(BC - 1) * LK + cm]);
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int row = part * RP + r;
        if (row < ch.len) grad_g[((ch.tok + row) * (int64_t)H + h) * K + c0 + cm] = x[r] + post;
      }
    }
  }
  if (threadIdx.x < BC) sc[G::oDB + blockIdx.z * BC + threadIdx.x] = sDb[threadIdx.x];
}

// dbeta = the T-side terms (already in grad_beta) + the gradient kernel's parts, in part order
template <int K>
__global__ __launch_bounds__(BC) void bwd_beta_kernel(int H, const ChunkRow* __restrict__ chunks,
                                                      const int32_t* __restrict__ ntot, int cb,
                                                      const float* __restrict__ scr,
                                                      float* __restrict__ grad_beta) {
  using G = GScr<K>;
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const int i = threadIdx.x;
  if (i >= ch.len) return;
  const float* sc = scr + ((size_t)h * gridDim.x + lc) * G::floats + G::oDB;
  float* gb = grad_beta + (ch.tok + i) * (int64_t)H + h;
  float y = *gb;
#pragma unroll
  for (int p = 0; p < G::KP; ++p) y += sc[p * BC + i];
  *gb = y;
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

// fp32 values the backward keeps per (chunk, head) of a segment: the record, the gradient
// kernels' scratch, and (see make_bwd_plan) the chunk-start state S, the chunk-end gradient X,
// Delta and dDelta. Zero sizes for unsupported head dims.
struct BwdFloats {
  size_t rec, scr, all;
};
static BwdFloats bwd_floats(int K, int V) {
#define KDA_BWD_FLOATS(KK, VV)                                                           \
  if (K == KK && V == VV)                                                                \
    return BwdFloats{(size_t)BRec<KK, VV>::floats, (size_t)GScr<KK>::floats,             \
                     (size_t)BRec<KK, VV>::floats + GScr<KK>::floats + 2 * (size_t)KK * VV + \
                         2 * (size_t)BC * VV};
  KDA_BWD_FLOATS(32, 32) KDA_BWD_FLOATS(32, 64) KDA_BWD_FLOATS(32, 128)
  KDA_BWD_FLOATS(64, 32) KDA_BWD_FLOATS(64, 64) KDA_BWD_FLOATS(64, 128)
  KDA_BWD_FLOATS(128, 32) KDA_BWD_FLOATS(128, 64) KDA_BWD_FLOATS(128, 128)
  KDA_BWD_FLOATS(32, 256) KDA_BWD_FLOATS(64, 256) KDA_BWD_FLOATS(128, 256)
#undef KDA_BWD_FLOATS
  return BwdFloats{0, 0, 0};
}

bool make_bwd_plan(int N, int64_t T, int H, int K, int V, uint32_t options, int64_t seg_chunks,
                   BwdPlan* p) {
  if (N <= 0 || H <= 0 || T < 0) return false;
  const BwdFloats fl = bwd_floats(K, V);
  if (fl.all == 0) return false;
  int64_t ub = (T + (int64_t)N * (BC - 1)) / BC;
  if (ub > T) ub = T;
  p->ub = ub;
  p->seg = (seg_chunks <= 0 || seg_chunks >= ub) ? (ub > 0 ? ub : 1) : seg_chunks;
  p->nseg = ub > 0 ? (ub + p->seg - 1) / p->seg : 1;
  // the per-chunk arrays are indexed with 32-bit chunk numbers
  if (ub >= (1LL << 31)) return false;
  const size_t chv = (size_t)p->seg * H;
  size_t off = 0;
  // with input options: the processed q, k, log alpha and beta (fp32, every token), and with
  // the scalar gate the per-channel gradient of log alpha before its sum over the channels
  const size_t tk = al256((size_t)T * H * K * 4);
  p->off_opt_q = p->off_opt_k = p->off_opt_g = p->off_opt_b = p->off_opt_dg = 0;
  if (options != 0) {
    p->off_opt_q = off;
    p->off_opt_k = off + tk;
    p->off_opt_g = off + 2 * tk;
    p->off_opt_b = off + 3 * tk;
    off += 3 * tk + al256((size_t)T * H * 4);
    if (options & OPT_SCALAR_GATE) {
      p->off_opt_dg = off;
      off += tk;
    }
  }
  p->off_seq = off;
  off += al256((size_t)(N + 1) * 4);
  p->off_chunks = off;
  off += al256((size_t)ub * sizeof(ChunkRow));
  // one [H][K][V] state per segment boundary: S of the sequence that spans it (forward pass),
  // then its X (reverse pass); none with a single segment
  p->off_ck = off;
  if (p->nseg > 1) off += al256((size_t)p->nseg * H * K * V * 4);
  p->off_rec = off;
  off += al256(chv * fl.rec * 4);
  p->off_ckS = off;
  off += al256(chv * K * V * 4);
  p->off_ckX = off;
  off += al256(chv * K * V * 4);
  p->off_D = off;
  off += al256(chv * BC * V * 4);
  p->off_dD = off;
  off += al256(chv * BC * V * 4);
  p->off_scr = off;
  off += al256(chv * fl.scr * 4);
  p->total_bytes = off;
  return true;
}

bool fit_bwd_plan(int N, int64_t T, int H, int K, int V, uint32_t options, size_t bytes,
                  BwdPlan* p, int64_t step) {
  if (!make_bwd_plan(N, T, H, K, V, options, 0, p)) return false;
  if (p->total_bytes <= bytes) return true;
  if (step < 1) step = 1;
  // the longest segments that fit: from the per-chunk bytes down, shorter until it fits
  const size_t per_chunk = (size_t)H * bwd_floats(K, V).all * 4;
  int64_t e = (int64_t)min(bytes / per_chunk, (size_t)p->ub - 1) / step * step;
  while (e >= step) {
    if (!make_bwd_plan(N, T, H, K, V, options, e, p)) return false;
    if (p->total_bytes <= bytes) return true;
    e = step > 1 ? e - step : e > 64 ? e - e / 32 : e - 1;
  }
  return false;
}

int64_t default_bwd_segment(int H, int K, int V) {
  const size_t per_chunk = (size_t)H * bwd_floats(K, V).all * 4;
  if (per_chunk == 0) return 1;
  const int64_t e = (int64_t)(BWD_SEGMENT_BYTES / per_chunk);
  return e > 1 ? e : 1;
}

// MT: v and dO; GT: q, k, log alpha and beta
template <int K, int V, typename MT, typename GT>
static hipError_t launch_bwd_t(const BwdArgs& a, const BwdPlan& p) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + p.off_seq);
  ChunkRow* chunks = reinterpret_cast<ChunkRow*>(ws + p.off_chunks);
  float* ck = reinterpret_cast<float*>(ws + p.off_ck);
  float* rec = reinterpret_cast<float*>(ws + p.off_rec);
  float* ckS = reinterpret_cast<float*>(ws + p.off_ckS);
  float* ckX = reinterpret_cast<float*>(ws + p.off_ckX);
  float* Dl = reinterpret_cast<float*>(ws + p.off_D);
  float* dDl = reinterpret_cast<float*>(ws + p.off_dD);
  float* scr = reinterpret_cast<float*>(ws + p.off_scr);
  const int N = a.num_seqs, H = a.num_heads;
  const int32_t* ntot = seq_first + N;
  const GT *q = (const GT*)a.q, *k = (const GT*)a.k, *g = (const GT*)a.g, *beta = (const GT*)a.beta;
  const MT *v = (const MT*)a.v, *dO = (const MT*)a.dO;
  launch_chunk_rows(a.cu_seqlens, N, a.total_tokens, p.ub, seq_first, chunks, st);
  const int chains8 = (N * H + 7) / 8 * 8;
  const dim3 sgrid((unsigned)(chains8 * (V / 16)));
  const size_t ckb = (size_t)H * K * V;  // one boundary's state
  auto bound = [&](int64_t s) { return ck + (size_t)s * ckb; };
  // segment s: chunks [cb, ce) of the call
  auto range = [&](int64_t s, int* cb, int* ce) {
    *cb = (int)(s * p.seg);
    *ce = (int)min((s + 1) * p.seg, p.ub);
  };
  auto prep = [&](int cb, int ce, auto light) {
    if (ce > cb)
      hipLaunchKernelGGL((bwd_prep_kernel<K, V, MT, GT, decltype(light)::value>),
                         dim3((unsigned)(ce - cb), (unsigned)H), dim3(NTP), 0, st, q, k, v, g,
                         beta, H, (const ChunkRow*)chunks, ntot, cb, rec);
  };
  // The state of the sequence that spans the start of segment s (chunk s * seg): from the
  // forward's checkpoint of that chunk, or from a forward pass through the segments but the
  // last that keeps each one's state at its end
  auto ck_start = [&](int64_t s) -> const float* {
    if (s == 0) return nullptr;
    return a.ckpt ? a.ckpt + (size_t)(s * p.seg / a.ckpt_interval - 1) * ckb : bound(s);
  };
  for (int64_t s = 0; a.ckpt == nullptr && s + 1 < p.nseg; ++s) {
    int cb, ce;
    range(s, &cb, &ce);
    prep(cb, ce, std::true_type());
    hipLaunchKernelGGL((bwd_fstate_kernel<K, V, false>), sgrid, dim3(64 * chain_waves<K>()), 0, st,
                       (const float*)rec, a.init_state, (const int32_t*)seq_first, N, H, chains8,
                       cb, ce, (const float*)(s > 0 ? bound(s) : nullptr), bound(s + 1),
                       (float*)nullptr, (float*)nullptr);
  }
  // Backwards through the segments: the record again, S_c and Delta from the segment's start
  // state, X_c and dDelta from its end gradient (X of the next segment, kept at the boundary),
  // then the chunks' gradients
  for (int64_t s = p.nseg - 1; s >= 0; --s) {
    int cb, ce;
    range(s, &cb, &ce);
    prep(cb, ce, std::false_type());
    hipLaunchKernelGGL((bwd_fstate_kernel<K, V, true>), sgrid, dim3(64 * chain_waves<K>()), 0, st,
                       (const float*)rec, a.init_state, (const int32_t*)seq_first, N, H, chains8,
                       cb, ce, ck_start(s), (float*)nullptr, ckS, Dl);
    hipLaunchKernelGGL((bwd_rstate_kernel<K, V, MT>), sgrid, dim3(64 * chain_waves<K>()), 0, st, (const float*)rec,
                       dO, a.dfinal, a.cu_seqlens, a.total_tokens, (const int32_t*)seq_first, N, H,
                       chains8, cb, ce, (const float*)(s + 1 < p.nseg ? bound(s + 1) : nullptr),
                       s > 0 ? bound(s) : (float*)nullptr, ckX, dDl, a.grad_init);
    if (ce > cb) {
      const dim3 cgrid((unsigned)(ce - cb), (unsigned)H);
      hipLaunchKernelGGL((bwd_ga_kernel<K, V, MT>), cgrid, dim3(NTGA), 0, st, dO,
                         (const float*)ckS, (const float*)ckX, (const float*)Dl,
                         (const float*)dDl, H, (const ChunkRow*)chunks, ntot, cb, scr);
      hipLaunchKernelGGL((bwd_gb_kernel<K, V, MT, GT>), cgrid, dim3(NTG), 0, st, k, v, g, beta,
                         (const float*)rec, (const float*)dDl, H, (const ChunkRow*)chunks, ntot,
                         cb, scr, a.grad_v, a.grad_beta);
      const dim3 pgrid(cgrid.x, cgrid.y, (unsigned)GScr<K>::KP);  // key-channel parts
      hipLaunchKernelGGL((bwd_gc_kernel<K, V, GT>), pgrid, dim3(NTG), 0, st, q, k, g, beta, H,
                         (const ChunkRow*)chunks, ntot, cb, scr, a.grad_q, a.grad_k, a.grad_g);
      hipLaunchKernelGGL((bwd_beta_kernel<K>), cgrid, dim3(BC), 0, st, H,
                         (const ChunkRow*)chunks, ntot, cb, (const float*)scr, a.grad_beta);
    }
  }
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdArgs& a, const BwdPlan& p) {
  hipStream_t st = (hipStream_t)a.stream;
  BwdArgs b = a;
  if (a.options != 0) {
    // the processed inputs first (fp32, in the workspace's leading region), the backward on
    // them, then the chain rule back to the raw inputs
    char* ws = reinterpret_cast<char*>(a.workspace);
    const OptBuffers ob{reinterpret_cast<float*>(ws + p.off_opt_q), reinterpret_cast<float*>(ws + p.off_opt_k),
                        reinterpret_cast<float*>(ws + p.off_opt_g), reinterpret_cast<float*>(ws + p.off_opt_b)};
    const OptInputs in{a.q, a.k, a.g, a.beta};
    launch_prologue(in, a.dtype_bf16, a.total_tokens, a.num_heads, a.dk, a.options, nullptr,
                    nullptr, 0, 0, ob, st, a.total_tokens);
    b.q = ob.q;
    b.k = ob.k;
    b.g = ob.g;
    b.beta = ob.beta;
    if (a.options & OPT_SCALAR_GATE) b.grad_g = reinterpret_cast<float*>(ws + p.off_opt_dg);
  }
  hipError_t e = hipErrorInvalidValue;
#define KDA_BWD_CASE(KK, VV)                                                                 \
  if (a.dk == KK && a.dv == VV)                                                              \
    e = a.options != 0 ? (a.dtype_bf16 ? launch_bwd_t<KK, VV, bf16, float>(b, p)              \
                                       : launch_bwd_t<KK, VV, float, float>(b, p))            \
                       : (a.dtype_bf16 ? launch_bwd_t<KK, VV, bf16, bf16>(b, p)               \
                                       : launch_bwd_t<KK, VV, float, float>(b, p));
  KDA_BWD_CASE(32, 32) KDA_BWD_CASE(32, 64) KDA_BWD_CASE(32, 128)
  KDA_BWD_CASE(64, 32) KDA_BWD_CASE(64, 64) KDA_BWD_CASE(64, 128)
  KDA_BWD_CASE(128, 32) KDA_BWD_CASE(128, 64) KDA_BWD_CASE(128, 128)
  KDA_BWD_CASE(32, 256) KDA_BWD_CASE(64, 256) KDA_BWD_CASE(128, 256)
#undef KDA_BWD_CASE
  if (e != hipSuccess || a.options == 0) return e;
  launch_bwd_epilogue(OptInputs{a.q, a.k, a.g, a.beta}, a.dtype_bf16, a.total_tokens,
                      a.num_heads, a.dk, a.options, a.grad_q, a.grad_k, b.grad_g, a.grad_g,
                      a.grad_beta, st);
  return hipGetLastError();
}

}  // namespace kda
