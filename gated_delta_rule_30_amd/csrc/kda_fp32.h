// fp32 chunk machinery shared by the training backward (kda_bwd.hip) and the wide-key forward
// (kda_wide.hip): thread counts, LDS loaders, the in-chunk cumulative decay and an LDS-operand
// fp32 matrix-core product. Everything here is device code with internal use only.
#pragma once

#include "kda_device.h"
#include "kda_paths.h"

namespace kda {
namespace fp32 {

constexpr int BC = CHUNK;  // 64 tokens per chunk
constexpr int NT = NTHREADS;  // the chains and the table kernels
constexpr int NTP = 512;      // the record kernel: 8 waves per workgroup
constexpr int NTG = 1024;     // the gradient kernels: 16 waves per workgroup
constexpr int NTGA = 512;     // the S/X product kernel: 8 waves, two workgroups per CU

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// fp32 16 x 16 x 4 matrix-core step: lane l = 16 g + m supplies A[m][g] and B[g][m]; the
// 16 x 16 result has lane (m, g) holding rows 4 g + r (r = 0..3) of column m.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum of x over the 16 lanes of a DPP row (lanes 16 q .. 16 q + 15), in every lane.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror 8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror 4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror 1
  return x;
}

// out(r, c, x) for x = sum_{k < R} A(r, k) B(k, c), r < 64, c < N, operands in LDS:
// A(r, k) = A[r][k] (row stride LA) or, with TA, A[k][r]; B(k, c) = B[k][c] (row stride LB)
// or, with TB, B[c][k]. The 4 N / 16 output tiles of 16 x 16 go round robin to the NTB / 64
// waves, each formed by R / 4 fp32 matrix-core steps. A wave's 64 operand reads fall in 64
// banks when an operand read along its rows (A, or B with TB) has a stride of 4 more than a
// multiple of 64 floats, and one read down its columns a stride of 16 more.
template <int N, int R, bool TA, bool TB, int LA, int LB, int NTB, typename F>
__device__ __forceinline__ void mmf(const float* sA, const float* sB, F&& out) {
  constexpr int TILES = 4 * (N / 16), WAVES = NTB / 64;
  const int wv = threadIdx.x >> 6, lm = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
  for (int t = wv; t < TILES; t += WAVES) {
    const int r0 = 16 * (t & 3), c0 = 16 * (t >> 2);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;  // two chains of dependent steps
#pragma unroll 8
    for (int k = 0; k < R; k += 8) {
      const float a0 = TA ? sA[(k + lg) * LA + r0 + lm] : sA[(r0 + lm) * LA + k + lg];
      const float b0 = TB ? sB[(c0 + lm) * LB + k + lg] : sB[(k + lg) * LB + c0 + lm];
      const float a1 = TA ? sA[(k + 4 + lg) * LA + r0 + lm] : sA[(r0 + lm) * LA + k + 4 + lg];
      const float b1 = TB ? sB[(c0 + lm) * LB + k + 4 + lg] : sB[(k + 4 + lg) * LB + c0 + lm];
      acc0 = mfma4(a0, b0, acc0);
      acc1 = mfma4(a1, b1, acc1);
    }
    const f32x4 acc = acc0 + acc1;
#pragma unroll
    for (int r = 0; r < 4; ++r) out(r0 + 4 * lg + r, c0 + lm, acc[r]);
  }
}

// mmf split over the reduction index: acc[i] += the partial product of the wave's i-th tile
// (tiles t = wave, wave + NTB / 64, ...; mmf_tiles<N, NTB>() per wave, the last ones skipped
// by waves past the tile count), and mmf_out hands the finished tiles to out(r, c, x).
template <int N, int NTB>
__host__ __device__ constexpr int mmf_tiles() {
  return (4 * (N / 16) + NTB / 64 - 1) / (NTB / 64);
}
template <int N, int R, bool TA, bool TB, int LA, int LB, int NTB>
__device__ __forceinline__ void mmf_acc(const float* sA, const float* sB, f32x4* acc) {
  constexpr int TILES = 4 * (N / 16), WAVES = NTB / 64;
  static_assert(R % 8 == 0, "reduction steps of 8");
  const int wv = threadIdx.x >> 6, lm = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int i = 0; i < mmf_tiles<N, NTB>(); ++i) {
    const int t = wv + WAVES * i;
    if (TILES % WAVES != 0 && t >= TILES) break;  // uniform per wave
    const int r0 = 16 * (t & 3), c0 = 16 * (t >> 2);
    f32x4 acc0 = acc[i], acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = 0; k < R; k += 8) {
      const float a0 = TA ? sA[(k + lg) * LA + r0 + lm] : sA[(r0 + lm) * LA + k + lg];
      const float b0 = TB ? sB[(c0 + lm) * LB + k + lg] : sB[(k + lg) * LB + c0 + lm];
      const float a1 = TA ? sA[(k + 4 + lg) * LA + r0 + lm] : sA[(r0 + lm) * LA + k + 4 + lg];
      const float b1 = TB ? sB[(c0 + lm) * LB + k + 4 + lg] : sB[(k + 4 + lg) * LB + c0 + lm];
      acc0 = mfma4(a0, b0, acc0);
      acc1 = mfma4(a1, b1, acc1);
    }
    acc[i] = acc0 + acc1;
  }
}
template <int N, int NTB, typename F>
__device__ __forceinline__ void mmf_out(const f32x4* acc, F&& out) {
  constexpr int TILES = 4 * (N / 16), WAVES = NTB / 64;
  const int wv = threadIdx.x >> 6, lm = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int i = 0; i < mmf_tiles<N, NTB>(); ++i) {
    const int t = wv + WAVES * i;
    if (TILES % WAVES != 0 && t >= TILES) break;  // uniform per wave
    const int r0 = 16 * (t & 3), c0 = 16 * (t >> 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) out(r0 + 4 * lg + r, c0 + lm, acc[i][r]);
  }
}

// The same products with each fp32 operand split into two bf16 parts, x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi), and each 16 x 16 x 32 step formed as hi*hi + hi*lo + lo*hi
// on the bf16 matrix cores (three bf16 steps where the fp32 form takes eight 16 x 16 x 4 steps).
// The dropped lo*lo term and the rounding of lo leave a relative error of at most about 3 * 2^-18
// per product (both parts of x keep fp32's exponent range); the sums stay in fp32.
// Operand fragment of a 32-step: lane (m, g) takes indices k + 4 g + e and k + 16 + 4 g + e
// (e = 0..3) of row (or column) idx. ROW: element (idx, k) at M[idx * L + k] (two 16-byte
// reads); otherwise at M[k * L + idx].
__device__ __forceinline__ void x3_split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
  hi = __builtin_convertvector(x, bf16x4);
  lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), bf16x4);
}
template <bool ROW, int L>
__device__ __forceinline__ void x3_frag(const float* M, int idx, int k, int g, bf16x8& hi, bf16x8& lo) {
  f32x4 x0, x1;
  if constexpr (ROW) {
    x0 = *reinterpret_cast<const f32x4*>(M + idx * L + k + 4 * g);
    x1 = *reinterpret_cast<const f32x4*>(M + idx * L + k + 16 + 4 * g);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = M[(k + 4 * g + e) * L + idx];
      x1[e] = M[(k + 16 + 4 * g + e) * L + idx];
    }
  }
  bf16x4 h0, h1, l0, l1;
  x3_split4(x0, h0, l0);
  x3_split4(x1, h1, l1);
  hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
  lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Register operands in the split form, for the state chains. An operand of a 16 x 16 x 16N
// step (N = 1 or 2) is held as N f32x4 pieces: piece i of lane (m, g) is reduction indices
// 16 i + 4 g .. + 3 (the fp32 16 x 16 x 4 steps' operands, four at a time). X3<N> is its split.
template <int N> struct X3;
template <> struct X3<1> { bf16x4 hi, lo; };
template <> struct X3<2> { bf16x8 hi, lo; };
__device__ __forceinline__ X3<1> x3_of(f32x4 x0) {
  X3<1> r;
  x3_split4(x0, r.hi, r.lo);
  return r;
}
__device__ __forceinline__ X3<2> x3_of(f32x4 x0, f32x4 x1) {
  bf16x4 h0, h1, l0, l1;
  x3_split4(x0, h0, l0);
  x3_split4(x1, h1, l1);
  return X3<2>{__builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7),
                __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7)};
}
template <int N>
__device__ __forceinline__ X3<N> x3_of(const f32x4* x) {
  if constexpr (N == 1) return x3_of(x[0]);
  else return x3_of(x[0], x[1]);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  typedef __attribute__((ext_vector_type(4))) short s4;
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// acc + A B in the split form; B_EXACT: B's low part is zero (bf16 data), one step fewer
template <bool B_EXACT = false, int N>
__device__ __forceinline__ f32x4 x3_mma(const X3<N>& a, const X3<N>& b, f32x4 acc) {
  acc = mma_bf16(a.lo, b.hi, acc);
  if constexpr (!B_EXACT) acc = mma_bf16(a.hi, b.lo, acc);
  return mma_bf16(a.hi, b.hi, acc);
}
// acc += the tile (r0, c0) of A B over k < R, by split-bf16 32-steps
template <int R, bool TA, bool TB, int LA, int LB>
__device__ __forceinline__ f32x4 x3_tile(const float* sA, const float* sB, int r0, int c0, f32x4 acc) {
  static_assert(R % 32 == 0, "reduction steps of 32");
  const int lm = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
#pragma unroll 1
  for (int k = 0; k < R; k += 32) {
    bf16x8 ah, al, bh, bl;
    x3_frag<!TA, LA>(sA, r0 + lm, k, lg, ah, al);
    x3_frag<TB, LB>(sB, c0 + lm, k, lg, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  }
  return acc;
}
// mmf and mmf_acc in the split-bf16 form (same arguments, tiles and output mapping)
template <int N, int R, bool TA, bool TB, int LA, int LB, int NTB, typename F>
__device__ __forceinline__ void mmx(const float* sA, const float* sB, F&& out) {
  constexpr int TILES = 4 * (N / 16), WAVES = NTB / 64;
  const int wv = threadIdx.x >> 6, lm = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
  for (int t = wv; t < TILES; t += WAVES) {
    const int r0 = 16 * (t & 3), c0 = 16 * (t >> 2);
    const f32x4 acc = x3_tile<R, TA, TB, LA, LB>(sA, sB, r0, c0, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) out(r0 + 4 * lg + r, c0 + lm, acc[r]);
  }
}
template <int N, int R, bool TA, bool TB, int LA, int LB, int NTB>
__device__ __forceinline__ void mmx_acc(const float* sA, const float* sB, f32x4* acc) {
  constexpr int TILES = 4 * (N / 16), WAVES = NTB / 64;
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < mmf_tiles<N, NTB>(); ++i) {
    const int t = wv + WAVES * i;
    if (TILES % WAVES != 0 && t >= TILES) break;  // uniform per wave
    acc[i] = x3_tile<R, TA, TB, LA, LB>(sA, sB, 16 * (t & 3), 16 * (t >> 2), acc[i]);
  }
}

// Four consecutive elements as fp32.
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  return __builtin_convertvector(*reinterpret_cast<const bf16x4*>(p), f32x4);
}

// Rows r < len of a [T][H][NTOT] tensor (token tok + r, head h), columns c0 .. c0 + N - 1, into
// LDS as fp32 (row stride L), zeros past len. Four elements per load, every load of the thread
// issued before the first store (rows past len read the last row, in bounds, and are dropped
// by a select).
template <int N, int L, int NTB, typename MT, int NTOT = N>
__device__ __forceinline__ void load_rows(float* dst, const MT* src, int64_t tok, int len, int H,
                                          int h, int c0 = 0) {
  constexpr int PIECES = BC * N / 4, PT = (PIECES + NTB - 1) / NTB;
  f32x4 t[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    if (PIECES % NTB == 0 || e < PIECES)
      t[u] = load4(src + ((tok + min(r, len - 1)) * H + h) * (int64_t)NTOT + c0 + c);
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    if (PIECES % NTB == 0 || e < PIECES) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(dst + r * L + c) = r < len ? t[u] : z;
    }
  }
}

// dst[r][c] = src[r][c0 + c] * 2^{dst[r][c]} for rows r < len of a [T][H][NTOT] tensor, 0 past
// len (e.g. k e^b from b log2 e); the loads are issued first, as in load_rows.
template <int N, int L, int NTB, typename MT, int NTOT = N>
__device__ __forceinline__ void mul_rows_exp2(float* dst, const MT* src, int64_t tok, int len,
                                              int H, int h, int c0 = 0) {
  constexpr int PIECES = BC * N / 4, PT = (PIECES + NTB - 1) / NTB;
  f32x4 t[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    if (PIECES % NTB == 0 || e < PIECES)
      t[u] = load4(src + ((tok + min(r, len - 1)) * H + h) * (int64_t)NTOT + c0 + c);
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    if (PIECES % NTB == 0 || e < PIECES) {
      f32x4* d = reinterpret_cast<f32x4*>(dst + r * L + c);
      const f32x4 b = *d;
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = r < len ? t[u][j] * exp2_f(b[j]) : 0.f;
      *d = x;
    }
  }
}

// ROWS x N fp32 block (row-major, stride SRCN) into LDS (row stride L), loads first.
template <int N, int L, int NTB, int ROWS = BC, int SRCN = N>
__device__ __forceinline__ void load_block(float* dst, const float* src) {
  constexpr int PIECES = ROWS * N / 4, PT = (PIECES + NTB - 1) / NTB;
  f32x4 t[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    if (PIECES % NTB == 0 || e < PIECES) t[u] = load4(src + (e / (N / 4)) * SRCN + 4 * (e % (N / 4)));
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    if (PIECES % NTB == 0 || e < PIECES)
      *reinterpret_cast<f32x4*>(dst + (e / (N / 4)) * L + 4 * (e % (N / 4))) = t[u];
  }
}

// Cumulative log2 decay: sB (64 x K, stride L) holds log alpha on entry, b * log2 e on exit
// (scale = 1: sB already holds log2 alpha).
// P = NTB / K neighbouring threads share a channel: each sums its 64 / P consecutive rows, the
// running totals of the P threads are scanned with shuffles, and each adds its prefix.
template <int K, int L, int NTB>
__device__ __forceinline__ void cumsum_log2(float* sB, float scale = LOG2E) {
  constexpr int P = NTB / K, RP = BC / P;
  static_assert(P >= 1 && P <= 32 && RP >= 1, "threads per channel");
  const int c = threadIdx.x / P, part = threadIdx.x % P;
  float x[RP];
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    run += sB[(part * RP + r) * L + c];
    x[r] = run;
  }
  float pre = run;
#pragma unroll
  for (int o = 1; o < P; o <<= 1) {
    const float y = __shfl_up(pre, o, P);
    if (part >= o) pre += y;
  }
  pre -= run;  // the rows before this thread's
#pragma unroll
  for (int r = 0; r < RP; ++r) sB[(part * RP + r) * L + c] = (x[r] + pre) * scale;
}


// A_ij = sum_c k_ic k_jc e^{b_ic - b_jc} (j < i) and P_ij = sum_c q_ic k_jc e^{b_ic - b_jc}
// (j <= i) of a 64-token chunk, summed over the key channels part by part, with NTB = 512
// threads. The six 16 x 16 blocks below the diagonal (I > J) run on the fp32 matrix cores, one
// block per wave (waves 0-5), with the decay split at the end of token block I - 1:
// e^{b_i - b_j} = e^{b_i - e} e^{e - b_j}, both factors at most 1 for log alpha <= 0 (rows of
// block I follow that token, rows of block J precede it). The 4 x 136 entries of the diagonal
// blocks are summed pairwise, e^{b_i - b_j} <= 1, one or two entries per thread.
struct PairAcc {
  f32x4 a, p;      // this wave's off-diagonal block: lane (m, g) holds rows 4g + r, column m
  float da[2], dp[2];  // this thread's diagonal entries
  int dI[2], di[2], dj[2];
};

// the off-diagonal block of wave w < 6: (I, J) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ __forceinline__ int pair_block_I(int w) { return w < 1 ? 1 : w < 3 ? 2 : 3; }
__device__ __forceinline__ int pair_block_J(int w) { return w < 1 ? 0 : w < 3 ? w - 1 : w - 3; }

template <int NTB>
__device__ __forceinline__ void pair_acc_init(PairAcc& acc) {
  static_assert(NTB == 512, "eight waves");
  acc.a = acc.p = f32x4{0.f, 0.f, 0.f, 0.f};
  // diagonal entry d in [0, 544): block d / 136, (i, j) the (d % 136)-th of j <= i < 16
  const int tid = threadIdx.x;
  const int d2 = (tid >= 384 && tid < 416) ? 512 + tid - 384 : -1;  // waves 6-7 take the rest
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int d = t == 0 ? tid : d2;
    acc.da[t] = acc.dp[t] = 0.f;
    acc.dI[t] = -1;
    if (d >= 0) {
      const int I = d / 136;
      int r = d % 136, i = 0;
      while (r > i) {
        r -= i + 1;
        ++i;
      }
      acc.dI[t] = I;
      acc.di[t] = 16 * I + i;
      acc.dj[t] = 16 * I + r;
    }
  }
}

// One part of KP channels: q in sQ ([64][LQ] fp32), k and b log2 e in sK, sB ([64][LK]); rows
// past the chunk hold q = k = 0 and b at its last value. WITH_P = false forms A alone (sQ is
// not read).
template <int KP, int LK, int LQ = LK, bool WITH_P = true>
__device__ __forceinline__ void pair_acc_part(PairAcc& acc, const float* sQ, const float* sK,
                                              const float* sB) {
  const int w = threadIdx.x >> 6, m = threadIdx.x & 15, g = (threadIdx.x >> 4) & 3;
  if (w < 6) {
    const int I = pair_block_I(w), J = pair_block_J(w);
    const float* rowI = sK + (16 * I + m) * LK;
    const float* rowQ = sQ + (16 * I + m) * LQ;
    const float* bI = sB + (16 * I + m) * LK;
    const float* bE = sB + (16 * I - 1) * LK;
    const float* rowJ = sK + (16 * J + m) * LK;
    const float* bJ = sB + (16 * J + m) * LK;
#pragma unroll 4
    for (int c = g; c < KP; c += 4) {
      const float e = bE[c];
      const float fi = exp2_f(bI[c] - e), fj = exp2_f(e - bJ[c]);
      const float kj = rowJ[c] * fj;
      acc.a = mfma4(rowI[c] * fi, kj, acc.a);
      if constexpr (WITH_P) acc.p = mfma4(rowQ[c] * fi, kj, acc.p);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (acc.dI[t] < 0) continue;
    const float* ki = sK + acc.di[t] * LK;
    const float* qi = sQ + acc.di[t] * LQ;
    const float* bi = sB + acc.di[t] * LK;
    const float* kj = sK + acc.dj[t] * LK;
    const float* bj = sB + acc.dj[t] * LK;
    float sa = 0.f, sp = 0.f;
#pragma unroll 2
    for (int c = 0; c < KP; c += 4) {
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(ki + c);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(bi + c), k2 = *reinterpret_cast<const f32x4*>(kj + c);
      const f32x4 b2 = *reinterpret_cast<const f32x4*>(bj + c);
      f32x4 x;
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = k2[u] * exp2_f(b1[u] - b2[u]);
      sa += dot4(k1, x);
      if constexpr (WITH_P) sp += dot4(*reinterpret_cast<const f32x4*>(qi + c), x);
    }
    acc.da[t] += sa;
    acc.dp[t] += sp;
  }
}

// The sums out: outA(i, j, x) for every j < i and outP(i, j, x) for every j <= i (each entry
// once; entries above the diagonal are not visited).
template <typename FA, typename FP>
__device__ __forceinline__ void pair_acc_out(const PairAcc& acc, FA&& outA, FP&& outP) {
  const int w = threadIdx.x >> 6, m = threadIdx.x & 15, g = (threadIdx.x >> 4) & 3;
  if (w < 6) {
    const int I = pair_block_I(w), J = pair_block_J(w);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      outA(16 * I + 4 * g + r, 16 * J + m, acc.a[r]);
      outP(16 * I + 4 * g + r, 16 * J + m, acc.p[r]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (acc.dI[t] < 0) continue;
    if (acc.dj[t] < acc.di[t]) outA(acc.di[t], acc.dj[t], acc.da[t]);
    outP(acc.di[t], acc.dj[t], acc.dp[t]);
  }
}

// T = (I + A)^{-1} in place for the strictly lower 64 x 64 A in sA (row stride 68; on return
// zero above the diagonal), with NTB = 512 threads: the four diagonal 16 x 16 blocks by forward
// substitution (waves 0-3, one column per lane of the first 16), then the blocks below by
// distance d = I - J, one block per wave, on the fp32 matrix cores:
// T_IJ = -T_II (sum_{M=J}^{I-1} A_IM T_MJ). Until the end T_IJ (I > J) sits in the unused upper
// block (J, I), so that T_MJ (M >= J) is always at rows 16J.., columns 16M.. and the A blocks
// below stay intact; a last pass moves them down. LDS-only barriers between the steps.
template <int NTB>
__device__ __forceinline__ void unit_lower_inverse_blocked(float* sA) {
  static_assert(NTB == 512, "eight waves");
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  if (w < 4 && lane < 16) {  // the wave's lanes run in step: every read of A_ww precedes the writes
    float* a = sA + (16 * w) * 68 + 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float ps = r == lane ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) ps -= a[r * 68 + j] * x[j];
      x[r] = ps;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r * 68 + lane] = x[r];
  }
  lds_barrier();
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int J = w, I = w + d;
      float* tij = sA + (16 * J) * 68 + 16 * I;  // T_IJ's slot: the upper block (J, I)
      // X = sum_M A_IM T_MJ: lane (m, g) ends with rows 4g + r of column m
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          X = mfma4(sA[(16 * I + m) * 68 + 16 * M + 4 * s + g],
                    sA[(16 * J + 4 * s + g) * 68 + 16 * M + m], X);
      }
      // X through the slot (the wave's LDS accesses take effect in order), then T_IJ = -T_II X
#pragma unroll
      for (int r = 0; r < 4; ++r) tij[(4 * g + r) * 68 + m] = X[r];
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        Y = mfma4(sA[(16 * I + m) * 68 + 16 * I + 4 * s + g], tij[(4 * s + g) * 68 + m], Y);
#pragma unroll
      for (int r = 0; r < 4; ++r) tij[(4 * g + r) * 68 + m] = -Y[r];
    }
    lds_barrier();
  }
  // T_IJ down to its place, zeros above the diagonal (each element moved by one thread)
  for (int e = tid; e < BC * BC; e += NTB) {
    const int r = e / BC, c = e % BC;
    if ((c >> 4) > (r >> 4)) {
      const int J = r >> 4, I = c >> 4;
      sA[(16 * I + (r & 15)) * 68 + 16 * J + (c & 15)] = sA[r * 68 + c];
      sA[r * 68 + c] = 0.f;
    }
  }
  lds_barrier();
}

// the token range of sequence n
__device__ __forceinline__ void seq_range(const int32_t* cu, int N, int64_t T, int n, int64_t* s0,
                                          int64_t* s1) {
  *s0 = cu ? (int64_t)cu[n] : (T / N) * n;
  *s1 = cu ? (int64_t)cu[n + 1] : (T / N) * (n + 1);
}

}  // namespace fp32
}  // namespace kda
