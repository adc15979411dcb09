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
constexpr int NTGA = 1024;    // the S/X product kernel: 16 waves, two workgroups per CU

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

// Cumulative log2 decay: sB (64 x K, stride L) holds log alpha on entry, b * log2 e on exit.
// P = NTB / K neighbouring threads share a channel: each sums its 64 / P consecutive rows, the
// running totals of the P threads are scanned with shuffles, and each adds its prefix.
template <int K, int L, int NTB>
__device__ __forceinline__ void cumsum_log2(float* sB) {
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
  for (int r = 0; r < RP; ++r) sB[(part * RP + r) * L + c] = (x[r] + pre) * LOG2E;
}


// the token range of sequence n
__device__ __forceinline__ void seq_range(const int32_t* cu, int N, int64_t T, int n, int64_t* s0,
                                          int64_t* s1) {
  *s0 = cu ? (int64_t)cu[n] : (T / N) * n;
  *s1 = cu ? (int64_t)cu[n + 1] : (T / N) * (n + 1);
}

}  // namespace fp32
}  // namespace kda
