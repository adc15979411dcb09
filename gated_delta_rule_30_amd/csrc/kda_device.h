// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

// Compile-time loop: f(std::integral_constant<int, I>()) for I = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned v2u32;
typedef __attribute__((ext_vector_type(4))) unsigned v4u32;

// ------------------------------------------------------------------ scalar conversions
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// e^x through the hardware base-2 exponential; exp2_f takes the exponent in log2 units.
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;

// Input prologue (the option bits of the C ABI). log2(sigmoid(z)) = -log2(1 + 2^{-z log2 e}),
// evaluated as min(z, 0) log2 e - log2(1 + 2^{-|z| log2 e}) so that nothing overflows for any
// finite z; v_log_f32 is the hardware base-2 logarithm.
__device__ __forceinline__ float log2_sigmoid(float z) {
  return fminf(z, 0.f) * LOG2E - __builtin_amdgcn_logf(1.f + exp2_f(-fabsf(z) * LOG2E));
}
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + exp2_f(-x * LOG2E));  // 1 / inf = 0 for very negative x
}

// ------------------------------------------------------------------ MFMA 16x16 tiles
// A "fragment" is what one lane feeds to one 16x16xKS reduction step: 16 bytes.
// Lane l has row/column index m = l % 16 and group g = l / 16.
// Within a reduction step of KS elements, element e of group g covers the index
//     kk(g, e) = 16 * (e / 4) + 4 * g + (e % 4)
// (bf16: KS = 32, 8 elements per lane; fp32: KS = 16, 4 elements per lane).
// A-operand fragments and B-operand fragments use the same kk mapping, so the products pair
// up whatever order the hardware sums in. The 16x16 fp32 result tile has lane l holding
// rows 4 * g + r (r = 0..3) of column m. With this kk mapping a 16-row result tile (two
// tiles for bf16) is directly a fragment along its row index.
template <typename MT> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 32;
  static constexpr int EPL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 16;
  static constexpr int EPL = 4;
  typedef f32x4 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

// Fragment of reduction step s for group g from a row whose reduction index is contiguous.
__device__ __forceinline__ bf16x8 load_frag(const bf16* row, int s, int g) {
  const bf16* p = row + 32 * s + 4 * g;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 load_frag(const float* row, int s, int g) {
  return *reinterpret_cast<const f32x4*>(row + 16 * s + 4 * g);
}

// Same, from an fp32 row scaled elementwise by an fp32 vector, rounded to MT.
__device__ __forceinline__ bf16x8 load_frag_scaled(const float* row, const float* scale, int s,
                                                   int g, bf16) {
  const int o = 32 * s + 4 * g;
  f32x4 a = *reinterpret_cast<const f32x4*>(row + o);
  f32x4 b = *reinterpret_cast<const f32x4*>(row + o + 16);
  f32x4 sa = *reinterpret_cast<const f32x4*>(scale + o);
  f32x4 sb = *reinterpret_cast<const f32x4*>(scale + o + 16);
  a *= sa;
  b *= sb;
  return __builtin_shufflevector(__builtin_convertvector(a, bf16x4), __builtin_convertvector(b, bf16x4),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 load_frag_scaled(const float* row, const float* scale, int s,
                                                  int g, float) {
  const int o = 16 * s + 4 * g;
  return *reinterpret_cast<const f32x4*>(row + o) * *reinterpret_cast<const f32x4*>(scale + o);
}

// Fragment made of two fp32 result tiles (rows 0-15 and 16-31 of a reduction step): bf16.
__device__ __forceinline__ bf16x8 frag_from_acc(f32x4 lo, f32x4 hi, bf16) {
  return __builtin_shufflevector(__builtin_convertvector(lo, bf16x4), __builtin_convertvector(hi, bf16x4),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// A fragment (reduction step s) of X^T for the 16 rows c0 .. c0+15 of X^T, where X is stored
// row-major with ld elements per row and rows = reduction index: lane (m, g) receives
// X[KS*s + kk(g, e)][c0 + m]. ds_read_b64_tr_b16 works per group of 16 lanes: lane 4p + r of
// the group receives element r of the 8 bytes addressed by lanes 4e + p (e = 0..3). So lane
// (m, g) supplies the address of row 4g + m/4, columns c0 + 4(m%4) .. +3, and receives rows
// 4g .. 4g+3 of column c0 + m.
__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  const v4bf v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) v4bf*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 frag_t(const bf16* X, int ld, int c0, int s, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const bf16* p = X + (32 * s + 4 * g + (m >> 2)) * ld + c0 + 4 * (m & 3);
  const bf16x4 lo = ds_read_tr4(p);
  const bf16x4 hi = ds_read_tr4(p + 16 * ld);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 frag_t(const float* X, int ld, int c0, int s, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const float* p = X + (16 * s + 4 * g) * ld + c0 + m;
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// Workgroup barrier that orders LDS accesses only: the fences are workgroup-scope and limited
// to the local address space, so the wait before s_barrier covers this wave's LDS operations
// but not its outstanding global loads and stores, which stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

}  // namespace kda
