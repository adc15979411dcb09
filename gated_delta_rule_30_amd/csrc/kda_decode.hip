// Recurrent KDA decode step: one token per (sequence, head), fp32 state updated in place.
//
// Per head (state S: K x V fp32, row c = key channel):
//   S' = Diag(alpha) S                         (decay first; "A Technical Breakdown" 3.3)
//   u  = S'^T k                                (prediction of the decayed memory along k)
//   S  = S' + beta k (v - u)^T                 (erase along k and write v)
//   o  = S^T q = S'^T q + beta (k.q) (v - u)   (read after the write; explainer "Step 4")
// All four are fused into one pass: each workgroup streams its 64 KB state (K=V=128) from
// HBM once into registers, reduces u and S'^T q across row groups through LDS, and writes
// the updated state back once. The state is touched exactly once per step, so loads and
// stores are non-temporal. The kernel is HBM-bound: 2*K*V*4 bytes of state traffic per head.
// Input options: a scalar gate per head, alpha = sigmoid(z) from gate logits, beta from
// logits, and unit-norm q and k. Since u, S'^T q and k.q are linear in k and q, the sums are
// formed from the raw k and q and scaled by the inverse norms afterwards.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename TI>
__device__ __forceinline__ f32x4 load4(const TI* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

template <typename TI>
__device__ __forceinline__ void store4(TI* p, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, f32x4 x) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// Threads per head: up to 1024, one per 16-byte state vector (K*V/4) where that is fewer. With
// K=V=128 each thread holds four vectors of one column group; measured on MI355X the whole
// 8192-head step streams at about 6.1 TB/s with 1024 threads, 5.7 with 512 and 5.6 with 256 (the
// barrier between the loads and the stores idles a smaller workgroup's share of the CU).
template <int K, int V>
struct DecodeShape {
  static constexpr int TPB = K * V / 4 < 1024 ? K * V / 4 : 1024;
  static constexpr int CG = V / 4;      // column groups of 4 value columns
  static constexpr int RG = TPB / CG;   // row groups
  static constexpr int RPT = K / RG;    // rows per thread
  static_assert(RPT >= 1 && RG * CG == TPB, "decode shape");
};

// Column group cg holds 4 value columns; row group rg holds rows rg, rg + RG, rg + 2 RG, ...
template <int K, int V, typename TI>
__global__ __launch_bounds__((DecodeShape<K, V>::TPB)) void decode_step_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const TI* __restrict__ g, const TI* __restrict__ beta, float* __restrict__ state,
    TI* __restrict__ o, uint32_t opts) {
  using DS = DecodeShape<K, V>;
  constexpr int CG = DS::CG;
  constexpr int RG = DS::RG;
  constexpr int RPT = DS::RPT;
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;

  f32x4* S = reinterpret_cast<f32x4*>(state + (size_t)head * K * V);
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S[(rg + RG * i) * CG + cg]);

  const TI* qh = q + (size_t)head * K;
  const TI* kh = k + (size_t)head * K;
  const bool scalar_gate = (opts & OPT_SCALAR_GATE) != 0;
  const bool gate_logits = (opts & OPT_GATE_LOGITS) != 0;
  const TI* gh = g + (size_t)head * (scalar_gate ? 1 : K);
  float a[RPT], kk[RPT];
  f32x4 pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
  float pkq = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float z = to_f32(gh[scalar_gate ? 0 : r]);
    a[i] = gate_logits ? sigmoid_f(z) : exp_f(z);
    kk[i] = to_f32(kh[r]);
    const float qq = to_f32(qh[r]);
    pu += (a[i] * kk[i]) * s[i];
    pw += (a[i] * qq) * s[i];
    pkq += kk[i] * qq;
  }

  // unit-norm k and q: every wave sums the squares of the whole k and q (K <= 256 values),
  // and the sums that are linear in k or q are scaled afterwards
  float nk = 1.f, nq = 1.f;
  if (opts & OPT_L2NORM_QK) {
    const int lane = tid & 63;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int c = lane; c < K; c += 64) {
      const float x = to_f32(kh[c]), y = to_f32(qh[c]);
      sk += x * x;
      sq += y * y;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sk += __shfl_xor(sk, off);
      sq += __shfl_xor(sq, off);
    }
    nk = 1.f / sqrtf(sk + L2NORM_EPS);
    nq = 1.f / sqrtf(sq + L2NORM_EPS);
  }
  float b = to_f32(beta[head]);
  if (opts & OPT_BETA_LOGITS) b = sigmoid_f(b);

  __shared__ f32x4 red_u[RG][CG];
  __shared__ f32x4 red_w[RG][CG];
  __shared__ float red_kq[RG];
  red_u[rg][cg] = pu;
  red_w[rg][cg] = pw;
  if (cg == 0) red_kq[rg] = pkq;
  __syncthreads();

  f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    u += red_u[r][cg];
    w += red_w[r][cg];
    kq += red_kq[r];
  }
  u *= nk;
  w *= nq;
  kq *= nk * nq;
  const f32x4 vv = load4(v + (size_t)head * V + 4 * cg);
  const f32x4 d = b * (vv - u);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    f32x4 ns = a[i] * s[i] + (kk[i] * nk) * d;
    __builtin_nontemporal_store(ns, &S[(rg + RG * i) * CG + cg]);
  }
  if (rg == 0) store4(o + (size_t)head * V + 4 * cg, w + kq * d);
}

template <int K, int V, typename TI>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int heads = a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((decode_step_kernel<K, V, TI>), dim3(heads), dim3(DecodeShape<K, V>::TPB), 0,
                     (hipStream_t)a.stream, (const TI*)a.q, (const TI*)a.k, (const TI*)a.v,
                     (const TI*)a.g, (const TI*)a.beta, a.state, (TI*)a.o, a.options);
  return hipGetLastError();
}

template <typename TI>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
#define KDA_DEC_CASE(KK, VV) \
  if (a.dk == KK && a.dv == VV) return launch_decode_t<KK, VV, TI>(a);
  KDA_DEC_CASE(32, 32) KDA_DEC_CASE(32, 64) KDA_DEC_CASE(32, 128) KDA_DEC_CASE(32, 256)
  KDA_DEC_CASE(64, 32) KDA_DEC_CASE(64, 64) KDA_DEC_CASE(64, 128) KDA_DEC_CASE(64, 256)
  KDA_DEC_CASE(128, 32) KDA_DEC_CASE(128, 64) KDA_DEC_CASE(128, 128) KDA_DEC_CASE(128, 256)
  KDA_DEC_CASE(256, 32) KDA_DEC_CASE(256, 64) KDA_DEC_CASE(256, 128) KDA_DEC_CASE(256, 256)
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.dtype_bf16) return launch_decode_dt<bf16>(a);
  return launch_decode_dt<float>(a);
}

}  // namespace kda
