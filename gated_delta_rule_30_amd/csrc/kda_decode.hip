// Recurrent KDA decode step: one token per (sequence, head), fp32 state updated in place.
//
// Per head (state S: K x V fp32, row c = key channel):
//   S' = Diag(alpha) S                         (decay first; "A Technical Breakdown" 3.3)
//   u  = S'^T k                                (prediction of the decayed memory along k)
//   S  = S' + beta k (v - u)^T                 (erase along k and write v)
//   o  = S^T q = S'^T q + beta (k.q) (v - u)   (read after the write; explainer "Step 4")
// All four are fused into one pass: each workgroup streams its slice of the state from HBM
// once into registers, reduces u and S'^T q across the key channels, and writes the updated
// slice back once. The state is touched exactly once per step, so loads and
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

// A workgroup takes one (sequence, head) and a slice of VS value columns (the columns of S evolve
// independently, and u, S'^T q and k.q are sums over the key channels only). Thread (rg, cg)
// holds the 4 columns of column group cg in rows rg, rg + RG, rg + 2 RG, ... The partial sums
// meet in two steps: across the row groups of one wave by lane exchanges, then across the waves
// through LDS, so a thread adds one partial per wave, not one per row group.
// (VS, TPB) per shape were measured on MI355X with 512 MB of state per step: every shape then
// streams at 76-82% of the HBM peak. Two rows per thread and 512-1024 threads are best almost
// everywhere; a whole 128 x 128 head in one workgroup with 4 rows per thread ran 2% slower than
// two slices of 64 columns, and a 256 x 256 head in one workgroup (16 rows per thread) spilled.
constexpr int decode_vs(int K, int V) {
  return V == 32 ? 32 : V == 64 ? 64 : V == 128 ? (K == 128 ? 64 : K == 256 ? 32 : 128) : 128;
}
constexpr int decode_tpb(int K, int V) {
  return K == 32    ? (V == 32 ? 128 : V == 64 ? 256 : 512)
         : K == 64  ? (V == 32 ? 256 : V == 64 ? 512 : V == 128 ? 1024 : 512)
         : K == 128 ? (V == 32 ? 512 : 1024)
                    : 1024;
}

template <int K, int V>
struct DecodeShape {
  static constexpr int VS = decode_vs(K, V);   // value columns per workgroup
  static constexpr int NSL = V / VS;           // workgroups per head
  static constexpr int TPB = decode_tpb(K, V);
  static constexpr int CG = VS / 4;            // column groups of 4 value columns
  static constexpr int RG = TPB / CG;          // row groups
  static constexpr int RPT = K / RG;           // rows per thread
  static constexpr int RGW = CG < 64 ? 64 / CG : 1;  // row groups per wave
  static constexpr int NW = RG / RGW;          // partials per column group after the lane step
  static_assert(NSL * VS == V && RG * CG == TPB && RPT * RG == K && RPT >= 1 && NW >= 1,
                "decode shape");
};

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 x, int off) {
  return f32x4{__shfl_xor(x[0], off), __shfl_xor(x[1], off), __shfl_xor(x[2], off),
               __shfl_xor(x[3], off)};
}

// L2N: the unit-norm option (a compile-time case, so that the plain kernel carries none of it).
template <int K, int V, typename TI, bool L2N>
__global__ __launch_bounds__((DecodeShape<K, V>::TPB)) void decode_step_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const TI* __restrict__ g, const TI* __restrict__ beta, float* __restrict__ state,
    TI* __restrict__ o, uint32_t opts) {
  using DS = DecodeShape<K, V>;
  constexpr int CG = DS::CG;
  constexpr int RG = DS::RG;
  constexpr int RPT = DS::RPT;
  constexpr int RGW = DS::RGW;
  const int head = blockIdx.x / DS::NSL;
  const int col0 = (blockIdx.x % DS::NSL) * DS::VS;
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const TI* qh = q + (size_t)head * K;
  const TI* kh = k + (size_t)head * K;

  // unit-norm k and q: every wave sums the squares of the whole k and q (K <= 256 values),
  // and the sums that are linear in k or q are scaled afterwards. Their loads go out before
  // the state's, and the sums are formed while the state is in flight, so that the option adds
  // no step between the state's arrival and its store.
  constexpr int NKL = L2N ? (K + 63) / 64 : 1;
  float kn[NKL], qn[NKL];
  if constexpr (L2N) {
    const int lane = tid & 63;
#pragma unroll
    for (int j = 0; j < NKL; ++j) {
      const int c = min(lane + 64 * j, K - 1);  // lanes past K (K = 32) repeat an element
      kn[j] = to_f32(kh[c]);
      qn[j] = to_f32(qh[c]);
    }
  }

  // column group cg of this slice, row 0; row r is V / 4 vectors further
  f32x4* S = reinterpret_cast<f32x4*>(state + (size_t)head * K * V + col0) + cg;
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S[(rg + RG * i) * (V / 4)]);

  float nk = 1.f, nq = 1.f;
  if constexpr (L2N) {
    const int lane = tid & 63;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < NKL; ++j) {
      const bool in = lane + 64 * j < K;
      sk += in ? kn[j] * kn[j] : 0.f;
      sq += in ? qn[j] * qn[j] : 0.f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sk += __shfl_xor(sk, off);
      sq += __shfl_xor(sq, off);
    }
    nk = 1.f / sqrtf(sk + L2NORM_EPS);
    nq = 1.f / sqrtf(sq + L2NORM_EPS);
  }

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

  float b = to_f32(beta[head]);
  if (opts & OPT_BETA_LOGITS) b = sigmoid_f(b);

  // row groups of one wave are the lanes cg + CG j: add them up by lane exchanges
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
    pu += shfl_xor4(pu, off);
    pw += shfl_xor4(pw, off);
    pkq += __shfl_xor(pkq, off);
  }
  __shared__ f32x4 red_u[DS::NW][CG];
  __shared__ f32x4 red_w[DS::NW][CG];
  __shared__ float red_kq[DS::NW];
  if (rg % RGW == 0) {
    red_u[rg / RGW][cg] = pu;
    red_w[rg / RGW][cg] = pw;
    if (cg == 0) red_kq[rg / RGW] = pkq;
  }
  __syncthreads();

  f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int r = 0; r < DS::NW; ++r) {
    u += red_u[r][cg];
    w += red_w[r][cg];
    kq += red_kq[r];
  }
  u *= nk;
  w *= nq;
  kq *= nk * nq;
  const f32x4 vv = load4(v + (size_t)head * V + col0 + 4 * cg);
  const f32x4 d = b * (vv - u);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    f32x4 ns = a[i] * s[i] + (kk[i] * nk) * d;
    __builtin_nontemporal_store(ns, &S[(rg + RG * i) * (V / 4)]);
  }
  if (rg == 0) store4(o + (size_t)head * V + col0 + 4 * cg, w + kq * d);
}

template <int K, int V, typename TI>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int heads = a.num_seqs * a.num_heads;
  const dim3 grid(heads * DecodeShape<K, V>::NSL), block(DecodeShape<K, V>::TPB);
  if (a.options & OPT_L2NORM_QK)
    hipLaunchKernelGGL((decode_step_kernel<K, V, TI, true>), grid, block, 0, (hipStream_t)a.stream,
                       (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, (const TI*)a.g,
                       (const TI*)a.beta, a.state, (TI*)a.o, a.options);
  else
    hipLaunchKernelGGL((decode_step_kernel<K, V, TI, false>), grid, block, 0, (hipStream_t)a.stream,
                       (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, (const TI*)a.g,
                       (const TI*)a.beta, a.state, (TI*)a.o, a.options);
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
