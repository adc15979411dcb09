// The input options (KDA_OPT_*) as a pass of their own, for the paths whose kernels read the
// plain inputs: the training backward and the wide-key forward. prologue_kernel writes the
// processed q, k, log alpha and beta in fp32 (the "Kimi Linear" explainer, "Step 2: Per-Channel
// Decay": alpha = sigmoid(z); "A Technical Breakdown", section 3.2: one gate per head; unit-norm
// q and k; beta = sigmoid(x)), and bwd_epilogue_kernel carries the backward's gradients with
// respect to those back to the raw inputs (the chain rule through each option).
//
// One wave per (token, head) row, lane l holding key channels l, l + 64, ...; the row's sums
// (the L2 norms, q^T dq, the scalar gate's sum over channels) are shuffle trees in a fixed
// order, so results are the same on every run.
#include "kda_device.h"
#include "kda_paths.h"

namespace kda {

namespace {

constexpr int PRO_THREADS = 256;  // four rows per workgroup
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace

// Rows (t, h) of the tokens [t0, t1): with `chunks`, t0 and t1 are the first token of chunk cb
// and the end of chunk min(ce, ntot) - 1 and row (t, h) lands at position t - t0 of the outputs;
// without, every token of the call at its own position.
template <typename MT, int KMAX>
__global__ __launch_bounds__(PRO_THREADS) void prologue_kernel(
    const MT* __restrict__ q, const MT* __restrict__ k, const MT* __restrict__ g,
    const MT* __restrict__ beta, int64_t T, int H, int K, uint32_t options,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, int cb, int ce,
    float* __restrict__ q2, float* __restrict__ k2, float* __restrict__ g2,
    float* __restrict__ b2) {
  constexpr int PL = KMAX / 64 > 0 ? KMAX / 64 : 1;  // channels per lane
  int64_t t0 = 0, t1 = T;
  if (chunks != nullptr) {
    const int last = min(ce, *ntot) - 1;
    if (last < cb) return;
    t0 = chunks[cb].tok;
    t1 = (int64_t)chunks[last].tok + chunks[last].len;
  }
  const int lane = threadIdx.x & 63;
  const int64_t rows = (t1 - t0) * H;
  const int64_t wstride = (int64_t)gridDim.x * (PRO_THREADS / 64);
  const bool l2 = (options & OPT_L2NORM_QK) != 0, logits = (options & OPT_GATE_LOGITS) != 0;
  const bool scalar = (options & OPT_SCALAR_GATE) != 0;
  for (int64_t r = (int64_t)blockIdx.x * (PRO_THREADS / 64) + (threadIdx.x >> 6); r < rows;
       r += wstride) {
    const int64_t src = t0 * H + r;  // row (t, h) of the inputs; r is its row in the outputs
    float qv[PL], kv[PL], gv[PL];
    float sq = 0.f, sk = 0.f;
    const float zs = scalar ? to_f32(g[src]) : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int c = lane + 64 * i;
      const bool on = c < K;
      qv[i] = on ? to_f32(q[src * K + c]) : 0.f;
      kv[i] = on ? to_f32(k[src * K + c]) : 0.f;
      const float z = scalar ? zs : on ? to_f32(g[src * K + c]) : 0.f;
      gv[i] = logits ? log2_sigmoid(z) * LN2 : z;
      sq += qv[i] * qv[i];
      sk += kv[i] * kv[i];
    }
    float nq = 1.f, nk = 1.f;
    if (l2) {
      nq = 1.f / sqrtf(wave_sum(sq) + L2NORM_EPS);
      nk = 1.f / sqrtf(wave_sum(sk) + L2NORM_EPS);
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int c = lane + 64 * i;
      if (c < K) {
        q2[r * K + c] = qv[i] * nq;
        k2[r * K + c] = kv[i] * nk;
        g2[r * K + c] = gv[i];
      }
    }
    if (lane == 0) {
      const float b = to_f32(beta[src]);
      b2[r] = (options & OPT_BETA_LOGITS) ? sigmoid_f(b) : b;
    }
  }
}

// The backward's gradients with respect to the processed inputs (grad_q, grad_k in place,
// dg [rows][K] and grad_beta in place) become those with respect to the raw inputs:
//   unit norm y = x r, r = (|x|^2 + eps)^{-1/2}:  dx = r dy - r^3 x (x^T dy)
//   log alpha = log sigmoid(z):                   dz = d(log alpha) sigmoid(-z)
//   one gate per head:                            dz = sum over the channels (then as above)
//   beta = sigmoid(x):                            dx = dbeta sigmoid(x) sigmoid(-x)
// grad_g is [rows][K], or [rows] with the scalar gate (then dg is a separate buffer; otherwise
// dg may be grad_g itself).
template <typename MT, int KMAX>
__global__ __launch_bounds__(PRO_THREADS) void bwd_epilogue_kernel(
    const MT* __restrict__ q, const MT* __restrict__ k, const MT* __restrict__ g,
    const MT* __restrict__ beta, int64_t rows, int K, uint32_t options, float* grad_q,
    float* grad_k, const float* dg, float* grad_g, float* grad_beta) {
  constexpr int PL = KMAX / 64 > 0 ? KMAX / 64 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * (PRO_THREADS / 64);
  const bool l2 = (options & OPT_L2NORM_QK) != 0, logits = (options & OPT_GATE_LOGITS) != 0;
  const bool scalar = (options & OPT_SCALAR_GATE) != 0;
  for (int64_t r = (int64_t)blockIdx.x * (PRO_THREADS / 64) + (threadIdx.x >> 6); r < rows;
       r += wstride) {
    if (l2) {
      float xq[PL], dq[PL], xk[PL], dk[PL];
      float sq = 0.f, sk = 0.f, pq = 0.f, pk = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        const bool on = c < K;
        xq[i] = on ? to_f32(q[r * K + c]) : 0.f;
        xk[i] = on ? to_f32(k[r * K + c]) : 0.f;
        dq[i] = on ? grad_q[r * K + c] : 0.f;
        dk[i] = on ? grad_k[r * K + c] : 0.f;
        sq += xq[i] * xq[i];
        sk += xk[i] * xk[i];
        pq += xq[i] * dq[i];
        pk += xk[i] * dk[i];
      }
      const float rq = 1.f / sqrtf(wave_sum(sq) + L2NORM_EPS);
      const float rk = 1.f / sqrtf(wave_sum(sk) + L2NORM_EPS);
      const float cq = rq * rq * rq * wave_sum(pq), ck = rk * rk * rk * wave_sum(pk);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < K) {
          grad_q[r * K + c] = rq * dq[i] - cq * xq[i];
          grad_k[r * K + c] = rk * dk[i] - ck * xk[i];
        }
      }
    }
    if (scalar) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < K) s += dg[r * K + c];
      }
      s = wave_sum(s);
      if (lane == 0) grad_g[r] = logits ? s * sigmoid_f(-to_f32(g[r])) : s;
    } else if (logits) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < K) grad_g[r * K + c] = dg[r * K + c] * sigmoid_f(-to_f32(g[r * K + c]));
      }
    }
    if ((options & OPT_BETA_LOGITS) && lane == 0) {
      const float x = to_f32(beta[r]);
      grad_beta[r] *= sigmoid_f(x) * sigmoid_f(-x);
    }
  }
}

// ---------------------------------------------------------------- host
static unsigned pro_grid(int64_t rows) {
  const int64_t wgs = (rows + PRO_THREADS / 64 - 1) / (PRO_THREADS / 64);
  return (unsigned)(wgs < 4096 ? (wgs > 0 ? wgs : 1) : 4096);
}

template <typename MT>
static void launch_prologue_t(const OptInputs& in, int64_t T, int H, int K, uint32_t options,
                              const ChunkRow* chunks, const int32_t* ntot, int cb, int ce,
                              const OptBuffers& out, hipStream_t st, int64_t max_rows) {
  const MT *q = (const MT*)in.q, *k = (const MT*)in.k, *g = (const MT*)in.g, *b = (const MT*)in.beta;
  const dim3 grid(pro_grid(max_rows * H)), block(PRO_THREADS);
  if (K <= 64)
    hipLaunchKernelGGL((prologue_kernel<MT, 64>), grid, block, 0, st, q, k, g, b, T, H, K, options,
                       chunks, ntot, cb, ce, out.q, out.k, out.g, out.beta);
  else if (K <= 128)
    hipLaunchKernelGGL((prologue_kernel<MT, 128>), grid, block, 0, st, q, k, g, b, T, H, K, options,
                       chunks, ntot, cb, ce, out.q, out.k, out.g, out.beta);
  else
    hipLaunchKernelGGL((prologue_kernel<MT, 256>), grid, block, 0, st, q, k, g, b, T, H, K, options,
                       chunks, ntot, cb, ce, out.q, out.k, out.g, out.beta);
}

void launch_prologue(const OptInputs& in, bool bf16, int64_t T, int H, int K, uint32_t options,
                     const ChunkRow* chunks, const int32_t* ntot, int cb, int ce,
                     const OptBuffers& out, hipStream_t st, int64_t max_rows) {
  if (bf16)
    launch_prologue_t<kda::bf16>(in, T, H, K, options, chunks, ntot, cb, ce, out, st, max_rows);
  else
    launch_prologue_t<float>(in, T, H, K, options, chunks, ntot, cb, ce, out, st, max_rows);
}

template <typename MT>
static void launch_epilogue_t(const OptInputs& in, int64_t T, int H, int K, uint32_t options,
                              float* grad_q, float* grad_k, const float* dg, float* grad_g,
                              float* grad_beta, hipStream_t st) {
  const MT *q = (const MT*)in.q, *k = (const MT*)in.k, *g = (const MT*)in.g, *b = (const MT*)in.beta;
  const int64_t rows = T * H;
  const dim3 grid(pro_grid(rows)), block(PRO_THREADS);
  if (K <= 64)
    hipLaunchKernelGGL((bwd_epilogue_kernel<MT, 64>), grid, block, 0, st, q, k, g, b, rows, K,
                       options, grad_q, grad_k, dg, grad_g, grad_beta);
  else
    hipLaunchKernelGGL((bwd_epilogue_kernel<MT, 128>), grid, block, 0, st, q, k, g, b, rows, K,
                       options, grad_q, grad_k, dg, grad_g, grad_beta);
}

void launch_bwd_epilogue(const OptInputs& in, bool bf16, int64_t T, int H, int K,
                         uint32_t options, float* grad_q, float* grad_k, const float* dg,
                         float* grad_g, float* grad_beta, hipStream_t st) {
  if (T == 0) return;
  if (bf16)
    launch_epilogue_t<kda::bf16>(in, T, H, K, options, grad_q, grad_k, dg, grad_g, grad_beta, st);
  else
    launch_epilogue_t<float>(in, T, H, K, options, grad_q, grad_k, dg, grad_g, grad_beta, st);
}

}  // namespace kda
