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
#include "kda_record.h"

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

constexpr int LKQ = KQ + 4;  // LDS row of a channel part

}  // namespace

// The chunks [cb, ...) of one segment, records indexed from cb. MT: v; GT: q, k, log alpha and
// beta, at the call's token positions, or (local) from the first token of chunk cb on (the
// fp32 output of the input-option pass over the segment's tokens).
template <int KW, int V, typename MT, typename GT>
__global__ __launch_bounds__(NTP, 4) void wide_prep_kernel(
    const GT* __restrict__ q, const GT* __restrict__ k, const MT* __restrict__ v,
    const GT* __restrict__ g, const GT* __restrict__ beta, int H,
    const ChunkRow* __restrict__ chunks, const int32_t* __restrict__ ntot, int cb, bool local,
    float* __restrict__ rec) {
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
  const int lc = blockIdx.x, c = cb + lc, h = blockIdx.y;  // chunk of the segment, of the call
  if (c >= *ntot) return;
  const ChunkRow ch = chunks[c];
  const int64_t gtok = local ? (int64_t)ch.tok - chunks[cb].tok : ch.tok;  // q, k, g, beta row
  float* rc = rec + ((size_t)lc * H + h) * R::floats;
  if (threadIdx.x < BC)
    sBeta[threadIdx.x] = threadIdx.x < ch.len ? to_f32(beta[(gtok + threadIdx.x) * (int64_t)H + h]) : 0.f;
  // A and P, summed over the four quarters (off-diagonal 16 x 16 blocks on the matrix cores)
  PairAcc acc;
  pair_acc_init<NTP>(acc);
  for (int hh = 0; hh < KW / KQ; ++hh) {
    const int c0 = hh * KQ;
    load_rows<KQ, LK, NTP, GT, KW>(sQ, q, gtok, ch.len, H, h, c0);
    load_rows<KQ, LK, NTP, GT, KW>(sK, k, gtok, ch.len, H, h, c0);
    load_rows<KQ, LK, NTP, GT, KW>(sB, g, gtok, ch.len, H, h, c0);
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
    pair_acc_part<KQ, LK>(acc, sQ, sK, sB);
    lds_barrier();  // the quarter's reads done before the next quarter overwrites it
  }
  // (the solve reads A below the diagonal only)
  pair_acc_out(acc, [&](int i, int j, float x) { sA[i * 68 + j] = sBeta[i] * x; },
               [&](int i, int j, float x) { rc[R::oP + i * BC + j] = x; });
  for (int e = threadIdx.x; e < BC * BC; e += NTP)  // P's upper triangle
    if (e % BC > e / BC) rc[R::oP + e] = 0.f;
  lds_barrier();
  unit_lower_inverse_blocked<NTP>(sA);  // T = (I + A)^{-1} into sT (= sA)
  // W = T diag(beta) (k e^b), quarter by quarter
  for (int hh = 0; hh < KW / KQ; ++hh) {
    const int c0 = hh * KQ;
    load_rows<KQ, LK, NTP, GT, KW>(sB, g, gtok, ch.len, H, h, c0);
    lds_barrier();
    cumsum_log2<KQ, LK, NTP>(sB);
    lds_barrier();
    mul_rows_exp2<KQ, LK, NTP, GT, KW>(sB, k, gtok, ch.len, H, h, c0);
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

// Records of the chunk path at 256 key channels (bf16 inputs): the same chunk form as
// wide_prep_kernel, in fp32 with the key channels in parts of 64, written as the bf16 MFMA
// fragment records that prep_kernel writes for K <= 128 -- -W, Qe, Ktilde^T, T' =
// T diag(beta), P, gamma and V slice-major -- so that state_split_kernel runs the chain on the
// bf16 matrix cores. One workgroup of 512 threads per (chunk, head) of the segment: task j is
// entry seg_begin + j of the chunk table. Each thread writes one 16-byte fragment slot of a
// 4 x 2 block of slots (token or channel tile ft, reduction step fsl) per matrix part.
// OPTS = true applies the input options to the raw inputs as they are read, in fp32, as
// prep_kernel does at K <= 128: q and k scaled by their inverse L2 norms over the 256 channels
// (formed in a pass before the parts), log2 alpha = log2 sigmoid(z) for gate logits (one value
// per token with the scalar gate), beta = sigmoid(x) for beta logits.

// The part's log2 alpha (c0 .. c0 + N - 1 of a [T][H][NTOT] tensor, or of [T][H] for the
// scalar gate) into dst, zero past len; the same thread-to-element map as load_rows.
template <int N, int L, int NTB, int NTOT>
__device__ __forceinline__ void gate_rows_opts(float* dst, const bf16* g, int64_t tok, int len,
                                               int H, int h, int c0, uint32_t opts) {
  constexpr int PIECES = BC * N / 4, PT = PIECES / NTB;
  static_assert(PIECES % NTB == 0, "whole pieces per thread");
  const bool scalar = (opts & OPT_SCALAR_GATE) != 0, logits = (opts & OPT_GATE_LOGITS) != 0;
  f32x4 t[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    const int64_t row = (tok + min(r, len - 1)) * H + h;
    if (scalar) {
      const float z = to_f32(g[row]);
      t[u] = f32x4{z, z, z, z};
    } else {
      t[u] = load4(g + row * (int64_t)NTOT + c0 + c);
    }
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = r < len ? (logits ? log2_sigmoid(t[u][j]) : t[u][j] * LOG2E) : 0.f;
    *reinterpret_cast<f32x4*>(dst + r * L + c) = x;
  }
}

// dst[r][c] *= sc[r] over the elements this thread wrote in load_rows (no barrier needed).
template <int N, int L, int NTB>
__device__ __forceinline__ void scale_rows(float* dst, const float* sc) {
  constexpr int PIECES = BC * N / 4, PT = PIECES / NTB;
  static_assert(PIECES % NTB == 0, "whole pieces per thread");
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = threadIdx.x + NTB * u;
    const int r = e / (N / 4), c = 4 * (e % (N / 4));
    *reinterpret_cast<f32x4*>(dst + r * L + c) *= sc[r];
  }
}

template <bool OPTS>
__global__ __launch_bounds__(NTP, 4) void rec256_kernel(Rec256Params p) {
  constexpr int KW = 256;
  using R = Rec<KW, bf16>;
  __shared__ __align__(16) float sQ[BC * LKQ];  // q (part), then P, then W (part)
  __shared__ __align__(16) float sK[BC * LKQ];  // k (part)
  __shared__ __align__(16) float sB[BC * LKQ];  // b log2 e (part), then beta k e^b (part)
  __shared__ __align__(16) float sA[BC * 68];   // A (strict lower), then T = (I + A)^{-1}
  __shared__ float sBeta[BC];
  const int jj = blockIdx.x, h = blockIdx.y, H = p.H;
  const int64_t e = p.seg_begin + jj;
  if (jj >= p.E || e >= p.header[0]) return;
  const Entry en = p.entries[e];
  const int64_t tok = en.tok;
  const int len = en.len;
  const bf16 *q = (const bf16*)p.q, *k = (const bf16*)p.k, *g = (const bf16*)p.g,
             *beta = (const bf16*)p.beta, *v = (const bf16*)p.v;
  char* rc = p.rec + ((int64_t)jj * H + h) * p.rec_bytes;
  bf16* recM = reinterpret_cast<bf16*>(rc);
  float* recGam = reinterpret_cast<float*>(rc + R::oGamBytes);
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, gg = lane >> 4;
  const int ft = tid >> 7, fsl = (tid >> 6) & 1;
  // element e of a slot covers reduction index 32 step + kk(e) of row 16 tile + m
  auto kk = [&](int el) { return 16 * (el >> 2) + 4 * gg + (el & 3); };
  auto put = [&](size_t elem, const float (&x)[8]) {
    bf16x8 f;
#pragma unroll
    for (int el = 0; el < 8; ++el) f[el] = (bf16)x[el];
    *reinterpret_cast<bf16x8*>(recM + elem) = f;
  };
  const uint32_t opts = OPTS ? p.opts : 0u;
  __shared__ float sNq[OPTS ? BC : 1], sNk[OPTS ? BC : 1];  // inverse L2 norms of q and k rows
  if (tid < BC) {
    float b = tid < len ? to_f32(beta[(tok + tid) * H + h]) : 0.f;
    if (opts & OPT_BETA_LOGITS) b = tid < len ? sigmoid_f(b) : 0.f;
    sBeta[tid] = b;
  }
  if constexpr (OPTS) {
    if (opts & OPT_L2NORM_QK) {
      // eight threads per token row, 32 channels each (rows past len repeat the last token)
      static_assert(NTP == 8 * BC, "eight threads per row");
      const int r = tid >> 3, part = tid & 7;
      const int64_t row = ((tok + min(r, len - 1)) * H + h) * (int64_t)KW + 32 * part;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(q + row + 8 * i);
        const bf16x8 xk = *reinterpret_cast<const bf16x8*>(k + row + 8 * i);
#pragma unroll
        for (int el = 0; el < 8; ++el) {
          const float a = (float)xq[el], b = (float)xk[el];
          sq += a * a;
          sk += b * b;
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        sq += __shfl_xor(sq, o);
        sk += __shfl_xor(sk, o);
      }
      if (part == 0) {
        sNq[r] = 1.f / sqrtf(sq + L2NORM_EPS);
        sNk[r] = 1.f / sqrtf(sk + L2NORM_EPS);
      }
    }
    lds_barrier();
  }
  PairAcc acc;
  pair_acc_init<NTP>(acc);
  for (int hh = 0; hh < KW / KQ; ++hh) {
    const int c0 = hh * KQ;
    load_rows<KQ, LKQ, NTP, bf16, KW>(sQ, q, tok, len, H, h, c0);
    load_rows<KQ, LKQ, NTP, bf16, KW>(sK, k, tok, len, H, h, c0);
    if constexpr (OPTS) {
      gate_rows_opts<KQ, LKQ, NTP, KW>(sB, g, tok, len, H, h, c0, opts);
      if (opts & OPT_L2NORM_QK) {
        scale_rows<KQ, LKQ, NTP>(sQ, sNq);
        scale_rows<KQ, LKQ, NTP>(sK, sNk);
      }
    } else {
      load_rows<KQ, LKQ, NTP, bf16, KW>(sB, g, tok, len, H, h, c0);
    }
    lds_barrier();
    cumsum_log2<KQ, LKQ, NTP>(sB, OPTS ? 1.f : LOG2E);  // the option path holds log2 alpha
    lds_barrier();
    // Qe = q e^b (token tile ft, channel step 2 hh + fsl) and Ktilde^T = (k e^{b_last - b})^T
    // (channel tile 4 hh + ft, token step fsl); rows past len hold q = k = 0. beta k e^b goes
    // to the slot of W that this thread fills from it later (the W pass reads it back).
    {
      float x[8], y[8];
      const int r = 16 * ft + m;
#pragma unroll
      for (int el = 0; el < 8; ++el) {
        const int cq = 32 * fsl + kk(el);
        const float eb = exp2_f(sB[r * LKQ + cq]);
        x[el] = sQ[r * LKQ + cq] * eb;
        y[el] = sK[r * LKQ + cq] * eb * sBeta[r];
      }
      put(R::oQ + slot_elem<bf16>(ft, 2 * hh + fsl, lane, KW), x);
      put(R::oW + slot_elem<bf16>(ft, 2 * hh + fsl, lane, KW), y);
    }
    {
      float y[8];
      const int c = 16 * ft + m;
      const float bl = sB[(BC - 1) * LKQ + c];
#pragma unroll
      for (int el = 0; el < 8; ++el) {
        const int rk = 32 * fsl + kk(el);
        y[el] = sK[rk * LKQ + c] * exp2_f(bl - sB[rk * LKQ + c]);
      }
      put(R::oKt + slot_elem<bf16>(4 * hh + ft, fsl, lane, CHUNK), y);
    }
    if (tid < KQ) recGam[c0 + tid] = exp2_f(sB[(BC - 1) * LKQ + tid]);
    pair_acc_part<KQ, LKQ>(acc, sQ, sK, sB);
    lds_barrier();  // the part's reads done before the next part overwrites it
  }
  // A (beta-scaled, zero on and above the diagonal) into sA; P (zero above the diagonal) into
  // sQ, then its fragments
  for (int el = tid; el < BC * BC; el += NTP) {
    sQ[(el / BC) * LKQ + el % BC] = 0.f;
    sA[(el / BC) * 68 + el % BC] = 0.f;
  }
  lds_barrier();
  pair_acc_out(acc, [&](int i, int j, float x) { sA[i * 68 + j] = sBeta[i] * x; },
               [&](int i, int j, float x) { sQ[i * LKQ + j] = x; });
  lds_barrier();
  {
    float x[8];
#pragma unroll
    for (int el = 0; el < 8; ++el) x[el] = sQ[(16 * ft + m) * LKQ + 32 * fsl + kk(el)];
    put(R::oPb + slot_elem<bf16>(ft, fsl, lane, CHUNK), x);
  }
  float* sT = sA;
  unit_lower_inverse_blocked<NTP>(sT);  // T over A
  {  // T' = T diag(beta) (zero above the diagonal)
    float x[8];
#pragma unroll
    for (int el = 0; el < 8; ++el) {
      const int c = 32 * fsl + kk(el);
      x[el] = sT[(16 * ft + m) * 68 + c] * sBeta[c];
    }
    put(R::oTb + slot_elem<bf16>(ft, fsl, lane, CHUNK), x);
  }
  // -W = -T (beta k e^b), part by part (token tile ft, channel step 2 hh + fsl), from the
  // part's beta k e^b this thread left in its W slot (and in sB through the other threads');
  // the slot's store has completed before its load (all memory counters waited out)
  __builtin_amdgcn_s_waitcnt(0);
  for (int hh = 0; hh < KW / KQ; ++hh) {
    {
      const bf16x8 f = *reinterpret_cast<const bf16x8*>(recM + R::oW + slot_elem<bf16>(ft, 2 * hh + fsl, lane, KW));
#pragma unroll
      for (int el = 0; el < 8; ++el) sB[(16 * ft + m) * LKQ + 32 * fsl + kk(el)] = (float)f[el];
    }
    lds_barrier();
    mmf<KQ, BC, false, false, 68, LKQ, NTP>(sT, sB, [&](int r, int cc, float x) { sK[r * LKQ + cc] = x; });
    lds_barrier();
    float x[8];
#pragma unroll
    for (int el = 0; el < 8; ++el) x[el] = -sK[(16 * ft + m) * LKQ + 32 * fsl + kk(el)];
    put(R::oW + slot_elem<bf16>(ft, 2 * hh + fsl, lane, KW), x);
    lds_barrier();
  }
  // V slice-major: row r of slice c (value columns 16c .. 16c + 15) at oVBytes + c * vslice +
  // 32 r bytes; rows past len repeat the last valid row (T' is zero in those columns)
  const int ppr = p.V / 8;  // 16-byte pieces per row
  for (int id = tid; id < BC * ppr; id += NTP) {
    const int r = id / ppr, c = id % ppr;
    const int64_t t = tok + min(r, len - 1);
    const uint4 x = *reinterpret_cast<const uint4*>(v + (t * H + h) * (int64_t)p.V + 8 * c);
    *reinterpret_cast<uint4*>(rc + R::oVBytes + (size_t)(c >> 1) * R::vslice_bytes +
                              (size_t)r * 32 + 16 * (c & 1)) = x;
  }
}

void launch_rec256(const Rec256Params& p, hipStream_t st) {
  if (p.opts != 0)
    hipLaunchKernelGGL(rec256_kernel<true>, dim3((unsigned)p.E, (unsigned)p.H), dim3(NTP), 0, st, p);
  else
    hipLaunchKernelGGL(rec256_kernel<false>, dim3((unsigned)p.E, (unsigned)p.H), dim3(NTP), 0, st, p);
}

// The chain of one (sequence, head, CW value columns); blockIdx = slice * chains8 + chain, so
// the slices of a chain share one XCD's L2. Per chunk: W staged, Delta = U - W S (wave w:
// rows 16 w ..); Qe staged, O = Qe S + P Delta (wave w: rows 16 w ..); Kt staged,
// S' = diag(gamma) S + Kt^T Delta (wave w: 16-row tiles w, w + 4, ..), each staged A operand
// read once for the CW / 16 column blocks. The next block's loads are issued before the
// current block's products. CW = 32 at V = 256 keeps the chains to one wave of workgroups.
// The chunks [cb, ce) of one segment (records indexed from cb): a sequence that began before
// the segment starts from its state in `run`, and one that goes on past it leaves its state
// there (run may be fin); empty sequences (final state = initial state) belong to the segment
// at chunk 0.
template <int KW, int V, int CW, typename MT>
__global__ __launch_bounds__(NT) void wide_state_kernel(
    const float* __restrict__ rec, const float* __restrict__ init, const int32_t* __restrict__ cu,
    int64_t T, const int32_t* __restrict__ seq_first, int N, int H, int chains8, int cb, int ce,
    float* run, MT* __restrict__ o, float* fin) {
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
  const int sfirst = seq_first[n], slast = seq_first[n + 1];
  const int first = max(sfirst, cb), last = min(slast, ce);  // the sequence's chunks here
  if (sfirst < slast ? first >= last : cb != 0) return;
  const size_t sb = (size_t)nh * KW * V;
  const float* src = sfirst < cb ? run + sb : (init ? init + sb : nullptr);
  for (int e = tid; e < KW * CW; e += NT)
    sS[(e / CW) * LS + e % CW] = src ? src[(e / CW) * V + c0 + e % CW] : 0.f;
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
  if (first < last) fetch_head(rec + ((size_t)(first - cb) * H + h) * R::floats);
  for (int c = first; c < last; ++c) {
    const float* rc = rec + ((size_t)(c - cb) * H + h) * R::floats;
    const int64_t tok = s0 + (int64_t)(c - sfirst) * BC;
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
    fetch_head(rec + ((size_t)((c + 1 < last ? c + 1 : c) - cb) * H + h) * R::floats);
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
  float* dst = (sfirst < slast && slast > ce) ? run + sb : (fin ? fin + sb : nullptr);
  if (dst) {
    __syncthreads();
    for (int e = tid; e < KW * CW; e += NT) dst[(e / CW) * V + c0 + e % CW] = sS[(e / CW) * LS + e % CW];
  }
}

// ---------------------------------------------------------------- host
static size_t al256w(size_t x) { return (x + 255) / 256 * 256; }

// fp32 values of one (chunk, head) record (0 for unsupported head dims)
static size_t wide_rec_floats(int K, int V) {
#define KDA_WREC(KK, VV) \
  if (K == KK && V == VV) return WRec<KK, VV>::floats;
  KDA_WREC(128, 32) KDA_WREC(128, 64) KDA_WREC(128, 128) KDA_WREC(128, 256)
  KDA_WREC(256, 32) KDA_WREC(256, 64) KDA_WREC(256, 128) KDA_WREC(256, 256)
#undef KDA_WREC
  return 0;
}

bool make_wide_plan(int N, int64_t T, int H, int K, int V, WidePlan* p) {
  if (N <= 0 || H <= 0 || T < 0) return false;
  const size_t rec_floats = wide_rec_floats(K, V);
  if (rec_floats == 0) return false;
  int64_t ub = (T + (int64_t)N * (BC - 1)) / BC;
  if (ub > T) ub = T;
  p->ub = ub;
  // segments of at most WIDE_SEGMENT_BYTES of records
  int64_t e = (int64_t)(WIDE_SEGMENT_BYTES / ((size_t)H * rec_floats * 4));
  if (e < 1) e = 1;
  p->seg = ub > 0 && e > ub ? ub : e;
  p->nseg = ub > 0 ? (ub + p->seg - 1) / p->seg : 1;
  if (ub >= (1LL << 31)) return false;
  size_t off = 0;
  p->off_seq = off;
  off += al256w((size_t)(N + 1) * 4);
  p->off_rows = off;
  off += al256w((size_t)ub * sizeof(ChunkRow));
  p->off_rec = off;
  off += al256w((size_t)p->seg * H * rec_floats * 4);
  // the input-option pass over one segment's tokens: q, k, log alpha, beta in fp32
  const size_t tk = al256w((size_t)p->seg * BC * H * K * 4);
  p->off_opt_q = off;
  p->off_opt_k = off + tk;
  p->off_opt_g = off + 2 * tk;
  p->off_opt_b = off + 3 * tk;
  off += 3 * tk + al256w((size_t)p->seg * BC * H * 4);
  // the running state between segments when the caller keeps no final state
  p->off_run = off;
  if (p->nseg > 1) off += al256w((size_t)N * H * K * V * 4);
  p->total_bytes = off;
  return true;
}

template <int K, int V, typename MT, typename GT>
static hipError_t launch_wide_t(const ChunkArgs& a, const WidePlan& p) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + p.off_seq);
  ChunkRow* rows = reinterpret_cast<ChunkRow*>(ws + p.off_rows);
  float* rec = reinterpret_cast<float*>(ws + p.off_rec);
  float* run = a.final_state ? a.final_state : reinterpret_cast<float*>(ws + p.off_run);
  const int N = a.num_seqs, H = a.num_heads;
  const int32_t* ntot = seq_first + N;
  hipError_t e = launch_chunk_rows(a.cu_seqlens, N, a.total_tokens, p.ub, seq_first, rows, st);
  if (e != hipSuccess) return e;
  const bool opts = a.options != 0;
  const OptBuffers ob{reinterpret_cast<float*>(ws + p.off_opt_q), reinterpret_cast<float*>(ws + p.off_opt_k),
                      reinterpret_cast<float*>(ws + p.off_opt_g), reinterpret_cast<float*>(ws + p.off_opt_b)};
  const GT *q = opts ? (const GT*)ob.q : (const GT*)a.q, *k = opts ? (const GT*)ob.k : (const GT*)a.k,
           *g = opts ? (const GT*)ob.g : (const GT*)a.g, *beta = opts ? (const GT*)ob.beta : (const GT*)a.beta;
  const int chains8 = (N * H + 7) / 8 * 8;
  constexpr int CW = V == 256 ? 32 : 16;  // value columns per chain workgroup
  for (int64_t s = 0; s < p.nseg; ++s) {
    const int cb = (int)(s * p.seg), ce = (int)min((s + 1) * p.seg, p.ub);
    if (ce > cb) {
      if (opts)
        launch_prologue(OptInputs{a.q, a.k, a.g, a.beta}, a.dtype_bf16, a.total_tokens, H, K,
                        a.options, rows, ntot, cb, ce, ob, st, (int64_t)(ce - cb) * BC);
      hipLaunchKernelGGL((wide_prep_kernel<K, V, MT, GT>), dim3((unsigned)(ce - cb), (unsigned)H),
                         dim3(NTP), 0, st, q, k, (const MT*)a.v, g, beta, H, (const ChunkRow*)rows,
                         ntot, cb, opts, rec);
    }
    hipLaunchKernelGGL((wide_state_kernel<K, V, CW, MT>), dim3((unsigned)(chains8 * (V / CW))),
                       dim3(NT), 0, st, (const float*)rec, a.init_state, a.cu_seqlens,
                       a.total_tokens, (const int32_t*)seq_first, N, H, chains8, cb, ce, run,
                       (MT*)a.o, a.final_state);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_fwd_wide(const ChunkArgs& a, const WidePlan& p) {
  const bool o = a.options != 0;
#define KDA_WIDE_CASE(KK, VV)                                                               \
  if (a.dk == KK && a.dv == VV)                                                             \
    return a.dtype_bf16 ? (o ? launch_wide_t<KK, VV, bf16, float>(a, p)                     \
                             : launch_wide_t<KK, VV, bf16, bf16>(a, p))                     \
                        : launch_wide_t<KK, VV, float, float>(a, p);
  KDA_WIDE_CASE(256, 32) KDA_WIDE_CASE(256, 64) KDA_WIDE_CASE(256, 128) KDA_WIDE_CASE(256, 256)
#undef KDA_WIDE_CASE
  // K = 128 comes here for fp32 inputs only (bf16 takes the chunk path)
#define KDA_WIDE_CASE(VV) \
  if (a.dk == 128 && a.dv == VV && !a.dtype_bf16) return launch_wide_t<128, VV, float, float>(a, p);
  KDA_WIDE_CASE(32) KDA_WIDE_CASE(64) KDA_WIDE_CASE(128) KDA_WIDE_CASE(256)
#undef KDA_WIDE_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
