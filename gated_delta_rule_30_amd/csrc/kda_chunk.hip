// Chunkwise KDA forward on gfx950.
//
// Method ("Kimi Linear's Hybrid Linear Attention Architecture: A Technical Breakdown",
// section 4; the exponents are derived from the token recurrence because the printed
// superscripts are garbled). For one chunk of tokens with chunk-start state S and
// b_i = sum_{s<=i} log alpha_s (per key channel):
//   A_ij  = beta_i sum_c k_ic k_jc e^{b_ic - b_jc}    (j < i)        KGammaK^T block
//   T     = (I + A)^{-1}                                               UT triangular solve
//   T'    = T diag(beta),  W = T' (K * e^{b}),  U = T' V               WY factors
//   P_ij  = sum_c q_ic k_jc e^{b_ic - b_jc}           (j <= i)       QGammaK^T block
//   Delta = U - W S                                                    delta corrections
//   O     = (Q * e^{b}) S + P Delta = Q_eff S + P' V,  Q_eff = Q*e^{b} - P W,  P' = P T'
//   S'    = Diag(e^{b_last}) S + (K * e^{b_last - b})^T Delta          state passing
// The WY / UT form of the chunk's rank-1 updates and the triangular solve follow the pages'
// description ("Kimi Linear" explainer, "WY Representation"; wpnews article, DPLR paragraph).
//
// Execution. Work that does not depend on the state (everything but the three state
// GEMMs) is independent per (chunk, head) and runs in the chunk-parallel PREP kernel, which
// writes one compact record per (chunk, head): W, Q_eff, Ktilde^T, T', P' (bf16 MFMA
// fragments) and e^{b_last}. The STATE kernel walks each sequence's chunks in order, one
// workgroup per (sequence, head, V-slice) -- the columns of S evolve independently, so the
// V split is exact -- and does only U = T'V, O = Q_eff S + P'V, Delta = U - W S and the
// update S' = Diag(gamma) S + Ktilde^T Delta on the matrix cores. The sequence is processed
// in segments of about SEG_CHUNK_HEADS records so the record buffers stay resident in the
// Infinity Cache between the two kernels.
//
// Numerics. Inside a chunk every decay factor is formed relative to a 16-token sub-block
// reference so it stays in fp32 range: row factors e^{b_i - e_{I-1}} <= 1, column factors
// e^{e_J - b_j} <= 1 and per-channel block factors e^{e_{I-1} - e_J} <= 1 (J < I), with only
// the diagonal sub-block using e^{-(block decay)} >= 1 (the renormalisation the Technical
// Breakdown asks for in section 4's numerical-stability note). The solve runs in fp32 on
// VALU (diagonal 16x16 blocks) and fp32 MFMA (off-diagonal blocks). The state stays fp32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ====================================================================== record layout
// Matrices are stored as MFMA A-operand fragments: for a matrix with R rows and reduction
// length L, the 16-byte slot of (row tile, reduction step, lane) is at element
//     ((tile * (L / KS) + step) * 64 + lane) * EPL
// and element e of the slot of lane (m, g) is (row 16*tile + m, index KS*step + kk(g, e)).
template <int K, typename MT>
struct Rec {
  static constexpr size_t oW = 0;                                // [CHUNK rows][K]
  static constexpr size_t oQ = oW + (size_t)CHUNK * K;           // [CHUNK rows][K]
  static constexpr size_t oKt = oQ + (size_t)CHUNK * K;          // [K rows][CHUNK]
  static constexpr size_t oTb = oKt + (size_t)K * CHUNK;         // [CHUNK rows][CHUNK]
  static constexpr size_t oPb = oTb + (size_t)CHUNK * CHUNK;     // [CHUNK rows][CHUNK]
  static constexpr size_t nMat = oPb + (size_t)CHUNK * CHUNK;
  static constexpr size_t oGamBytes = nMat * sizeof(MT);         // K fp32
  static constexpr size_t bytes = (oGamBytes + K * 4 + 255) / 256 * 256;
};

template <typename MT>
__device__ __forceinline__ size_t slot_elem(int tile, int step, int lane, int L) {
  return ((size_t)(tile * (L / Mma<MT>::KS) + step) * 64 + lane) * Mma<MT>::EPL;
}

// four consecutive MT values from fp32
__device__ __forceinline__ void st4(bf16* p, f32x4 x) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
__device__ __forceinline__ void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// ====================================================================== chunk table
// Entries are ordered depth-major: chunk d of every sequence that has one, then chunk d+1,
// so one segment advances many sequences at once and short sequences drop out early.
// position(n, d) = sum_{n'} min(nc_{n'}, d) + #{n' < n : nc_{n'} > d}.
struct SeqView {
  const int32_t* cu;
  int num_seqs;
  int64_t total;
  __device__ int64_t start(int n) const { return cu ? (int64_t)cu[n] : (total / num_seqs) * n; }
  __device__ int64_t len(int n) const {
    return cu ? (int64_t)cu[n + 1] - (int64_t)cu[n] : total / num_seqs;
  }
  __device__ int64_t nchunks(int n) const { return (len(n) + CHUNK - 1) / CHUNK; }
};

__global__ __launch_bounds__(256) void table_kernel(SeqView sv, int H, int64_t KV, int64_t ub,
                                                    const float* __restrict__ init,
                                                    float* __restrict__ fin,
                                                    Entry* __restrict__ entries,
                                                    int32_t* __restrict__ header) {
  const int n = blockIdx.x;
  const int64_t len = sv.len(n);
  const int64_t nc = sv.nchunks(n);
  for (int64_t d = threadIdx.x; d < nc; d += blockDim.x) {
    int64_t pos = 0, posm = 0, posp = 0;
    for (int j = 0; j < sv.num_seqs; ++j) {
      const int64_t cj = sv.nchunks(j);
      pos += min(cj, d) + ((j < n && cj > d) ? 1 : 0);
      posm += min(cj, d - 1) + ((j < n && cj > d - 1) ? 1 : 0);
      posp += min(cj, d + 1) + ((j < n && cj > d + 1) ? 1 : 0);
    }
    Entry en;
    en.seq = n;
    en.tok = (int32_t)(sv.start(n) + d * CHUNK);
    en.len = (int32_t)min((int64_t)CHUNK, len - d * CHUNK);
    en.depth = (int32_t)d;
    en.prev = d > 0 ? (int32_t)posm : -1;
    en.next = d + 1 < nc ? (int32_t)posp : -1;
    en.pad0 = en.pad1 = 0;
    if (pos < ub) entries[pos] = en;  // always true for a well-formed cu_seqlens
  }
  if (nc == 0 && fin != nullptr) {  // empty sequence: final state = initial state (or zero)
    const int64_t base = (int64_t)n * H * KV;
    for (int64_t i = threadIdx.x; i < (int64_t)H * KV; i += blockDim.x)
      fin[base + i] = init ? init[base + i] : 0.f;
  }
  if (n == 0 && threadIdx.x == 0) {
    int64_t tot = 0;
    for (int j = 0; j < sv.num_seqs; ++j) tot += sv.nchunks(j);
    header[0] = (int32_t)min(tot, ub);
  }
}

// Per segment, the ordered list of entries that start a sequence's run inside the segment.
__global__ __launch_bounds__(256) void segment_kernel(const Entry* __restrict__ entries,
                                                      const int32_t* __restrict__ header,
                                                      int64_t E, int64_t slots,
                                                      int32_t* __restrict__ seg_first,
                                                      int32_t* __restrict__ seg_count) {
  const int64_t s = blockIdx.x;
  const int64_t total = header[0];
  const int64_t b = s * E;
  const int64_t end = min(b + E, total);
  const int64_t per = (E + 255) / 256;
  const int64_t lo = b + threadIdx.x * per;
  const int64_t hi = min(lo + per, end);
  int cnt = 0;
  for (int64_t e = lo; e < hi; ++e) cnt += (entries[e].prev < b) ? 1 : 0;
  __shared__ int scan[256];
  scan[threadIdx.x] = cnt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int x = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += x;
    __syncthreads();
  }
  int out = scan[threadIdx.x] - cnt;
  for (int64_t e = lo; e < hi; ++e)
    if (entries[e].prev < b && out < slots) seg_first[s * slots + out++] = (int32_t)e;
  if (threadIdx.x == 255) seg_count[s] = (int32_t)min((int64_t)scan[255], slots);
}

// ====================================================================== PREP kernel
template <int K, typename MT>
struct PrepLayout {
  static constexpr int PADM = 16 / (int)sizeof(MT);
  static constexpr int LK = K + PADM;        // MT rows of length K
  static constexpr int LC = CHUNK + PADM;    // MT rows of length CHUNK
  static constexpr int LKF = K + 4;          // fp32 rows of length K
  static constexpr int LCF = CHUNK + 4;      // fp32 rows of length CHUNK
  static constexpr int NPAIR = NSUB * (NSUB + 1) / 2;
  static constexpr size_t szQh = (size_t)CHUNK * LK * sizeof(MT);
  static constexpr size_t szKh = szQh;
  static constexpr size_t szKb = (size_t)CHUNK * LKF * 4;
  static constexpr size_t szTri = (size_t)CHUNK * LC * sizeof(MT);
  static constexpr size_t szX = (szKh + szKb) > 3 * szTri ? (szKh + szKb) : 3 * szTri;
  static constexpr size_t szKaT = (size_t)K * LC * sizeof(MT);
  static constexpr size_t szD = (size_t)NPAIR * K * 4;
  static constexpr size_t szEx = (size_t)NSUB * K * 4;
  static constexpr size_t szDel = (size_t)NSUB * K * 4;
  static constexpr size_t szBeta = (size_t)CHUNK * 4;
  static constexpr size_t szAf = (size_t)CHUNK * LCF * 4;
  static constexpr size_t szY = 2 * szAf > szKaT ? 2 * szAf : szKaT;
  static constexpr size_t oQh = 0;
  static constexpr size_t oX = oQh + szQh;
  static constexpr size_t oKh = oX, oKb = oX + szKh;                             // phases 1-2
  static constexpr size_t oTb = oX, oTbT = oX + szTri, oPn = oX + 2 * szTri;     // phases 4-6
  static constexpr size_t oKaT = oX + szX;
  static constexpr size_t oD = oKaT + szKaT;
  static constexpr size_t oEx = oD + szD;
  static constexpr size_t oDel = oEx + szEx;
  static constexpr size_t oBeta = oDel + szDel;
  static constexpr size_t oY = oBeta + szBeta;
  static constexpr size_t oA = oY, oP = oY + szAf;                               // phases 2-4
  static constexpr size_t oWT = oY;                                               // phases 5-6
  static constexpr size_t total = oY + szY;
};

struct PrepParams {
  const void *q, *k, *g, *beta;
  const Entry* entries;
  const int32_t* header;
  int H;
  int64_t seg_begin;  // first entry of the segment
  int64_t E;          // entries per segment
  char* rec;          // record buffer of the segment
  int64_t rec_bytes;
};

template <int K, typename MT>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
  using L = PrepLayout<K, MT>;
  using R = Rec<K, MT>;
  constexpr int KS = Mma<MT>::KS;
  constexpr int EPL = Mma<MT>::EPL;
  static_assert(L::total <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) char smem[L::total];
  MT* sQh = reinterpret_cast<MT*>(smem + L::oQh);
  MT* sKh = reinterpret_cast<MT*>(smem + L::oKh);
  float* sKb = reinterpret_cast<float*>(smem + L::oKb);
  MT* sTb = reinterpret_cast<MT*>(smem + L::oTb);
  MT* sTbT = reinterpret_cast<MT*>(smem + L::oTbT);
  MT* sPn = reinterpret_cast<MT*>(smem + L::oPn);
  MT* sKaT = reinterpret_cast<MT*>(smem + L::oKaT);
  float* sD = reinterpret_cast<float*>(smem + L::oD);
  float* sEx = reinterpret_cast<float*>(smem + L::oEx);
  float* sDel = reinterpret_cast<float*>(smem + L::oDel);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  float* sP = reinterpret_cast<float*>(smem + L::oP);
  MT* sWT = reinterpret_cast<MT*>(smem + L::oWT);

  const int H = p.H;
  const int64_t j = blockIdx.x / H;
  const int h = blockIdx.x % H;
  const int64_t e = p.seg_begin + j;
  if (j >= p.E || e >= (int64_t)p.header[0]) return;
  const Entry en = p.entries[e];
  const int len = en.len;
  const int64_t tok0 = en.tok;
  const MT* gq_ = reinterpret_cast<const MT*>(p.q);
  const MT* gk_ = reinterpret_cast<const MT*>(p.k);
  const MT* gg_ = reinterpret_cast<const MT*>(p.g);
  const MT* gb_ = reinterpret_cast<const MT*>(p.beta);
  char* rec = p.rec + (j * H + h) * p.rec_bytes;
  MT* recM = reinterpret_cast<MT*>(rec);
  float* recGam = reinterpret_cast<float*>(rec + R::oGamBytes);

  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = lane_id();
  const int m = lane & 15;
  const int gq = lane >> 4;
  const int64_t rowstride = (int64_t)H * K;  // elements between consecutive tokens

  // ---------------- phase 1a: in-block cumulative log decay per (channel, sub-block)
  constexpr int NPAIRS_CB = K * NSUB;
  constexpr int PPT = (NPAIRS_CB + NTHREADS - 1) / NTHREADS;
  float lreg[PPT][SUBBLK];
  if (tid < CHUNK) sBeta[tid] = tid < len ? to_f32(gb_[(tok0 + tid) * H + h]) : 0.f;
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    const int pidx = tid + pp * NTHREADS;
    if (pidx < NPAIRS_CB) {
      const int c = pidx % K, I = pidx / K;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < SUBBLK; ++i) {
        const int t = I * SUBBLK + i;
        const float gv = t < len ? to_f32(gg_[(tok0 + t) * rowstride + (int64_t)h * K + c]) : 0.f;
        acc += gv;
        lreg[pp][i] = acc;
      }
      sDel[I * K + c] = acc;
    }
  }
  __syncthreads();

  // ---------------- phase 1b: decayed operands, D table, Ktilde^T and gamma to the record
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    const int pidx = tid + pp * NTHREADS;
    if (pidx < NPAIRS_CB) {
      const int c = pidx % K, I = pidx / K;
      float ecum[NSUB + 1];  // ecum[J+1] = e_J, ecum[0] = 0 (chunk start)
      ecum[0] = 0.f;
#pragma unroll
      for (int J = 0; J < NSUB; ++J) ecum[J + 1] = ecum[J] + sDel[J * K + c];
      const float eprev = ecum[I];          // e_{I-1}
      const float dI = sDel[I * K + c];     // block decay (log), <= 0
      const float elast = ecum[NSUB];
      const float Eprev = exp_f(eprev);
      const float tailf = exp_f(elast - ecum[I + 1]);  // e^{e_last - e_I}
      sEx[I * K + c] = Eprev;
      // D table for pairs (I, J <= I)
      const int pbase = I * (I + 1) / 2;
#pragma unroll
      for (int J = 0; J < NSUB; ++J)
        if (J <= I) sD[(pbase + J) * K + c] = (J < I) ? exp_f(eprev - ecum[J + 1]) : exp_f(-dI);
      if (I == NSUB - 1) recGam[c] = exp_f(elast);
      float ktv[SUBBLK];
#pragma unroll
      for (int i = 0; i < SUBBLK; ++i) {
        const int t = I * SUBBLK + i;
        float qv = 0.f, kv = 0.f;
        if (t < len) {
          const int64_t off = (tok0 + t) * rowstride + (int64_t)h * K + c;
          qv = to_f32(gq_[off]);
          kv = to_f32(gk_[off]);
        }
        const float l = lreg[pp][i];
        const float r = exp_f(l);          // e^{b_t - e_{I-1}} <= 1
        const float cc = exp_f(dI - l);    // e^{e_I - b_t} <= 1
        sQh[t * L::LK + c] = from_f32<MT>(qv * r);
        sKh[t * L::LK + c] = from_f32<MT>(kv * r);
        sKb[t * L::LKF + c] = kv * cc;
        sKaT[c * L::LC + t] = from_f32<MT>(kv * r * Eprev);
        ktv[i] = kv * cc * tailf;          // k * e^{b_last - b_t}
      }
      // Ktilde^T rows = channels, reduction = tokens: 4 quads of consecutive tokens
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int t0 = I * SUBBLK + 4 * qd;
        const int s = t0 / KS, kp = t0 % KS;
        const int ln = ((kp & 15) >> 2) * 16 + (c & 15);
        st4(recM + R::oKt + slot_elem<MT>(c >> 4, s, ln, CHUNK) + 4 * (kp >> 4),
            f32x4{ktv[4 * qd], ktv[4 * qd + 1], ktv[4 * qd + 2], ktv[4 * qd + 3]});
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: A (strictly lower, row-scaled by beta) and P (lower) blocks
  {
    int pr = 0;
#pragma unroll
    for (int I = 0; I < NSUB; ++I) {
#pragma unroll
      for (int J = 0; J <= I; ++J, ++pr) {
        if ((pr & 3) != w) continue;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < K / KS; ++s) {
          auto ak = load_frag(sKh + (16 * I + m) * L::LK, s, gq);
          auto aq = load_frag(sQh + (16 * I + m) * L::LK, s, gq);
          auto b = load_frag_scaled(sKb + (16 * J + m) * L::LKF, sD + pr * K, s, gq, MT());
          accA = Mma<MT>::mma(ak, b, accA);
          accP = Mma<MT>::mma(aq, b, accP);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * gq + r, jj = 16 * J + m;
          float a = accA[r] * sBeta[i];
          float pv = accP[r];
          if (I == J) {
            if (jj >= i) a = 0.f;
            if (jj > i) pv = 0.f;
          }
          sA[i * L::LCF + jj] = a;
          sP[i * L::LCF + jj] = pv;
        }
      }
    }
    // upper blocks (J > I) of P are zero; those of A are never read
    for (int idx = tid; idx < NSUB * NSUB * 256; idx += NTHREADS) {
      const int blk = idx >> 8, I = blk / NSUB, J = blk % NSUB;
      if (J > I) {
        const int i = 16 * I + ((idx >> 4) & 15), jj = 16 * J + (idx & 15);
        sP[i * L::LCF + jj] = 0.f;
      }
    }
  }
  __syncthreads();

  // ---------------- phase 3: T = (I + A)^{-1}
  // Diagonal 16x16 blocks: forward substitution, one lane per column, in place.
  if (w == 0) {
    const int I = lane >> 4, c = lane & 15;
    float* Ab = sA + (16 * I) * L::LCF + 16 * I;
    float t[SUBBLK];
#pragma unroll
    for (int i = 0; i < SUBBLK; ++i) {
      float x = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < i; ++jj) x -= Ab[i * L::LCF + jj] * t[jj];
      t[i] = x;
    }
#pragma unroll
    for (int i = 0; i < SUBBLK; ++i) Ab[i * L::LCF + c] = t[i];
  }
  __syncthreads();
  // T[16I+a][16J+b] for I > J is stored at sA[(16J+a)][16I+b] (the unused upper block).
  auto Tget = [&](int i, int jj) -> float {
    const int I = i >> 4, J = jj >> 4;
    if (I == J) return sA[i * L::LCF + jj];
    if (I > J) return sA[(16 * J + (i & 15)) * L::LCF + 16 * I + (jj & 15)];
    return 0.f;
  };
  // Off-diagonal blocks by block distance: T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ (fp32 MFMA).
#pragma unroll
  for (int d = 1; d < NSUB; ++d) {
    if (w < NSUB - d) {
      const int J = w, I = w + d;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
        const f32x4 af = *reinterpret_cast<const f32x4*>(sA + (16 * I + m) * L::LCF + 16 * M + 4 * gq);
        f32x4 bf;
#pragma unroll
        for (int r = 0; r < 4; ++r) bf[r] = Tget(16 * M + 4 * gq + r, 16 * J + m);
        X = Mma<float>::mma(af, bf, X);
      }
      const f32x4 tf = *reinterpret_cast<const f32x4*>(sA + (16 * I + m) * L::LCF + 16 * I + 4 * gq);
      const f32x4 Y = Mma<float>::mma(tf, X, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sA[(16 * J + 4 * gq + r) * L::LCF + 16 * I + m] = -Y[r];
    }
    __syncthreads();
  }

  // ---------------- phase 4: T' = T diag(beta) (and its transpose), -P, all in MT
  for (int idx = tid; idx < CHUNK * CHUNK; idx += NTHREADS) {
    const int i = idx / CHUNK, jj = idx % CHUNK;
    const float tb = (i >= jj) ? Tget(i, jj) * sBeta[jj] : 0.f;
    sTb[i * L::LC + jj] = from_f32<MT>(tb);
    sTbT[jj * L::LC + i] = from_f32<MT>(tb);
    sPn[i * L::LC + jj] = from_f32<MT>(-sP[i * L::LCF + jj]);
  }
  __syncthreads();
  // T' to the record
  {
    constexpr int NSL = (CHUNK / 16) * (CHUNK / KS) * 64;
    for (int sl = tid; sl < NSL; sl += NTHREADS) {
      const int ln = sl & 63, ts = sl >> 6;
      const int s = ts % (CHUNK / KS), tile = ts / (CHUNK / KS);
      const auto f = load_frag(sTb + (16 * tile + (ln & 15)) * L::LC, s, ln >> 4);
      *reinterpret_cast<typename Mma<MT>::frag*>(recM + R::oTb + (size_t)sl * EPL) = f;
    }
  }

  // ---------------- phase 5: W^T = Ka^T T'^T  -> record (as W fragments) and LDS (W^T)
#pragma unroll
  for (int a = w; a < K / 16; a += 4) {
#pragma unroll
    for (int b = 0; b < NSUB; ++b) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int nsteps = (16 * b + 16 + KS - 1) / KS;
      for (int s = 0; s < nsteps; ++s) {
        const auto af = load_frag(sKaT + (16 * a + m) * L::LC, s, gq);
        const auto bfr = load_frag(sTb + (16 * b + m) * L::LC, s, gq);
        acc = Mma<MT>::mma(af, bfr, acc);
      }
      st4(recM + R::oW + slot_elem<MT>(b, (16 * a) / KS, lane, K) + 4 * ((16 * a % KS) / 16), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sWT[(16 * a + 4 * gq + r) * L::LC + 16 * b + m] = from_f32<MT>(acc[r]);
    }
  }
  __syncthreads();

  // ---------------- phase 6a: Q_eff^T = (Q e^{b})^T + W^T (-P)^T -> record (as Q_eff fragments)
#pragma unroll
  for (int a = w; a < K / 16; a += 4) {
#pragma unroll
    for (int b = 0; b < NSUB; ++b) {
      const int i = 16 * b + m;
      const f32x4 qh = ld4f(sQh + i * L::LK + 16 * a + 4 * gq);
      const f32x4 ex = *reinterpret_cast<const f32x4*>(sEx + b * K + 16 * a + 4 * gq);
      f32x4 acc = qh * ex;
      const int nsteps = (16 * b + 16 + KS - 1) / KS;
      for (int s = 0; s < nsteps; ++s) {
        const auto af = load_frag(sWT + (16 * a + m) * L::LC, s, gq);
        const auto bfr = load_frag(sPn + (16 * b + m) * L::LC, s, gq);
        acc = Mma<MT>::mma(af, bfr, acc);
      }
      st4(recM + R::oQ + slot_elem<MT>(b, (16 * a) / KS, lane, K) + 4 * ((16 * a % KS) / 16), acc);
    }
  }
  // ---------------- phase 6b: P'^T = -(T'^T (-P)^T) -> record (as P' fragments)
  for (int tix = w; tix < NSUB * NSUB; tix += 4) {
    const int a = tix % NSUB, b = tix / NSUB;  // a: column tile (j), b: row tile (i)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a <= b) {
      const int nsteps = (16 * b + 16 + KS - 1) / KS;
      for (int s = 0; s < nsteps; ++s) {
        const auto af = load_frag(sTbT + (16 * a + m) * L::LC, s, gq);
        const auto bfr = load_frag(sPn + (16 * b + m) * L::LC, s, gq);
        acc = Mma<MT>::mma(af, bfr, acc);
      }
      acc = -acc;
    }
    st4(recM + R::oPb + slot_elem<MT>(b, (16 * a) / KS, lane, CHUNK) + 4 * ((16 * a % KS) / 16), acc);
  }
}

// ====================================================================== STATE kernel
template <int K, int NVT, typename MT>
struct StateLayout {
  static constexpr int VS = 16 * NVT;
  static constexpr int PADM = 16 / (int)sizeof(MT);
  static constexpr int LKs = K + PADM;
  static constexpr int LCs = CHUNK + PADM;
  static constexpr int LOs = VS + PADM;
  static constexpr size_t oS = 0;
  static constexpr size_t oDl = oS + (size_t)VS * LKs * sizeof(MT);
  static constexpr size_t oV = oDl + (size_t)VS * LCs * sizeof(MT);
  static constexpr size_t oO = oV + (size_t)VS * LCs * sizeof(MT);
  static constexpr size_t total = oO + (size_t)CHUNK * LOs * sizeof(MT);
};

struct StateParams {
  const void* v;
  void* o;
  const float* init_state;
  float* state;  // running and final state [N][H][K][V]
  const Entry* entries;
  const int32_t* header;
  const int32_t* seg_first;  // this segment's list
  const int32_t* seg_count;  // this segment's count
  int64_t seg_begin, E;
  int H, V, n_slices;
  int64_t chains;  // slots * H
  const char* rec;
  int64_t rec_bytes;
};

template <int K, int NVT, typename MT>
__global__ __launch_bounds__(256) void state_kernel(StateParams p) {
  using SL = StateLayout<K, NVT, MT>;
  using R = Rec<K, MT>;
  using frag = typename Mma<MT>::frag;
  constexpr int KS = Mma<MT>::KS;
  constexpr int VS = SL::VS;
  constexpr int NKT = K / 16;             // row tiles of S
  constexpr int TPW = (NKT + 3) / 4;      // S row tiles per wave
  __shared__ __align__(16) char smem[SL::total];
  MT* sS = reinterpret_cast<MT*>(smem + SL::oS);    // S^T: [VS][K]
  MT* sDl = reinterpret_cast<MT*>(smem + SL::oDl);  // Delta^T: [VS][CHUNK]
  MT* sV = reinterpret_cast<MT*>(smem + SL::oV);    // V^T: [VS][CHUNK]
  MT* sO = reinterpret_cast<MT*>(smem + SL::oO);    // O: [CHUNK][VS]

  // XCD-aware decode: all V-slices of a chain share blockIdx % 8 (the same XCD / L2).
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int rr = bid >> 3;
  const int slice = rr % p.n_slices;
  const int64_t chain = (int64_t)(rr / p.n_slices) * 8 + xcd;
  if (chain >= p.chains) return;
  const int H = p.H, V = p.V;
  const int64_t slot = chain / H;
  const int h = (int)(chain % H);
  if (slot >= p.seg_count[0]) return;
  const int64_t total = p.header[0];
  const int64_t seg_end = min(p.seg_begin + p.E, total);
  int64_t e = p.seg_first[slot];
  const Entry e0 = p.entries[e];
  const int col0 = slice * VS;

  const int w = wave_id();
  const int lane = lane_id();
  const int m = lane & 15;
  const int gq = lane >> 4;

  const size_t sbase = ((size_t)e0.seq * H + h) * (size_t)K * V + col0;
  const float* src = (e0.depth == 0) ? p.init_state : p.state;
  f32x4 Sr[TPW][NVT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int t = w + 4 * tt;
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (t < NKT && src != nullptr) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = src[sbase + (size_t)(16 * t + 4 * gq + r) * V + 16 * nt + m];
      }
      Sr[tt][nt] = x;
      if (t < NKT) st4(sS + (16 * nt + m) * SL::LKs + 16 * t + 4 * gq, x);
    }
  }

  const MT* gv = reinterpret_cast<const MT*>(p.v);
  MT* go = reinterpret_cast<MT*>(p.o);
  const int64_t vrow = (int64_t)H * V;
  const int nst_tri = (16 * w + 16 + KS - 1) / KS;  // reduction steps of T', P' for row tile w

  while (e >= 0 && e < seg_end) {
    const Entry en = p.entries[e];
    const char* rc = p.rec + ((e - p.seg_begin) * H + h) * p.rec_bytes;
    const MT* rm = reinterpret_cast<const MT*>(rc);
    const float* rg = reinterpret_cast<const float*>(rc + R::oGamBytes);

    // V slice of the chunk, transposed into LDS, zero beyond the chunk's length
    for (int idx = threadIdx.x; idx < CHUNK * VS; idx += NTHREADS) {
      const int t = idx / VS, cc = idx % VS;
      const float x = t < en.len ? to_f32(gv[((int64_t)en.tok + t) * vrow + (int64_t)h * V + col0 + cc]) : 0.f;
      sV[cc * SL::LCs + t] = from_f32<MT>(x);
    }
    // this wave's record fragments
    frag wf[K / KS], qf[K / KS], tf[CHUNK / KS], pf[CHUNK / KS], kf[TPW][CHUNK / KS];
#pragma unroll
    for (int s = 0; s < K / KS; ++s) {
      wf[s] = *reinterpret_cast<const frag*>(rm + R::oW + slot_elem<MT>(w, s, lane, K));
      qf[s] = *reinterpret_cast<const frag*>(rm + R::oQ + slot_elem<MT>(w, s, lane, K));
    }
#pragma unroll
    for (int s = 0; s < CHUNK / KS; ++s) {
      tf[s] = *reinterpret_cast<const frag*>(rm + R::oTb + slot_elem<MT>(w, s, lane, CHUNK));
      pf[s] = *reinterpret_cast<const frag*>(rm + R::oPb + slot_elem<MT>(w, s, lane, CHUNK));
    }
    f32x4 gam[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = w + 4 * tt;
      if (t < NKT) {
#pragma unroll
        for (int s = 0; s < CHUNK / KS; ++s)
          kf[tt][s] = *reinterpret_cast<const frag*>(rm + R::oKt + slot_elem<MT>(t, s, lane, CHUNK));
        gam[tt] = *reinterpret_cast<const f32x4*>(rg + 16 * t + 4 * gq);
      }
    }
    __syncthreads();  // sV and sS ready

#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) {
      f32x4 U = {0.f, 0.f, 0.f, 0.f}, Ol = U, Y = U, Z = U;
      for (int s = 0; s < nst_tri; ++s) {
        const auto bv = load_frag(sV + (16 * nt + m) * SL::LCs, s, gq);
        U = Mma<MT>::mma(tf[s], bv, U);
        Ol = Mma<MT>::mma(pf[s], bv, Ol);
      }
#pragma unroll
      for (int s = 0; s < K / KS; ++s) {
        const auto bs = load_frag(sS + (16 * nt + m) * SL::LKs, s, gq);
        Y = Mma<MT>::mma(wf[s], bs, Y);
        Z = Mma<MT>::mma(qf[s], bs, Z);
      }
      const f32x4 D = U - Y;
      const f32x4 O = Ol + Z;
      st4(sDl + (16 * nt + m) * SL::LCs + 16 * w + 4 * gq, D);
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[(16 * w + 4 * gq + r) * SL::LOs + 16 * nt + m] = from_f32<MT>(O[r]);
    }
    __syncthreads();  // Delta and O complete

    // output rows of this chunk
    {
      constexpr int EPV = 16 / (int)sizeof(MT);
      constexpr int VPR = VS / EPV;
      for (int idx = threadIdx.x; idx < CHUNK * VPR; idx += NTHREADS) {
        const int t = idx / VPR, vi = idx % VPR;
        if (t < en.len) {
          const uint4 x = *reinterpret_cast<const uint4*>(sO + t * SL::LOs + vi * EPV);
          *reinterpret_cast<uint4*>(go + ((int64_t)en.tok + t) * vrow + (int64_t)h * V + col0 + vi * EPV) = x;
        }
      }
    }
    // state update S = gamma * S + Ktilde^T Delta
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = w + 4 * tt;
      if (t < NKT) {
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) {
          f32x4 acc = gam[tt] * Sr[tt][nt];
#pragma unroll
          for (int s = 0; s < CHUNK / KS; ++s) {
            const auto bd = load_frag(sDl + (16 * nt + m) * SL::LCs, s, gq);
            acc = Mma<MT>::mma(kf[tt][s], bd, acc);
          }
          Sr[tt][nt] = acc;
          st4(sS + (16 * nt + m) * SL::LKs + 16 * t + 4 * gq, acc);
        }
      }
    }
    e = en.next > e ? en.next : -1;  // entries of a sequence are strictly increasing
  }

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int t = w + 4 * tt;
    if (t < NKT) {
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p.state[sbase + (size_t)(16 * t + 4 * gq + r) * V + 16 * nt + m] = Sr[tt][nt][r];
    }
  }
}

// ====================================================================== host side
bool make_chunk_plan(int N, int64_t T, int H, int K, int V, bool bf16, ChunkPlan* p) {
  if (N <= 0 || H <= 0 || T < 0 || K <= 0 || V <= 0) return false;
  const int64_t es = bf16 ? 2 : 4;
  int64_t ub = (T + (int64_t)N * (CHUNK - 1)) / CHUNK;
  if (ub > T) ub = T;
  p->ub_entries = ub;
  int64_t E = SEG_CHUNK_HEADS / H;
  if (E < 1) E = 1;
  if (ub > 0 && E > ub) E = ub;
  p->seg_entries = E;
  p->num_segs = ub > 0 ? (ub + E - 1) / E : 0;
  p->slots = N < E ? N : E;
  p->rec_bytes = ((3LL * CHUNK * K + 2LL * CHUNK * CHUNK) * es + 4LL * K + 255) / 256 * 256;
  // V split: enough (sequence, head, slice) workgroups to cover the CUs, slices of 16..64
  const int64_t chains = p->slots * H;
  int ns = 1;
  while (chains * ns < 512 && ns < V / 16) ns *= 2;
  while (V / ns > 64) ns *= 2;
  p->n_slices = ns;
  p->vs = V / ns;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p->off_header = off;
  off += 256;
  p->off_entries = off;
  off += al((size_t)ub * sizeof(Entry));
  p->off_seg_first = off;
  off += al((size_t)p->num_segs * p->slots * 4);
  p->off_seg_count = off;
  off += al((size_t)p->num_segs * 4);
  p->off_state = off;
  off += al((size_t)N * H * K * V * 4);
  p->off_rec = off;
  p->rec_buf_bytes = (size_t)E * H * p->rec_bytes;
  off += 2 * p->rec_buf_bytes;
  p->total_bytes = off;
  return true;
}

template <int K, typename MT>
static hipError_t launch_chunk_t(const ChunkArgs& a, const ChunkPlan& pl) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  Entry* entries = reinterpret_cast<Entry*>(ws + pl.off_entries);
  int32_t* header = reinterpret_cast<int32_t*>(ws + pl.off_header);
  int32_t* seg_first = reinterpret_cast<int32_t*>(ws + pl.off_seg_first);
  int32_t* seg_count = reinterpret_cast<int32_t*>(ws + pl.off_seg_count);
  float* run_state = a.final_state ? a.final_state : reinterpret_cast<float*>(ws + pl.off_state);
  if ((int64_t)Rec<K, MT>::bytes != pl.rec_bytes) return hipErrorInvalidValue;

  SeqView sv{a.cu_seqlens, a.num_seqs, a.total_tokens};
  hipLaunchKernelGGL(table_kernel, dim3(a.num_seqs), dim3(256), 0, st, sv, a.num_heads,
                     (int64_t)a.dk * a.dv, pl.ub_entries, a.init_state, a.final_state, entries,
                     header);
  if (pl.num_segs == 0) return hipGetLastError();
  hipLaunchKernelGGL(segment_kernel, dim3(pl.num_segs), dim3(256), 0, st, entries, header,
                     pl.seg_entries, pl.slots, seg_first, seg_count);

  const int64_t chains = pl.slots * a.num_heads;
  const int64_t chains8 = (chains + 7) / 8 * 8;
  const dim3 sgrid((unsigned)(chains8 * pl.n_slices));
  const dim3 pgrid((unsigned)(pl.seg_entries * a.num_heads));
  for (int64_t s = 0; s < pl.num_segs; ++s) {
    char* rec = ws + pl.off_rec + (s & 1) * pl.rec_buf_bytes;
    PrepParams pp{a.q, a.k, a.g, a.beta, entries, header, a.num_heads, s * pl.seg_entries,
                  pl.seg_entries, rec, pl.rec_bytes};
    hipLaunchKernelGGL((prep_kernel<K, MT>), pgrid, dim3(NTHREADS), 0, st, pp);
    StateParams sp{a.v, a.o, a.init_state, run_state, entries, header,
                   seg_first + s * pl.slots, seg_count + s, s * pl.seg_entries, pl.seg_entries,
                   a.num_heads, a.dv, pl.n_slices, chains, rec, pl.rec_bytes};
    switch (pl.vs) {
      case 16: hipLaunchKernelGGL((state_kernel<K, 1, MT>), sgrid, dim3(NTHREADS), 0, st, sp); break;
      case 32: hipLaunchKernelGGL((state_kernel<K, 2, MT>), sgrid, dim3(NTHREADS), 0, st, sp); break;
      case 64: hipLaunchKernelGGL((state_kernel<K, 4, MT>), sgrid, dim3(NTHREADS), 0, st, sp); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkPlan& pl) {
  if (a.dtype_bf16) {
    if (a.dk == 32) return launch_chunk_t<32, bf16>(a, pl);
    if (a.dk == 64) return launch_chunk_t<64, bf16>(a, pl);
    if (a.dk == 128) return launch_chunk_t<128, bf16>(a, pl);
  } else {
    if (a.dk == 32) return launch_chunk_t<32, float>(a, pl);
    if (a.dk == 64) return launch_chunk_t<64, float>(a, pl);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
