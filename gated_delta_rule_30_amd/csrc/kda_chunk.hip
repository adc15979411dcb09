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
// in segments of about SEG_CHUNK_HEADS records so the record buffer stays resident in the
// Infinity Cache between the two kernels.
//
// Numerics. Inside a chunk every decay factor is formed relative to a 16-token sub-block
// reference so it stays in fp32 range: row factors e^{b_i - e_{I-1}} <= 1, column factors
// e^{e_J - b_j} <= 1 and per-channel block factors e^{e_{I-1} - e_J} <= 1 (J < I), with only
// the diagonal sub-block using e^{-(block decay)} >= 1 (the renormalisation the Technical
// Breakdown asks for in section 4's numerical-stability note). The solve runs in fp32 on
// VALU (diagonal 16x16 blocks) and fp32 MFMA (off-diagonal blocks). The state stays fp32.
#include <type_traits>

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
  static constexpr size_t bytes = (oGamBytes + K * 4 + 1023) / 1024 * 1024;  // whole 1 KB slots
};

template <typename MT>
__device__ __forceinline__ size_t slot_elem(int tile, int step, int lane, int L) {
  return ((size_t)(tile * (L / Mma<MT>::KS) + step) * 64 + lane) * Mma<MT>::EPL;
}

// four consecutive MT values from fp32
__device__ __forceinline__ void st4(bf16* p, f32x4 x) {
  *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector(x, bf16x4);
}
__device__ __forceinline__ void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  return __builtin_convertvector(*reinterpret_cast<const bf16x4*>(p), f32x4);
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// N consecutive elements of T <-> fp32, with one vector memory access (N * sizeof(T) bytes,
// naturally aligned).
template <typename T, int N>
struct VecN {
  typedef T vec __attribute__((ext_vector_type(N)));
  __device__ __forceinline__ static void load(const T* p, float* out) {
    const vec x = *reinterpret_cast<const vec*>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f32<T>(x[i]);
  }
  __device__ __forceinline__ static void store(T* p, const float* in) {
    vec x;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = from_f32<T>(in[i]);
    *reinterpret_cast<vec*>(p) = x;
  }
};

// Compile-time loop: f(std::integral_constant<int, I>()) for I = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// ====================================================================== chunk table
// Entries are ordered depth-major (chunk d of every sequence that has one, then chunk d+1),
// so one segment advances many sequences at once and short sequences drop out early. Within a
// depth, sequences are ordered by decreasing chunk count (ties by index). With r_n the rank of
// sequence n in that order, every sequence ranked before n has at least as many chunks, so
//     pos(n, d) = base[d] + r_n,   base[d] = sum_{n'} min(nc_{n'}, d),
// and a sequence's chunk indices follow from base[] alone, without walking the table.
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
                                                    int32_t* __restrict__ header,
                                                    int32_t* __restrict__ basetab) {
  const int n = blockIdx.x;
  const int64_t len = sv.len(n);
  const int64_t nc = sv.nchunks(n);
  // rank of n: sequences with more chunks, or as many and a smaller index, come first
  __shared__ int64_t red[256];
  int64_t rk = 0;
  for (int j = threadIdx.x; j < sv.num_seqs; j += blockDim.x) {
    const int64_t cj = sv.nchunks(j);
    rk += (cj > nc || (cj == nc && j < n)) ? 1 : 0;
  }
  red[threadIdx.x] = rk;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const int64_t rank = red[0];
  for (int64_t d = threadIdx.x; d < nc; d += blockDim.x) {
    int64_t base = 0, cnt = 0, cntm = 0;  // base[d], #{nc > d}, #{nc > d-1}
    for (int j = 0; j < sv.num_seqs; ++j) {
      const int64_t cj = sv.nchunks(j);
      base += min(cj, d);
      cnt += cj > d ? 1 : 0;
      cntm += cj > d - 1 ? 1 : 0;
    }
    const int64_t pos = base + rank;
    Entry en;
    en.seq = n;
    en.tok = (int32_t)(sv.start(n) + d * CHUNK);
    en.len = (int32_t)min((int64_t)CHUNK, len - d * CHUNK);
    en.depth = (int32_t)d;
    en.prev = d > 0 ? (int32_t)(base - cntm + rank) : -1;
    en.next = d + 1 < nc ? (int32_t)(base + cnt + rank) : -1;
    en.end = (int32_t)(sv.start(n) + len);
    en.pad = 0;
    if (pos < ub) entries[pos] = en;  // always true for a well-formed cu_seqlens
    if (rank == 0 && d <= ub) {       // the longest sequence has a chunk at every depth
      basetab[d] = (int32_t)base;
      if (d + 1 == nc && d + 1 <= ub) basetab[d + 1] = (int32_t)(base + cnt);
    }
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
constexpr int PREP_THREADS = 256;

// Sub-block pairs (I, J), J <= I, in the order (0,0) (1,0) (1,1) (2,0) ... (3,3).
__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I + 1) / 2 + J; }

// Lane m of each 16-lane row reads lane m - SH of the same row; lanes below SH read 0.
template <int SH>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + SH, 0xf, 0xf, true));
}

// A fragment (EPL elements) from fp32 values.
__device__ __forceinline__ bf16x8 to_frag(f32x4 lo, f32x4 hi, bf16) { return frag_from_acc(lo, hi, bf16()); }
__device__ __forceinline__ f32x4 to_frag(f32x4 lo, f32x4, float) { return lo; }

// LDS of one prep workgroup. Regions are reused across phases (each reuse follows a barrier
// after which the earlier contents are dead); the total stays under half the CU's LDS at
// K = 128 bf16 so that two workgroups share a CU.
template <int K, typename MT>
struct PrepLayout {
  static constexpr int PADM = 4;
  static constexpr int LC = CHUNK + PADM;    // MT rows of length CHUNK
  static constexpr int LCF = CHUNK + 4;      // fp32 rows of length CHUNK
  static constexpr int NPAIR = NSUB * (NSUB + 1) / 2;
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t szFrag = (size_t)CHUNK * K * sizeof(MT);  // [CHUNK][K] as fragments
  static constexpr int LDK = K + 16 / (int)sizeof(MT);                // MT rows of length K
  static constexpr size_t szKR = (size_t)CHUNK * LDK * sizeof(MT);    // [CHUNK][K], token-major
  static constexpr size_t szTri = (size_t)CHUNK * LC * sizeof(MT);  // [CHUNK][CHUNK]
  static constexpr size_t szAf = (size_t)CHUNK * LCF * 4;
  static constexpr size_t szTab = (size_t)(NSUB + NPAIR + NSUB) * K * 4;
  // X: Q^ and K^ fragments (phases 1-2); T' (phases 4-6)
  static constexpr size_t szX = mx(2 * szFrag, szTri);
  // R1: Ktilde staging (phase 1); A, then T (phases 2-4); W (phases 5-6)
  static constexpr size_t szR1 = mx(szKR, szAf);
  // P: block decays and per-channel factor tables (phases 1-2); -P^T (phases 2-6)
  static constexpr size_t szP = mx(szTri, szTab);
  static constexpr size_t oQh = 0, oKh = szFrag, oTb = 0;
  static constexpr size_t oR1 = szX;
  static constexpr size_t oKa = oR1 + szR1;  // Ka, token-major (phases 1-5)
  static constexpr size_t oP = oKa + szKR;
  static constexpr size_t oEx = oP + szP;     // e^{e_{J-1}} per block and channel (phases 1-6)
  static constexpr size_t oBeta = oEx + (size_t)NSUB * K * 4;
  static constexpr size_t total = oBeta + (size_t)CHUNK * 4;
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

// Record slot offset (elements) of the 4 consecutive reduction indices j0 .. j0+3 (j0 % 4 == 0)
// of row r in a matrix with reduction length L.
template <typename MT>
__device__ __forceinline__ size_t slot4(int r, int j0, int L) {
  constexpr int KS = Mma<MT>::KS;
  const int jj = j0 % KS;
  return slot_elem<MT>(r >> 4, j0 / KS, (r & 15) + 16 * ((jj & 15) >> 2), L) + 4 * (jj >> 4);
}

// One workgroup of 4 waves per (chunk, head); wave w owns sub-block w (tokens 16w .. 16w+15).
// Lane (m, g) = (lane % 16, lane / 16) holds token 16w + m and the channels 16u + 4g .. +3,
// u = 0 .. K/16-1, which is exactly that token's MFMA fragment over the channels. Phases are
// separated by LDS-only barriers; record stores stay in flight.
template <int K, typename MT>
__global__ __launch_bounds__(PREP_THREADS, 2) void prep_kernel(PrepParams p) {
  using L = PrepLayout<K, MT>;
  using R = Rec<K, MT>;
  using frag = typename Mma<MT>::frag;
  constexpr int KS = Mma<MT>::KS;
  constexpr int EPL = Mma<MT>::EPL;
  constexpr int NG = K / 16;     // 4-channel groups per lane
  constexpr int NS = K / KS;     // reduction steps over the channels
  constexpr int GPS = KS / 16;   // groups per reduction step
  constexpr int NKT = K / 16;
  constexpr int NPAIR = L::NPAIR;
  static_assert(L::total <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) char smem[L::total];
  MT* sQh = reinterpret_cast<MT*>(smem + L::oQh);
  MT* sKh = reinterpret_cast<MT*>(smem + L::oKh);
  MT* sTb = reinterpret_cast<MT*>(smem + L::oTb);
  MT* sKt = reinterpret_cast<MT*>(smem + L::oR1);
  float* sA = reinterpret_cast<float*>(smem + L::oR1);
  MT* sW = reinterpret_cast<MT*>(smem + L::oR1);
  MT* sKa = reinterpret_cast<MT*>(smem + L::oKa);
  float* sDel = reinterpret_cast<float*>(smem + L::oP);
  float* sD = sDel + NSUB * K;
  float* sTail = sD + NPAIR * K;
  MT* sPnT = reinterpret_cast<MT*>(smem + L::oP);
  float* sEx = reinterpret_cast<float*>(smem + L::oEx);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);

  const int H = p.H;
  const MT* gq_ = reinterpret_cast<const MT*>(p.q);
  const MT* gk_ = reinterpret_cast<const MT*>(p.k);
  const MT* gg_ = reinterpret_cast<const MT*>(p.g);
  const MT* gb_ = reinterpret_cast<const MT*>(p.beta);
  const int w = wave_id();
  const int t0 = 16 * w + (lane_id() & 15);  // this lane's token in the chunk
  const int g0 = lane_id() >> 4;

  // Persistent workgroups: task = (chunk j of the segment, head h) = (task / H, task % H). The
  // raw inputs of the next task are loaded while the current one is computed (phases 2-6).
  // (32-bit: a segment holds at most SEG_CHUNK_HEADS records)
  const int ntask = (int)min(p.E, (int64_t)p.header[0] - p.seg_begin) * H;
  using raw4 = typename VecN<MT, 4>::vec;
  struct Raw {
    raw4 q[NG], k[NG], g[NG];
    MT b;
  };
  // Rows past the chunk's end load the last valid row again; they are zeroed after conversion
  // (q = k = 0, log alpha = 0, beta = 0 there), so every load is unconditional.
  auto load_raw = [&](Raw& r, int task) {
    const int jt = task / H;
    const Entry en = p.entries[p.seg_begin + jt];
    const int hh = task - jt * H;
    const int64_t tl = en.tok + min(t0, en.len - 1);
    const int64_t row = tl * (int64_t)H * K + (int64_t)hh * K + 4 * g0;
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      r.q[u] = *reinterpret_cast<const raw4*>(gq_ + row + 16 * u);
      r.k[u] = *reinterpret_cast<const raw4*>(gk_ + row + 16 * u);
      r.g[u] = *reinterpret_cast<const raw4*>(gg_ + row + 16 * u);
    }
    r.b = gb_[tl * H + hh];
  };
  int task = blockIdx.x;
  if (task >= ntask) return;
  Raw cur, nxt;
  load_raw(cur, task);
#pragma clang loop unroll(disable)
  for (; task < ntask; task += gridDim.x) {
  // Lane-dependent addresses are recomputed in every iteration: without the opaque copy the
  // compiler hoists all of them out of the loop and keeps them live, which spills.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g = lane >> 4;
  const int t = 16 * w + m;
  const int j = task / H;
  const int h = task - j * H;
  const Entry en = p.entries[p.seg_begin + j];
  const int len = en.len;  // 1 .. CHUNK
  MT* recM = reinterpret_cast<MT*>(p.rec + (j * H + h) * p.rec_bytes);
  float* recGam = reinterpret_cast<float*>(p.rec + (j * H + h) * p.rec_bytes + R::oGamBytes);
  const bool valid = t < len;

  // ---------------- phase 1: the token's q, k and log2 alpha (fp32). Past the chunk's end only
  // log alpha (and beta) are zeroed: the q and k rows there repeat the last valid token and are
  // never used -- beta = 0 zeroes their rows of A, their columns of T' and P', and so their
  // rows of W and Delta -- while log alpha = 0 keeps the decay products of the valid tokens.
  float qv[NG][4], kv[NG][4], lv[NG][4];
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      qv[u][r] = to_f32(cur.q[u][r]);
      kv[u][r] = to_f32(cur.k[u][r]);
      lv[u][r] = valid ? to_f32(cur.g[u][r]) * LOG2E : 0.f;
    }
  const float bval = to_f32(cur.b);
  if (g == 0) sBeta[t] = valid ? bval : 0.f;
  // inclusive cumsum of log2 alpha over the 16 tokens of the sub-block (one 16-lane row):
  // lv becomes b_t - e_{w-1}; dI = e_w - e_{w-1} is the row's last value (log2 units)
  float dI[NG][4];
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = lv[u][r];
      x += row_shr<1>(x);
      x += row_shr<2>(x);
      x += row_shr<4>(x);
      x += row_shr<8>(x);
      lv[u][r] = x;
    }
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) dI[u][r] = __shfl(lv[u][r], lane | 15);
  if (m == 0) {
#pragma unroll
    for (int u = 0; u < NG; ++u)
      *reinterpret_cast<f32x4*>(sDel + w * K + 16 * u + 4 * g) = f32x4{dI[u][0], dI[u][1], dI[u][2], dI[u][3]};
  }
  lds_barrier();
  // per-channel factors, each computed once: e^{e_{J-1}} (sEx), gamma = e^{e_3} (record),
  // D_{IJ} = e^{e_{I-1} - e_J} <= 1 for I > J and e^{e_{J-1} - e_J} for I = J (sD), and
  // e^{e_3 - e_J} (sTail); e_J is the log decay from the chunk start to the end of block J
  {
    constexpr int NROLE = PREP_THREADS / K;
    const int c = tid % K, role = tid / K;
    float ec[NSUB + 1];
    ec[0] = 0.f;
#pragma unroll
    for (int J = 0; J < NSUB; ++J) ec[J + 1] = ec[J] + sDel[J * K + c];
#pragma unroll
    for (int v = 0; v < 2 * NSUB + 1 + NPAIR; ++v) {
      if (v % NROLE != role) continue;
      if (v < NSUB) {
        sEx[v * K + c] = exp2_f(ec[v]);
      } else if (v == NSUB) {
        recGam[c] = exp2_f(ec[NSUB]);
      } else if (v < NSUB + 1 + NPAIR) {
        const int pi = v - NSUB - 1;
        const int I = (pi >= 1) + (pi >= 3) + (pi >= 6);
        const int J = pi - I * (I + 1) / 2;
        sD[pi * K + c] = exp2_f((I == J ? ec[J] : ec[I]) - ec[J + 1]);
      } else {
        const int J = v - NSUB - 1 - NPAIR;
        sTail[J * K + c] = exp2_f(ec[NSUB] - ec[J + 1]);
      }
    }
  }
  lds_barrier();
  // decayed operands of the lane's token:
  //   Q^ = q e^{b_t - e_{w-1}}, K^ = k e^{b_t - e_{w-1}}  (<= 1 factors, MFMA row operands)
  //   kc = k e^{e_w - b_t}                                (<= 1, column operand, registers)
  //   qe = q e^{b_t}  (registers, for Q_eff),  Ka = k e^{b_t},  Kt = k e^{b_last - b_t}
  float qe[NG][4], kc[NG][4];
  {
    f32x4 qh[NG], kh[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const f32x4 ex = *reinterpret_cast<const f32x4*>(sEx + w * K + 16 * u + 4 * g);
      const f32x4 tl = *reinterpret_cast<const f32x4*>(sTail + w * K + 16 * u + 4 * g);
      f32x4 ka, kt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rr = exp2_f(lv[u][r]);
        const float cc = exp2_f(dI[u][r] - lv[u][r]);
        qh[u][r] = qv[u][r] * rr;
        kh[u][r] = kv[u][r] * rr;
        kc[u][r] = kv[u][r] * cc;
        qe[u][r] = qh[u][r] * ex[r];
        ka[r] = kh[u][r] * ex[r];
        kt[r] = kc[u][r] * tl[r];
      }
      st4(sKa + t * L::LDK + 16 * u + 4 * g, ka);
      st4(sKt + t * L::LDK + 16 * u + 4 * g, kt);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const size_t slot = ((size_t)(w * NS + s) * 64 + lane) * EPL;
      *reinterpret_cast<frag*>(sQh + slot) = to_frag(qh[GPS * s], qh[GPS * s + GPS - 1], MT());
      *reinterpret_cast<frag*>(sKh + slot) = to_frag(kh[GPS * s], kh[GPS * s + GPS - 1], MT());
    }
  }
  lds_barrier();
  // Ktilde^T (rows = channels, reduction = tokens) to the record as fragment slots
  {
    constexpr int NSL = NKT * (CHUNK / KS) * 64;
    static_assert(NSL % PREP_THREADS == 0, "slot split");
#pragma unroll
    for (int i = 0; i < NSL / PREP_THREADS; ++i) {
      const int sl = tid + PREP_THREADS * i;
      const int ln = sl & 63, ts = sl >> 6;
      const int s = ts % (CHUNK / KS), tile = ts / (CHUNK / KS);
      *reinterpret_cast<frag*>(recM + R::oKt + (size_t)sl * EPL) = frag_t(sKt, L::LDK, 16 * tile, s, ln);
    }
  }

  // the next task's inputs load during phases 2-6 (phase 1's fp32 copies are dead by now)
  load_raw(nxt, task + gridDim.x < ntask ? task + gridDim.x : task);

  // ---------------- phase 2: blocks (I, w), I >= w, of A and P. The column operand (token
  // block w, scaled per channel by D_{Iw}) is this wave's own kc; the row operands are read as
  // fragments. Results stay in registers until every wave is done with Q^, K^ and D.
  f32x4 tA[NSUB], tP[NSUB];
#pragma unroll
  for (int I = 0; I < NSUB; ++I) {
    tA[I] = f32x4{0.f, 0.f, 0.f, 0.f};
    tP[I] = tA[I];
    if (I < w) continue;
    const float* drow = sD + pair_index(I, w) * K + 4 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(drow + KS * s);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(drow + KS * s + 16 * (GPS - 1));
      f32x4 c0, c1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        c0[r] = kc[GPS * s][r] * d0[r];
        c1[r] = kc[GPS * s + GPS - 1][r] * d1[r];
      }
      const frag bfr = to_frag(c0, c1, MT());
      const size_t slot = ((size_t)(I * NS + s) * 64 + lane) * EPL;
      tA[I] = Mma<MT>::mma(*reinterpret_cast<const frag*>(sKh + slot), bfr, tA[I]);
      tP[I] = Mma<MT>::mma(*reinterpret_cast<const frag*>(sQh + slot), bfr, tP[I]);
    }
  }
  lds_barrier();
  // A (row-scaled by beta, strictly lower) -> sA for the off-diagonal blocks; -P (lower, upper
  // blocks zero) -> sPnT, transposed. The diagonal block A_ww stays in registers for phase 3(a).
  f32x4 adiag = tA[0];
#pragma unroll
  for (int I = 1; I < NSUB; ++I) adiag = (I == w) ? tA[I] : adiag;
  {
    const int jj = 16 * w + m;
#pragma unroll
    for (int I = 0; I < NSUB; ++I) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        if (I > w) sA[i * L::LCF + jj] = tA[I][r] * sBeta[i];
      }
      // -P^T row jj, columns 16I + 4g .. +3
      f32x4 pn;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        pn[r] = (I > w || (I == w && jj <= i)) ? -tP[I][r] : 0.f;
      }
      st4(sPnT + jj * L::LC + 16 * I + 4 * g, pn);
    }
  }

  // ---------------- phase 3: T = (I + A)^{-1}
  // (a) Diagonal 16x16 block of wave w by right-looking forward substitution: lane c keeps
  //     column c of T_ww; once row j is final, column j of A_ww updates rows i > j
  //     independently. A_ww is staged transposed in the wave's own diagonal block of sA, so
  //     column j is one broadcast row read; T_ww then overwrites it.
  {
    float* Ab = sA + (16 * w) * L::LCF + 16 * w;
    f32x4 a;  // lane (m, g): A_ww[4g + r][m] = A_ww^T[m][4g + r], beta-scaled, strictly lower
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      a[r] = (m < i) ? adiag[r] * sBeta[16 * w + i] : 0.f;
    }
    *reinterpret_cast<f32x4*>(Ab + m * L::LCF + 4 * g) = a;
    const int c = lane & 15;
    float x[SUBBLK];
#pragma unroll
    for (int i = 0; i < SUBBLK; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < SUBBLK - 1; ++j) {
      float col[SUBBLK];  // A_ww[.][j], the same in every lane
#pragma unroll
      for (int q = 0; q < SUBBLK / 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(Ab + j * L::LCF + 4 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) col[4 * q + r] = v[r];
      }
#pragma unroll
      for (int i = j + 1; i < SUBBLK; ++i) x[i] -= col[i] * x[j];
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < SUBBLK; ++i) Ab[i * L::LCF + c] = x[i];
    }
  }
  lds_barrier();
  // (b) Off-diagonal blocks of row block I = w, right to left, with no further barrier:
  //     T_IJ = -(sum_{M=J+1}^{I} T_IM A_MJ) T_JJ, computed transposed so that every operand
  //     is a column read, a row read or the previous result tile. T_IJ (I > J) is stored
  //     row-major in the unused upper block (J, I) of sA.
  if (w >= 1) {
    const int Ib = w;
    auto tblock = [&](int I, int M) -> float* {  // base of T_IM (I >= M)
      return (I == M) ? sA + (16 * I) * L::LCF + 16 * I : sA + (16 * M) * L::LCF + 16 * I;
    };
    for (int J = Ib - 1; J >= 0; --J) {
      f32x4 X = {0.f, 0.f, 0.f, 0.f};  // X^T = sum_M A_MJ^T T_IM^T
      for (int M = J + 1; M <= Ib; ++M) {
        f32x4 af;
#pragma unroll
        for (int r = 0; r < 4; ++r) af[r] = sA[(16 * M + 4 * g + r) * L::LCF + 16 * J + m];
        const f32x4 bf = *reinterpret_cast<const f32x4*>(tblock(Ib, M) + m * L::LCF + 4 * g);
        X = Mma<float>::mma(af, bf, X);
      }
      f32x4 tjj;
#pragma unroll
      for (int r = 0; r < 4; ++r) tjj[r] = sA[(16 * J + 4 * g + r) * L::LCF + 16 * J + m];
      const f32x4 Y = Mma<float>::mma(tjj, X, f32x4{0.f, 0.f, 0.f, 0.f});  // (T_IJ)^T
      *reinterpret_cast<f32x4*>(tblock(Ib, J) + m * L::LCF + 4 * g) = -Y;
    }
  }
  lds_barrier();

  // ---------------- phase 4: T' = T diag(beta) -> LDS (row-major and transposed) and record
#pragma unroll
  for (int it = 0; it < CHUNK * CHUNK / 4 / PREP_THREADS; ++it) {
    const int idx = tid + PREP_THREADS * it;
    const int i = idx / (CHUNK / 4), j0 = 4 * (idx % (CHUNK / 4));
    const int Ii = i >> 4, Jj = j0 >> 4;
    const int src = (Ii == Jj) ? i * L::LCF + j0 : (16 * Jj + (i & 15)) * L::LCF + 16 * Ii + (j0 & 15);
    f32x4 tv = *reinterpret_cast<const f32x4*>(sA + src);
    tv *= *reinterpret_cast<const f32x4*>(sBeta + j0);
    if (Ii < Jj) tv = f32x4{0.f, 0.f, 0.f, 0.f};
    st4(sTb + i * L::LC + j0, tv);
    st4(recM + R::oTb + slot4<MT>(i, j0, CHUNK), tv);
  }
  lds_barrier();

  // ---------------- phase 5: W^T = Ka^T T'^T -> record (as W fragments) and LDS (W^T)
#pragma unroll
  for (int tix = 0; tix < NKT * NSUB; ++tix) {
    const int a = tix % NKT, b = tix / NKT;
    if (tix % 4 != w) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int nsteps = (16 * b + 16 + KS - 1) / KS;
#pragma unroll
    for (int s = 0; s < CHUNK / KS; ++s)
      if (s < nsteps)
        acc = Mma<MT>::mma(frag_t(sKa, L::LDK, 16 * a, s, lane),
                           load_frag(sTb + (16 * b + m) * L::LC, s, g), acc);
    st4(recM + R::oW + slot4<MT>(16 * b + m, 16 * a + 4 * g, K), acc);
    st4(sW + (16 * b + m) * L::LDK + 16 * a + 4 * g, acc);  // W row 16b + m
  }
  lds_barrier();

  // ---------------- phase 6a: Q_eff^T = (Q e^{b})^T + W^T (-P)^T, column tile b = w. The
  // accumulator starts from this lane's own q e^{b_t} (token 16w + m, channels 16a + 4g + r).
  {
    const int nsteps = (16 * w + 16 + KS - 1) / KS;
#pragma unroll
    for (int a = 0; a < NKT; ++a) {
      f32x4 acc = {qe[a][0], qe[a][1], qe[a][2], qe[a][3]};
#pragma unroll
      for (int s = 0; s < CHUNK / KS; ++s)
        if (s < nsteps)
          acc = Mma<MT>::mma(frag_t(sW, L::LDK, 16 * a, s, lane), frag_t(sPnT, L::LC, 16 * w, s, lane), acc);
      st4(recM + R::oQ + slot4<MT>(16 * w + m, 16 * a + 4 * g, K), acc);
    }
  }
  // ---------------- phase 6b: P'^T = -(T'^T (-P)^T) -> record (as P' fragments); column tile a = w
#pragma unroll
  for (int b = 0; b < NSUB; ++b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (w <= b) {
      const int nsteps = (16 * b + 16 + KS - 1) / KS;
#pragma unroll
      for (int s = 0; s < CHUNK / KS; ++s)
        if (s < nsteps)
          acc = Mma<MT>::mma(frag_t(sTb, L::LC, 16 * w, s, lane), frag_t(sPnT, L::LC, 16 * b, s, lane), acc);
      acc = -acc;
    }
    st4(recM + R::oPb + slot4<MT>(16 * b + m, 16 * w + 4 * g, CHUNK), acc);
  }
  lds_barrier();  // the next task reuses every LDS region
  cur = nxt;
  }
}

// ====================================================================== STATE kernel
// One workgroup of 4 waves per (sequence run, head, V-slice of VS = 16*NVT columns). The state
// GEMMs are computed transposed, with the chunk record as the B operand:
//   U^T = V^T T'^T,  (P'V)^T = V^T P'^T,  (W S)^T = S^T W^T,  (Q_eff S)^T = S^T Q_eff^T,
//   S'^T = S^T Diag(gamma) + Delta^T Ktilde
// so the record's fragment slots feed the matrix cores as loaded, and a result tile holds four
// consecutive V columns of one token (output, Delta) or of one key channel (state) per lane.
// Wave w owns token tile w (U, P'V, W S, Q_eff S, Delta, O for every column tile) and
// key-channel tiles w, w+4 of the state update, so each record byte is loaded once per
// workgroup, straight into registers, one chunk ahead of its use.
//
// S, V and Delta sit in LDS row-major (rows = key channel or token, VS columns), written with
// 8- and 16-byte stores straight from the result layout; the A fragments of S^T, V^T and
// Delta^T are read back with the transposing LDS read (bf16) or four scalar reads (fp32).
template <int K, int NVT, typename MT>
struct StateLayout {
  static constexpr int VS = 16 * NVT;
  static constexpr int LD = VS + 16 / (int)sizeof(MT);  // row length in elements (16-byte aligned rows)
  static constexpr size_t oS = 0;                                      // S: [K][VS]
  static constexpr size_t oV = oS + (size_t)K * LD * sizeof(MT);       // V: [CHUNK][VS]
  static constexpr size_t oD = oV + (size_t)CHUNK * LD * sizeof(MT);   // Delta: [CHUNK][VS]
  static constexpr size_t oRun = oD + (size_t)CHUNK * LD * sizeof(MT);
  static constexpr size_t total = oRun + (SEG_CHUNK_HEADS + 16) * 4;
  static_assert((LD * sizeof(MT)) % 16 == 0, "row alignment");
};

struct StateParams {
  const void* v;
  void* o;
  const float* init_state;
  float* state;  // running and final state [N][H][K][V]
  const Entry* entries;
  const int32_t* header;
  const int32_t* basetab;    // base[d] of the chunk table
  const int32_t* seg_first;  // this segment's list
  const int32_t* seg_count;  // this segment's count
  int64_t seg_begin, E;
  int H, V, n_slices;
  int64_t chains;  // slots * H
  const char* rec;
  int64_t rec_bytes;
  char* trash;  // >= 1 KB sink for output rows past a chunk's end
};

constexpr int STATE_THREADS = 256;

// What one wave loads for one chunk.
template <int K, int NVT, typename MT>
struct StateBundle {
  using frag = typename Mma<MT>::frag;
  static constexpr int KS = Mma<MT>::KS;
  static constexpr int NKT = K / 16;
  static constexpr int TPW = (NKT + 3) / 4;  // key-channel tiles per wave
  static constexpr int VE = 4 * NVT;         // V elements per lane: one token, VE columns
  frag tf[CHUNK / KS], pf[CHUNK / KS], wf[K / KS], qf[K / KS], kf[TPW][CHUNK / KS];
  float gam[TPW];
  typename VecN<MT, VE>::vec v;
};

template <int K, int NVT, typename MT>
__global__ __launch_bounds__(STATE_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void state_kernel(StateParams p) {
  using SL = StateLayout<K, NVT, MT>;
  using R = Rec<K, MT>;
  using B = StateBundle<K, NVT, MT>;
  using frag = typename Mma<MT>::frag;
  using vvec = typename VecN<MT, B::VE>::vec;
  constexpr int KS = Mma<MT>::KS;
  constexpr int VS = SL::VS;
  constexpr int LD = SL::LD;
  constexpr int NKT = B::NKT;
  constexpr int TPW = B::TPW;
  constexpr int VE = B::VE;
  static_assert(SL::total <= 64 * 1024, "state LDS budget");
  __shared__ __align__(16) char smem[SL::total];
  MT* sS = reinterpret_cast<MT*>(smem + SL::oS);
  MT* sV = reinterpret_cast<MT*>(smem + SL::oV);
  MT* sD = reinterpret_cast<MT*>(smem + SL::oD);
  int32_t* sRun = reinterpret_cast<int32_t*>(smem + SL::oRun);
  int32_t* sLen = sRun + SEG_CHUNK_HEADS;

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
  const int64_t e0 = p.seg_first[slot];
  const Entry en = p.entries[e0];
  const int col0 = slice * VS;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = lane_id();
  const int m = lane & 15;
  const int g = lane >> 4;

  // This workgroup's run: chunks d0, d0+1, ... of sequence en.seq inside the segment. Chunk
  // d0+k is entry base[d0+k] + rank; the run ends at the sequence's end or the segment's end.
  const int seq_start = en.tok - CHUNK * en.depth;
  const int nc = (en.end - seq_start + CHUNK - 1) / CHUNK;
  const int64_t rank = e0 - p.basetab[en.depth];
  const int kmax = (int)min((int64_t)(nc - en.depth), p.E);
  if (tid == 0) sLen[0] = kmax;
  __syncthreads();
  for (int k = tid; k < kmax; k += STATE_THREADS) {
    const int64_t ek = p.basetab[en.depth + k] + rank;
    sRun[k] = (int32_t)(ek - p.seg_begin);
    if (ek >= seg_end) atomicMin(&sLen[0], k);
  }

  // State tiles (nt, kt = w + 4 tt): lane (m, g) holds S[16kt + m][16nt + 4g .. +3] of the slice.
  const size_t sbase = ((size_t)en.seq * H + h) * (size_t)K * V + col0;
  const float* src = (en.depth == 0) ? p.init_state : p.state;
  f32x4 Sr[TPW][NVT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int kt = w + 4 * tt;
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (kt < NKT && src != nullptr)
        x = *reinterpret_cast<const f32x4*>(src + sbase + (size_t)(16 * kt + m) * V + 16 * nt + 4 * g);
      Sr[tt][nt] = x;
      if (kt < NKT) st4(sS + (16 * kt + m) * LD + 16 * nt + 4 * g, x);
    }
  }
  __syncthreads();
  const int run = sLen[0];

  const MT* gv = reinterpret_cast<const MT*>(p.v) + (int64_t)h * V + col0;
  MT* go = reinterpret_cast<MT*>(p.o) + (int64_t)h * V + col0;
  MT* trash = reinterpret_cast<MT*>(p.trash) + 4 * lane;
  const int64_t vrow = (int64_t)H * V;
  const char* rec_h = p.rec + (int64_t)h * p.rec_bytes;
  const int64_t rec_stride = (int64_t)H * p.rec_bytes;
  auto tok_of = [&](int k) { return seq_start + CHUNK * (en.depth + k); };
  auto len_of = [&](int k) { return min(CHUNK, en.end - tok_of(k)); };

  // Loop-invariant per-lane byte offsets inside a record; a chunk's loads then use one
  // wave-uniform base address plus these offsets (reduction steps are 1 KB apart).
  constexpr uint32_t STEP = 64 * 16;
  const uint32_t lo_t = (uint32_t)((R::oTb + slot_elem<MT>(w, 0, lane, CHUNK)) * sizeof(MT));
  const uint32_t lo_p = (uint32_t)((R::oPb + slot_elem<MT>(w, 0, lane, CHUNK)) * sizeof(MT));
  const uint32_t lo_w = (uint32_t)((R::oW + slot_elem<MT>(w, 0, lane, K)) * sizeof(MT));
  const uint32_t lo_q = (uint32_t)((R::oQ + slot_elem<MT>(w, 0, lane, K)) * sizeof(MT));
  uint32_t lo_k[TPW], lo_g[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int kt = min(w + 4 * tt, NKT - 1);
    lo_k[tt] = (uint32_t)((R::oKt + slot_elem<MT>(kt, 0, lane, CHUNK)) * sizeof(MT));
    lo_g[tt] = (uint32_t)(R::oGamBytes + (16 * kt + m) * 4);
  }
  auto ldf = [](const char* base, uint32_t off) -> frag { return *reinterpret_cast<const frag*>(base + off); };

  // Loads of chunk k (clamped to the run's last chunk; a duplicate load past the end is never
  // used). The V row of a token past the chunk's end repeats the last valid row and is zeroed
  // when staged, so every load is unconditional. Load i of the record part is piece(b, rc, i).
  constexpr int NTS = CHUNK / KS, NKS = K / KS;
  constexpr int NLOADS = 2 * NTS + 2 * NKS + TPW * (NTS + 1);
  auto rec_of = [&](int k) {
    const int kk = min(k, run - 1);
    const int ri = __builtin_amdgcn_readfirstlane(sRun[kk]);  // uniform record index
    return rec_h + (int64_t)ri * rec_stride;
  };
  auto load_v = [&](B& b, int k) {
    const int kk = min(k, run - 1);
    const int tok = tok_of(kk), len = len_of(kk);
    b.v = *reinterpret_cast<const vvec*>(gv + ((int64_t)tok + min(lane, len - 1)) * vrow + VE * w);
  };
  auto piece = [&](B& b, const char* rc, auto I) {
    constexpr int i = decltype(I)::value;
    if constexpr (i < NTS) {
      b.tf[i] = ldf(rc, lo_t + STEP * i);
    } else if constexpr (i < 2 * NTS) {
      b.pf[i - NTS] = ldf(rc, lo_p + STEP * (i - NTS));
    } else if constexpr (i < 2 * NTS + NKS) {
      b.wf[i - 2 * NTS] = ldf(rc, lo_w + STEP * (i - 2 * NTS));
    } else if constexpr (i < 2 * NTS + 2 * NKS) {
      b.qf[i - 2 * NTS - NKS] = ldf(rc, lo_q + STEP * (i - 2 * NTS - NKS));
    } else {
      constexpr int j = i - 2 * NTS - 2 * NKS, tt = j / (NTS + 1), s = j % (NTS + 1);
      if constexpr (s < NTS) b.kf[tt][s] = ldf(rc, lo_k[tt] + STEP * s);
      else b.gam[tt] = *reinterpret_cast<const float*>(rc + lo_g[tt]);
    }
  };
  auto issue_all = [&](B& b, int k) {
    load_v(b, k);
    __builtin_amdgcn_sched_barrier(0);
    const char* rc = rec_of(k);
    static_for<0, NLOADS>([&](auto I) { piece(b, rc, I); });
  };

  // V of chunk k into LDS: lane = token, wave w = columns VE*w .. +VE-1
  auto stage = [&](const B& b, int k) {
    const bool valid = lane < len_of(k);
    vvec x = b.v;
#pragma unroll
    for (int i = 0; i < VE; ++i) x[i] = valid ? x[i] : from_f32<MT>(0.f);
    *reinterpret_cast<vvec*>(sV + lane * LD + VE * w) = x;
  };

  // Chunk k for token tile w: U, P'V, W S, Q_eff S (Delta to LDS, O to memory), with the loads
  // of chunk k+1 spread between the matrix operations. The loads go through the CU's
  // vector-memory path at about 64 B per clock and a wave waits at a load until that path
  // accepts it, so one load follows each MFMA instead of all loads going out in one burst; the
  // scheduling barriers keep that order. Branch-free: the record holds zeros above the
  // diagonal of T' and P', so every reduction step runs.
  // MFMA j: reduction step s = j / (2 NVT) of U, P'V (j < NMF_T), then of W S, Q_eff S,
  // round-robin over the independent accumulators.
  constexpr int NMF_T = 2 * NVT * NTS, NMF_K = 2 * NVT * NKS, NMF = NMF_T + NMF_K;
  constexpr int NLC = 2 * NTS + 2 * NKS;  // pieces loaded during compute: T', P', W, Q_eff
  constexpr int LSTRIDE = NMF / NLC;      // MFMAs per piece
  static_assert(LSTRIDE >= 1, "one load per MFMA at most");
  f32x4 Opend[NVT];
  MT* Odst[NVT];
  auto compute = [&](const B& b, B& nxt, int k) {
    const int tok = tok_of(k), len = len_of(k);
    const int t = 16 * w + m;
    // fragments of reduction step s: V^T (s < NTS) and S^T (s < NKS), read one step ahead
    frag vf[2][NVT], sf[2][NVT];
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) {
      vf[0][nt] = frag_t(sV, LD, 16 * nt, 0, lane);
      sf[0][nt] = frag_t(sS, LD, 16 * nt, 0, lane);
    }
    load_v(nxt, k + 1);
    const char* rc = rec_of(k + 1);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 U[NVT], Ol[NVT], Y[NVT], Z[NVT];
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) U[nt] = Ol[nt] = Y[nt] = Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, NMF>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int s = j < NMF_T ? j / (2 * NVT) : (j - NMF_T) / (2 * NVT);
      constexpr bool first_of_step = (j < NMF_T ? j % (2 * NVT) : (j - NMF_T) % (2 * NVT)) == 0;
      if constexpr (first_of_step && j < NMF_T && s + 1 < NTS) {
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) vf[(s + 1) & 1][nt] = frag_t(sV, LD, 16 * nt, s + 1, lane);
      }
      if constexpr (first_of_step && j >= NMF_T && s + 1 < NKS) {
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) sf[(s + 1) & 1][nt] = frag_t(sS, LD, 16 * nt, s + 1, lane);
      }
      if constexpr (j < NMF_T) {
        constexpr int nt = (j % (2 * NVT)) / 2;
        if constexpr (j % 2 == 0) U[nt] = Mma<MT>::mma(vf[s & 1][nt], b.tf[s], U[nt]);
        else Ol[nt] = Mma<MT>::mma(vf[s & 1][nt], b.pf[s], Ol[nt]);
      } else {
        constexpr int jj = j - NMF_T, nt = (jj % (2 * NVT)) / 2;
        if constexpr (jj % 2 == 0) Y[nt] = Mma<MT>::mma(sf[s & 1][nt], b.wf[s], Y[nt]);
        else Z[nt] = Mma<MT>::mma(sf[s & 1][nt], b.qf[s], Z[nt]);
      }
      if constexpr (j % LSTRIDE == 0 && j / LSTRIDE < NLC)
        piece(nxt, rc, std::integral_constant<int, j / LSTRIDE>());
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) {
      st4(sD + t * LD + 16 * nt + 4 * g, U[nt] - Y[nt]);
      Opend[nt] = Ol[nt] + Z[nt];
      Odst[nt] = t < len ? go + ((int64_t)tok + t) * vrow + 16 * nt + 4 * g : trash;
    }
  };

  // S'^T = S^T Diag(gamma) + Delta^T Ktilde for key-channel tiles w, w+4
  auto update = [&](const B& b, B& nxt, int k) {
    {
      const char* rc = rec_of(k + 1);
      static_for<NLC, NLOADS>([&](auto I) { piece(nxt, rc, I); });
    }
    frag df[NVT][NTS];
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
      for (int s = 0; s < NTS; ++s) df[nt][s] = frag_t(sD, LD, 16 * nt, s, lane);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int kt = w + 4 * tt;
      if (kt < NKT) {
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) {
          f32x4 acc = Sr[tt][nt] * b.gam[tt];
#pragma unroll
          for (int s = 0; s < NTS; ++s) acc = Mma<MT>::mma(df[nt][s], b.kf[tt][s], acc);
          Sr[tt][nt] = acc;
          st4(sS + (16 * kt + m) * LD + 16 * nt + 4 * g, acc);
        }
      }
    }
    // the output rows of chunk k leave after the update, behind the loads issued above
#pragma unroll
    for (int nt = 0; nt < NVT; ++nt) st4(Odst[nt], Opend[nt]);
  };

  // Two register bundles in turn: chunk k+1's loads are issued while chunk k is computed. The
  // second half differs from the first (an extra scheduling barrier) so that the compiler keeps
  // both halves instead of folding them into one with register copies between bundles.
  auto chunk = [&](const B& cur, B& nxt, int k, auto PAR) {
    stage(cur, k);
    lds_barrier();  // V and S of chunk k ready
    compute(cur, nxt, k);
    if constexpr (decltype(PAR)::value) __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // Delta complete; S and V no longer read
    update(cur, nxt, k);
  };
  B b0, b1;
  issue_all(b0, 0);
  for (int k = 0; k < run; k += 2) {
    chunk(b0, b1, k, std::false_type());
    if (k + 1 >= run) break;
    chunk(b1, b0, k + 1, std::true_type());
  }

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int kt = w + 4 * tt;
    if (kt < NKT) {
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
        *reinterpret_cast<f32x4*>(p.state + sbase + (size_t)(16 * kt + m) * V + 16 * nt + 4 * g) = Sr[tt][nt];
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
  p->rec_bytes = ((3LL * CHUNK * K + 2LL * CHUNK * CHUNK) * es + 4LL * K + 1023) / 1024 * 1024;
  // V split: slices of 32 columns, one 4-wave workgroup each
  p->n_slices = V / 32;
  p->vs = 32;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p->off_header = off;
  off += 256;
  p->off_entries = off;
  off += al((size_t)ub * sizeof(Entry));
  p->off_basetab = off;
  off += al((size_t)(ub + 1) * 4);
  p->off_seg_first = off;
  off += al((size_t)p->num_segs * p->slots * 4);
  p->off_seg_count = off;
  off += al((size_t)p->num_segs * 4);
  p->off_state = off;
  off += al((size_t)N * H * K * V * 4);
  p->off_sink = off;  // 1 KB sink for output rows past a chunk's end
  off += 1024;
  p->off_rec = off;
  p->rec_buf_bytes = (size_t)E * H * p->rec_bytes;
  off += p->rec_buf_bytes;
  p->total_bytes = off;
  return true;
}

template <int K, typename MT>
static hipError_t launch_chunk_t(const ChunkArgs& a, const ChunkPlan& pl) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  Entry* entries = reinterpret_cast<Entry*>(ws + pl.off_entries);
  int32_t* header = reinterpret_cast<int32_t*>(ws + pl.off_header);
  int32_t* basetab = reinterpret_cast<int32_t*>(ws + pl.off_basetab);
  int32_t* seg_first = reinterpret_cast<int32_t*>(ws + pl.off_seg_first);
  int32_t* seg_count = reinterpret_cast<int32_t*>(ws + pl.off_seg_count);
  float* run_state = a.final_state ? a.final_state : reinterpret_cast<float*>(ws + pl.off_state);
  if ((int64_t)Rec<K, MT>::bytes != pl.rec_bytes) return hipErrorInvalidValue;

  SeqView sv{a.cu_seqlens, a.num_seqs, a.total_tokens};
  hipLaunchKernelGGL(table_kernel, dim3(a.num_seqs), dim3(256), 0, st, sv, a.num_heads,
                     (int64_t)a.dk * a.dv, pl.ub_entries, a.init_state, a.final_state, entries,
                     header, basetab);
  if (pl.num_segs == 0) return hipGetLastError();
  hipLaunchKernelGGL(segment_kernel, dim3(pl.num_segs), dim3(256), 0, st, entries, header,
                     pl.seg_entries, pl.slots, seg_first, seg_count);

  const int64_t chains = pl.slots * a.num_heads;
  const int64_t chains8 = (chains + 7) / 8 * 8;
  const dim3 sgrid((unsigned)(chains8 * pl.n_slices));
  // prep: persistent workgroups, two per CU (its LDS and register budget), looping over tasks
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  const int64_t ptasks = pl.seg_entries * a.num_heads;
  const dim3 pgrid((unsigned)min(ptasks, (int64_t)2 * ncu));
  auto prep = [&](int64_t s, hipStream_t q) {
    char* rec = ws + pl.off_rec;
    PrepParams pp{a.q, a.k, a.g, a.beta, entries, header, a.num_heads, s * pl.seg_entries,
                  pl.seg_entries, rec, pl.rec_bytes};
    hipLaunchKernelGGL((prep_kernel<K, MT>), pgrid, dim3(PREP_THREADS), 0, q, pp);
  };
  auto state = [&](int64_t s, hipStream_t q) -> bool {
    const char* rec = ws + pl.off_rec;
    StateParams sp{a.v, a.o, a.init_state, run_state, entries, header, basetab,
                   seg_first + s * pl.slots, seg_count + s, s * pl.seg_entries, pl.seg_entries,
                   a.num_heads, a.dv, pl.n_slices, chains, rec, pl.rec_bytes,
                   ws + pl.off_sink};
    if (pl.vs != 32) return false;
    hipLaunchKernelGGL((state_kernel<K, 2, MT>), sgrid, dim3(STATE_THREADS), 0, q, sp);
    return true;
  };

  // Segments run in order on the caller's stream, each kernel with the whole device: the
  // prep kernel fills the record buffer, then the state kernel consumes it.
  for (int64_t s = 0; s < pl.num_segs; ++s) {
    prep(s, st);
    if (!state(s, st)) return hipErrorInvalidValue;
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
