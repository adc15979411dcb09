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
//   O     = (Q * e^{b}) S + P Delta                                   read after the write
//   S'    = Diag(e^{b_last}) S + (K * e^{b_last - b})^T Delta          state passing
// The WY / UT form of the chunk's rank-1 updates and the triangular solve follow the pages'
// description ("Kimi Linear" explainer, "WY Representation"; wpnews article, DPLR paragraph).
//
// Execution. Work that does not depend on the state is independent per (chunk, head) and runs
// in the chunk-parallel PREP kernel, which writes one compact record per (chunk, head): -W,
// Qe = Q * e^{b}, Ktilde^T, T', P (bf16 MFMA fragments) and e^{b_last}. The STATE kernel walks each sequence's chunks in order, one
// wave per (sequence, head, 16-column V-slice) -- the columns of S evolve independently, so
// the V split is exact -- and does only U = T'V, Delta = U - W S, O = Qe S + P Delta and the
// update S' = Diag(gamma) S + Ktilde^T Delta on the matrix cores. The sequence is processed
// in segments of about SEG_CHUNK_HEADS records so the record buffer stays resident in the
// Infinity Cache between the two kernels.
//
// Numerics. Inside a chunk every decay factor is formed relative to a 16-token sub-block
// reference so it stays in fp32 range: row factors e^{b_i - e_{I-1}} <= 1, column factors
// e^{e_J - b_j} <= 1 and per-channel block factors e^{e_{I-1} - e_J} <= 1 (J < I) (the
// renormalisation the Technical Breakdown asks for in section 4's numerical-stability note).
// A diagonal sub-block uses the column factor e^{-(block decay)} >= 1 only while every
// channel's decay over its 16 tokens stays within 2^96; a stronger decay forms that block from
// running products of the per-token decays instead, so any log alpha <= 0 gives finite
// results. The solve runs in fp32 on VALU (diagonal 16x16 blocks) and fp32 MFMA (off-diagonal
// blocks). The state stays fp32.
#include <atomic>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

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

// ====================================================================== chunk table
// Two orders, chosen per call from the head count (ChunkPlan::seq_major):
//  - depth-major (chunk d of every sequence that has one, then chunk d+1): one segment
//    advances many sequences at once and short sequences drop out early, which keeps the chip
//    busy when one sequence's chains (H heads x V/16 slices) are few. Within a depth,
//    sequences are ordered by decreasing chunk count (ties by index). With r_n the rank of
//    sequence n in that order, every sequence ranked before n has at least as many chunks, so
//        pos(n, d) = base[d] + r_n,   base[d] = sum_{n'} min(nc_{n'}, d),
//    and a sequence's chunk indices follow from base[] alone, without walking the table;
//  - sequence-major (token order): pos(n, d) = sum_{n' < n} nc_{n'} + d. Where one sequence's
//    chains fill the chip by themselves, a segment then holds long runs of one or two
//    sequences instead of E / N chunks of each of N, and a chain pays its start (state load,
//    the first chunk's record loads) once per segment rather than once every few chunks.
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
                                                    int32_t* __restrict__ basetab, int seq_major) {
  const int n = blockIdx.x;
  const int64_t len = sv.len(n);
  const int64_t nc = sv.nchunks(n);
  // depth-major: the rank of n (sequences with more chunks, or as many and a smaller index,
  // come first); sequence-major: the chunks of the sequences before n
  __shared__ int64_t red[256];
  int64_t rk = 0;
  for (int j = threadIdx.x; j < sv.num_seqs; j += blockDim.x) {
    const int64_t cj = sv.nchunks(j);
    if (seq_major) rk += j < n ? cj : 0;
    else rk += (cj > nc || (cj == nc && j < n)) ? 1 : 0;
  }
  red[threadIdx.x] = rk;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const int64_t rank = red[0];
  if (seq_major) {
    for (int64_t d = threadIdx.x; d < nc; d += blockDim.x) {
      const int64_t pos = rank + d;
      Entry en;
      en.seq = n;
      en.tok = (int32_t)(sv.start(n) + d * CHUNK);
      en.len = (int32_t)min((int64_t)CHUNK, len - d * CHUNK);
      en.depth = (int32_t)d;
      en.prev = d > 0 ? (int32_t)(pos - 1) : -1;
      en.next = d + 1 < nc ? (int32_t)(pos + 1) : -1;
      en.end = (int32_t)(sv.start(n) + len);
      en.pad = 0;
      if (pos < ub) entries[pos] = en;  // always true for a well-formed cu_seqlens
    }
  }
  for (int64_t d = threadIdx.x; d < (seq_major ? 0 : nc); d += blockDim.x) {
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
    int x = (int)threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
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
// Largest decay (log2 units) of a key channel over one 16-token sub-block for which the
// diagonal sub-block is formed on the matrix cores (its column factor is at most 2^this).
constexpr float DIAG_MAX_LOG2 = 96.f;

// Sub-block pairs (I, J), J <= I, in the order (0,0) (1,0) (1,1) (2,0) ... (3,3).
__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I + 1) / 2 + J; }

// Lane m of each 16-lane row reads lane m - SH of the same row; lanes below SH read 0.
template <int SH>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + SH, 0xf, 0xf, true));
}
// Issue priority of the calling wave (0 .. 3; s_setprio takes an immediate).
__device__ __forceinline__ void wave_prio(int p) {
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}
// The value of lane 15 of each 16-lane row, in every lane of that row (DPP row_newbcast:15).
__device__ __forceinline__ float row_last(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xf, 0xf, false));
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
  uint32_t opts;      // input option bits (OPT_*)
  const void* v;      // V [T][H][V], copied into the records slice-major
  int V;
};

// One workgroup of 4 waves per (chunk, head); wave w owns sub-block w (tokens 16w .. 16w+15).
// Lane (m, g) = (lane % 16, lane / 16) holds token 16w + m and the channels 16u + 4g .. +3,
// u = 0 .. K/16-1, which is exactly that token's MFMA fragment over the channels. Phases are
// separated by LDS-only barriers; record stores stay in flight.
// OPTS = false compiles the kernel without the input-option code (options == 0), which keeps
// that path's register allocation and schedule free of it. V256 = true fixes a token row of V
// at 256 bytes (bf16 V = 128, fp32 V = 64): the V copy is then one branch-free batch (at the
// join points of the generic copy's batch branches the compiler waits for all memory traffic).
// UREC = true (bf16, V = 128) writes the record's U form: U = T'V formed here, on the matrix
// cores from V staged in LDS, in place of T' and V.
template <int K, typename MT, bool OPTS, bool V256, bool UREC = false>
__global__ __launch_bounds__(PREP_THREADS, 2) void prep_kernel(PrepParams p) {
  static_assert(!UREC || (V256 && sizeof(MT) == 2 && K <= 128), "the U form: bf16, V = 128");
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
  // first token and length of a task's chunk (read one task ahead: the prefetch addresses
  // depend on them, and a load issued only there would stall every part of the prefetch)
  struct TaskPos {
    int tok, len;
  };
  auto task_pos = [&](int tk) -> TaskPos {
    const Entry* e = p.entries + p.seg_begin + tk / H;
    return TaskPos{e->tok, e->len};
  };
  // Rows past the chunk's end load the last valid row again; they are zeroed after conversion
  // (q = k = 0, log alpha = 0, beta = 0 there), so every load is unconditional.
  // part 0: q; part 1: k; part 2: log alpha and beta; part -1: everything. A scalar gate (one
  // value per token and head) is loaded into element 0 of r.g[0].
  const uint32_t opts = OPTS ? p.opts : 0u;
  const bool scalar_gate = (opts & OPT_SCALAR_GATE) != 0;
  auto load_raw = [&](Raw& r, TaskPos tp, int task, int part) {
    const int hh = task % H;
    const int64_t tl = tp.tok + min(t0, tp.len - 1);
    const int64_t row = tl * (int64_t)H * K + (int64_t)hh * K + 4 * g0;
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      if (part < 0 || part == 0) r.q[u] = *reinterpret_cast<const raw4*>(gq_ + row + 16 * u);
      if (part < 0 || part == 1) r.k[u] = *reinterpret_cast<const raw4*>(gk_ + row + 16 * u);
      if ((part < 0 || part == 2) && !scalar_gate)
        r.g[u] = *reinterpret_cast<const raw4*>(gg_ + row + 16 * u);
    }
    if ((part < 0 || part == 2) && scalar_gate) r.g[0][0] = gg_[tl * H + hh];
    if (part < 0 || part == 2) r.b = gb_[tl * H + hh];
  };
  // The same for the channel groups u of part 0, 1 or 2 that belong to step i of NSTEP: the
  // prefetch is spread over the loops of phases 2-4, a few loads at a time, so that no wave
  // stalls issuing a long burst of loads behind the record stores in flight.
  auto load_raw_step = [&](Raw& r, TaskPos tp, int task, int part, int i, int nstep) {
    const int hh = task % H;
    const int64_t tl = tp.tok + min(t0, tp.len - 1);
    const int64_t row = tl * (int64_t)H * K + (int64_t)hh * K + 4 * g0;
#pragma unroll
    for (int u = i * NG / nstep; u < (i + 1) * NG / nstep; ++u) {
      if (part == 0) r.q[u] = *reinterpret_cast<const raw4*>(gq_ + row + 16 * u);
      if (part == 1) r.k[u] = *reinterpret_cast<const raw4*>(gk_ + row + 16 * u);
      if (part == 2 && !scalar_gate) r.g[u] = *reinterpret_cast<const raw4*>(gg_ + row + 16 * u);
    }
    if (part == 2 && i == 0) {
      if (scalar_gate) r.g[0][0] = gg_[tl * H + hh];
      r.b = gb_[tl * H + hh];
    }
  };
  // V of the current task into its record, slice-major (the state kernel then reads a slice's
  // CHUNK x 16 values as one contiguous block instead of gathering 16 values from each of CHUNK
  // token rows). A token row is vpr 16-byte pieces; each thread copies vpt pieces.
  // Rows past the chunk's end repeat the last valid row (finite; T' is zero in those columns).
  typedef __attribute__((ext_vector_type(4))) unsigned u4;
  const MT* gv_ = reinterpret_cast<const MT*>(p.v);
  const int vpr = V256 ? 16 : p.V * (int)sizeof(MT) / 16;  // a power of two
  const int vsh = V256 ? 4 : __builtin_ctz((unsigned)vpr);
  const int vpt = V256 ? 4 : CHUNK * vpr / PREP_THREADS;  // 1 .. 16
  // pieces per batch. With 256-byte rows a thread's 4 pieces load together when the task starts
  // (ahead of the next task's prefetch) and are stored after phase 5, so that no store has to
  // wait for a load issued just after another store; otherwise up to four batches of four, each
  // loaded a phase before it is stored.
  constexpr int VB = 4;
  constexpr int LDVU = 128 + 8;  // row stride (elements) of V staged in LDS for the U form
  static_assert(!UREC || (size_t)CHUNK * LDVU * sizeof(MT) <= L::szR1, "V fits region R1");
  u4 vbuf[VB];
  // (tid: the loop's opaque copy of threadIdx.x, so that no address is hoisted and kept live)
  auto v_load = [&](int tid, TaskPos tp, int task, int batch) {
    const int hh = task % H;
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const int pi = batch * VB + i;
      if (pi < vpt) {
        const int id = tid + PREP_THREADS * pi;
        const int row = id >> vsh, c = id & (vpr - 1);
        const int64_t tl = tp.tok + min(row, tp.len - 1);
        vbuf[i] = *reinterpret_cast<const u4*>(gv_ + (tl * H + hh) * (int64_t)p.V + c * (16 / (int)sizeof(MT)));
      }
    }
  };
  auto v_store = [&](int tid, char* rec, int batch) {
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const int pi = batch * VB + i;
      if (pi < vpt) {
        const int id = tid + PREP_THREADS * pi;
        const int row = id >> vsh, c = id & (vpr - 1);
        const int slice = c / (int)sizeof(MT), sub = c % (int)sizeof(MT);  // sizeof(MT) pieces per slice row
        *reinterpret_cast<u4*>(rec + R::oVBytes + (size_t)slice * R::vslice_bytes +
                               (size_t)row * 16 * sizeof(MT) + 16 * sub) = vbuf[i];
      }
    }
  };
  int task = blockIdx.x;
  if (task >= ntask) return;
  // chunk positions of the current and the next task; the one after is read a task ahead. (A
  // load issued right after the record stores would be counted behind them: reading the
  // position one task ahead made the loop wait for every store of the task before.)
  TaskPos pcur = task_pos(task);
  TaskPos pnext = task_pos(task + (int)gridDim.x < ntask ? task + (int)gridDim.x : task);
  Raw raw;  // raw inputs of one task: filled one task ahead, consumed by phase 1
  load_raw(raw, pcur, task, -1);
  float kc[NG][4];  // phase 1 -> phase 2: this wave's column operand
  bool diag_exact = false;     // phase 1 -> phase 2: this wave's diagonal block is formed
  f32x4 adiag_x, pdiag_x;      // without the MFMA (strong decay): its A and P entries

  // Phase 1 of a task: its raw inputs become the LDS operands, the per-channel tables, kc and
  // the record parts that need nothing else (Qe, gamma, Ktilde^T).
  auto front = [&](const int task, const TaskPos pc, const Raw& cur) {
    // Lane-dependent addresses are recomputed for every task: without the opaque copy the
    // compiler hoists all of them out of the loop and keeps them live, which spills.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int m = lane & 15;
    const int g = lane >> 4;
    const int t = 16 * w + m;
    const int j = task / H;
    const int h = task - j * H;
    const int len = pc.len;  // 1 .. CHUNK
    MT* recM = reinterpret_cast<MT*>(p.rec + (j * H + h) * p.rec_bytes);
    float* recGam = reinterpret_cast<float*>(p.rec + (j * H + h) * p.rec_bytes + R::oGamBytes);
    const bool valid = t < len;

    // ---------------- phase 1: the token's q, k and log2 alpha (fp32). Past the chunk's end only
    // log alpha (and beta) are zeroed: the q and k rows there repeat the last valid token and
    // have no effect -- beta = 0 zeroes their rows of A and their rows and columns of T', and so
    // their rows of W and Delta (their columns of P meet only those zero rows of Delta) -- while
    // log alpha = 0 keeps the decay products of the valid tokens.
    float qv[NG][4], kv[NG][4], lv[NG][4];
    const bool gate_logits = (opts & OPT_GATE_LOGITS) != 0;
    auto log2_alpha = [&](float z) { return gate_logits ? log2_sigmoid(z) : z * LOG2E; };
    const float l0 = valid ? log2_alpha(to_f32(cur.g[0][0])) : 0.f;  // the scalar gate
  #pragma unroll
    for (int u = 0; u < NG; ++u)
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        qv[u][r] = to_f32(cur.q[u][r]);
        kv[u][r] = to_f32(cur.k[u][r]);
        lv[u][r] = scalar_gate ? l0 : valid ? log2_alpha(to_f32(cur.g[u][r])) : 0.f;
      }
    if (opts & OPT_L2NORM_QK) {
      // the token's K channels sit in the four lanes m, m + 16, m + 32, m + 48
      float sq = 0.f, sk = 0.f;
  #pragma unroll
      for (int u = 0; u < NG; ++u)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          sq += qv[u][r] * qv[u][r];
          sk += kv[u][r] * kv[u][r];
        }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      const float nq = 1.f / sqrtf(sq + L2NORM_EPS), nk = 1.f / sqrtf(sk + L2NORM_EPS);
  #pragma unroll
      for (int u = 0; u < NG; ++u)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          qv[u][r] *= nq;
          kv[u][r] *= nk;
        }
    }
    float bval = to_f32(cur.b);
    if (opts & OPT_BETA_LOGITS) bval = sigmoid_f(bval);
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
      for (int r = 0; r < 4; ++r) dI[u][r] = row_last(lv[u][r]);
    // Diagonal sub-block of this wave. Its MFMA form scales the column operand by the block's
    // inverse decay 2^{-dI} >= 1, which is exact up to rounding while no channel decays by more
    // than 2^DIAG_MAX_LOG2 over the sub-block. Beyond that, the block's A and P entries are
    // formed without any factor above 1: for the token shift s, lane t carries
    // Z_s(t) = k_{t-s} * alpha_{t-s+1} * ... * alpha_t (one DPP row shift and one product per
    // step), so A_{t,t-s} = k_t . Z_s(t) and P_{t,t-s} = q_t . Z_s(t) over this lane's channels,
    // summed over the four lanes that hold the token's channels. Decays then only underflow.
    bool any_big = false;
  #pragma unroll
    for (int u = 0; u < NG; ++u)
  #pragma unroll
      for (int r = 0; r < 4; ++r) any_big |= dI[u][r] < -DIAG_MAX_LOG2;
    diag_exact = __any(any_big);
    if (diag_exact) {
      float* scr = sA + w * 2 * SUBBLK * SUBBLK;  // this wave's two 16 x 16 tiles (R1, free here)
      float z[NG][4], al[NG][4];
  #pragma unroll
      for (int u = 0; u < NG; ++u)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[u][r] = kv[u][r];
          al[u][r] = exp2_f(lv[u][r] - row_shr<1>(lv[u][r]));  // the token's own decay
        }
  #pragma unroll
      for (int s = 0; s < SUBBLK; ++s) {
        float a = 0.f, pq = 0.f;
  #pragma unroll
        for (int u = 0; u < NG; ++u)
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            a += kv[u][r] * z[u][r];
            pq += qv[u][r] * z[u][r];
          }
        a += __shfl_xor(a, 16);
        pq += __shfl_xor(pq, 16);
        a += __shfl_xor(a, 32);
        pq += __shfl_xor(pq, 32);
        // row t = m, column t - s (lanes m < s hold zero: the shift brought nothing in)
        if (g == (s >> 2) && m >= s) {
          scr[m * SUBBLK + (m - s)] = a;
          scr[SUBBLK * SUBBLK + m * SUBBLK + (m - s)] = pq;
        }
        if (s + 1 < SUBBLK) {
  #pragma unroll
          for (int u = 0; u < NG; ++u)
  #pragma unroll
            for (int r = 0; r < 4; ++r) z[u][r] = row_shr<1>(z[u][r]) * al[u][r];
        }
      }
      // back in the accumulator layout of the MFMA tile: lane (m, g) holds rows 4g .. 4g+3 of
      // column m; entries above the diagonal are never written here and are masked later
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        adiag_x[r] = (m <= i) ? scr[i * SUBBLK + m] : 0.f;
        pdiag_x[r] = (m <= i) ? scr[SUBBLK * SUBBLK + i * SUBBLK + m] : 0.f;
      }
    }
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
    //   Qe = q e^{b_t} (record, from registers),  Ka = k e^{b_t},  Kt = k e^{b_last - b_t}
    {
      f32x4 qh[NG], kh[NG], qe[NG];
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
        // this lane's slot of Qe's row tile w, step s is exactly its own token and channels
        *reinterpret_cast<frag*>(recM + R::oQ + slot) = to_frag(qe[GPS * s], qe[GPS * s + GPS - 1], MT());
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

  };
  front(task, pcur, raw);

  // Each iteration runs phases 2-5 of one task and then phase 1 of the next, so the waits for
  // the prefetched inputs come after the record stores in straight-line code.
#pragma clang loop unroll(disable)
  for (;;) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g = lane >> 4;
  const int j = task / H;
  const int h = task - j * H;
  const int ntsk = task + (int)gridDim.x < ntask ? task + (int)gridDim.x : task;
  const TaskPos pn = pnext;
  const int nntsk = ntsk + (int)gridDim.x < ntask ? ntsk + (int)gridDim.x : ntsk;
  pnext = task_pos(nntsk);
  MT* recM = reinterpret_cast<MT*>(p.rec + (j * H + h) * p.rec_bytes);

  // the next task's inputs load during phases 2-4 (phase 1's fp32 copies are dead by now):
  // q in phase 2's loop, k in the loop that stores A and P, log alpha and beta in phase 4's
  v_load(tid, pcur, task, 0);

  // ---------------- phase 2: blocks (I, w), I >= w, of A and P. The column operand (token
  // block w, scaled per channel by D_{Iw}) is this wave's own kc; the row operands are read as
  // fragments. Results stay in registers until every wave is done with Q^, K^ and D.
  f32x4 tA[NSUB], tP[NSUB];
  wave_prio(NSUB - 1 - w);  // wave w forms NSUB - w blocks: the busiest issue first
#pragma unroll
  for (int I = 0; I < NSUB; ++I) {
    tA[I] = f32x4{0.f, 0.f, 0.f, 0.f};
    tP[I] = tA[I];
    load_raw_step(raw, pn, ntsk, 0, I, NSUB);
    if (I < w) continue;
    if (I == w && diag_exact) {
      tA[I] = adiag_x;
      tP[I] = pdiag_x;
      continue;
    }
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
  wave_prio(0);
  lds_barrier();
  // A (row-scaled by beta, strictly lower) -> sA for the off-diagonal blocks; P (lower with the
  // diagonal, zero above) -> sPnT, transposed. The diagonal block A_ww stays in registers for
  // phase 3(a).
  f32x4 adiag = tA[0];
#pragma unroll
  for (int I = 1; I < NSUB; ++I) adiag = (I == w) ? tA[I] : adiag;
  {
    const int jj = 16 * w + m;
#pragma unroll
    for (int I = 0; I < NSUB; ++I) {
      load_raw_step(raw, pn, ntsk, 1, I, NSUB);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        if (I > w) sA[i * L::LCF + jj] = tA[I][r] * sBeta[i];
      }
      // P^T row jj, columns 16I + 4g .. +3
      f32x4 pn;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        pn[r] = (I > w || (I == w && jj <= i)) ? tP[I][r] : 0.f;
      }
      st4(sPnT + jj * L::LC + 16 * I + 4 * g, pn);
    }
  }

  if (!V256) v_store(tid, reinterpret_cast<char*>(recM), 0);
  if (vpt > VB) v_load(tid, pcur, task, 1);

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
  //     row-major in the unused upper block (J, I) of sA. Before that, every wave copies its
  //     share of P's fragment slots from sPnT to the record (wave 0 has no block to solve).
  {
    constexpr int NSL = NSUB * (CHUNK / KS) * 64;
    static_assert(NSL % PREP_THREADS == 0, "slot split");
#pragma unroll
    for (int i = 0; i < NSL / PREP_THREADS; ++i) {
      const int sl = tid + PREP_THREADS * i;
      const int ln = sl & 63, ts = sl >> 6;
      const int s = ts % (CHUNK / KS), tile = ts / (CHUNK / KS);
      // the slots above the diagonal (all zero) are never read: not written
      if (KS * s <= 16 * tile + 15)
        *reinterpret_cast<frag*>(recM + R::oPb + (size_t)sl * EPL) = frag_t(sPnT, L::LC, 16 * tile, s, ln);
    }
  }
  if (w >= 1) {
    const int Ib = w;
    wave_prio(w);  // row block w has w blocks to solve, one after another
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
    wave_prio(0);
  }
  lds_barrier();

  if (vpt > VB) v_store(tid, reinterpret_cast<char*>(recM), 1);
  if (vpt > 2 * VB) v_load(tid, pcur, task, 2);

  // ---------------- phase 4: T' = T diag(beta) -> LDS (row-major)
#pragma unroll
  for (int it = 0; it < CHUNK * CHUNK / 4 / PREP_THREADS; ++it) {
    load_raw_step(raw, pn, ntsk, 2, it, CHUNK * CHUNK / 4 / PREP_THREADS);
    const int idx = tid + PREP_THREADS * it;
    const unsigned i = (unsigned)idx / (CHUNK / 4), j0 = 4u * ((unsigned)idx % (CHUNK / 4));
    const unsigned Ii = i >> 4, Jj = j0 >> 4;
    // diagonal blocks of T sit in place, block (Ii, Jj < Ii) transposed in the upper block (Jj, Ii)
    // (selected arithmetically: a branch here made the compiler wait on the pending prefetch)
    const unsigned srcd = i * L::LCF + j0, srco = (16u * Jj + (i & 15u)) * L::LCF + 16u * Ii + (j0 & 15u);
    const unsigned sel = 0u - (unsigned)(Ii == Jj);
    const unsigned src = (srcd & sel) | (srco & ~sel);
    f32x4 tv = *reinterpret_cast<const f32x4*>(sA + src);
    tv *= *reinterpret_cast<const f32x4*>(sBeta + j0);
    if (Ii < Jj) tv = f32x4{0.f, 0.f, 0.f, 0.f};
    st4(sTb + i * L::LC + j0, tv);
  }
  lds_barrier();
  if (vpt > 2 * VB) v_store(tid, reinterpret_cast<char*>(recM), 2);
  if (vpt > 3 * VB) v_load(tid, pcur, task, 3);

  // ---------------- phase 5: T' fragments to the record (whole 16-byte lane slots), then
  // W^T = Ka^T T'^T -> record (as -W fragments). In the U form V goes to LDS (region R1, free
  // since phase 4) instead, for U = T'V after W.
  if constexpr (UREC) {
    MT* sVs = reinterpret_cast<MT*>(smem + L::oR1);  // V, [CHUNK][LDVU] row-major
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const int id = tid + PREP_THREADS * i;
      const int row = id >> 4, c = id & 15;
      *reinterpret_cast<u4*>(sVs + row * LDVU + 8 * c) = vbuf[i];
    }
  }
  if constexpr (!UREC) {
    constexpr int NSL = NSUB * (CHUNK / KS) * 64;
#pragma unroll
    for (int i = 0; i < NSL / PREP_THREADS; ++i) {
      const int sl = tid + PREP_THREADS * i;
      const int ln = sl & 63, ts = sl >> 6;
      const int s = ts % (CHUNK / KS), tile = ts / (CHUNK / KS);
      if (KS * s <= 16 * tile + 15)  // as for P: the all-zero slots are not written
        *reinterpret_cast<frag*>(recM + R::oTb + (size_t)sl * EPL) =
            load_frag(sTb + (16 * tile + (ln & 15)) * L::LC, s, ln >> 4);
    }
  }
  // Result tile (channel tile a, token tile b): lane (m, g) holds W[16b + m][16a + 4g + r]. A
  // wave takes the KS / 16 channel tiles of one reduction step together, which together are
  // exactly its lanes' slots of W's fragment (token tile b, step ap).
  {
    constexpr int TPS = KS / 16;  // channel tiles per reduction step
#pragma unroll
    for (int tix = 0; tix < (NKT / TPS) * NSUB; ++tix) {
      const int ap = tix % (NKT / TPS), b = tix / (NKT / TPS);
      if (tix % 4 != w) continue;
      const int nsteps = (16 * b + 16 + KS - 1) / KS;
      f32x4 acc[TPS];
#pragma unroll
      for (int t = 0; t < TPS; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < CHUNK / KS; ++s)
          if (s < nsteps)
            acc[t] = Mma<MT>::mma(frag_t(sKa, L::LDK, 16 * (TPS * ap + t), s, lane),
                                  load_frag(sTb + (16 * b + m) * L::LC, s, g), acc[t]);
        acc[t] = -acc[t];  // the record holds -W
      }
      *reinterpret_cast<frag*>(recM + R::oW + slot_elem<MT>(b, ap, lane, K)) = to_frag(acc[0], acc[TPS - 1], MT());
    }
  }

  if (vpt > 3 * VB) v_store(tid, reinterpret_cast<char*>(recM), 3);
  if constexpr (UREC) {
    // U = T'V: result tile (token tile tt, value tile ct) over the steps T' is not zero in;
    // wave w takes the tiles with (8 tt + ct) % 4 == w
    lds_barrier();
    const MT* sVs = reinterpret_cast<const MT*>(smem + L::oR1);
#pragma unroll
    for (int tix = 0; tix < NSUB * 8; ++tix) {
      if (tix % 4 != w) continue;
      const int tt = tix / 8, ct = tix % 8;
      const int nsteps = (16 * tt + 16 + KS - 1) / KS;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CHUNK / KS; ++s)
        if (s < nsteps)
          acc = Mma<MT>::mma(load_frag(sTb + (16 * tt + m) * L::LC, s, g),
                             frag_t(sVs, LDVU, 16 * ct, s, lane), acc);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(recM) + R::u_tile_byte(ct, tt, lane)) =
          __builtin_convertvector(acc, bf16x4);
    }
  } else if (V256) {
    v_store(tid, reinterpret_cast<char*>(recM), 0);
  }
  lds_barrier();  // the next task reuses every LDS region
  task += gridDim.x;
  if (task >= ntask) break;
  pcur = pn;
  front(task, pn, raw);
  }
}

// ====================================================================== STATE kernel
// One wave per (sequence run, head, 16-column slice of V). The columns of S evolve
// independently, so a slice needs nothing from its neighbours: its state S [K x 16] (fp32),
// U and Delta [CHUNK x 16] and its output tile all live in registers. Each product takes the
// chunk record's fragments as loaded, and every result tile is already in the operand layout
// of the product that consumes it (a 16-row result tile -- two for bf16 -- is a fragment
// along its row index):
//   Delta = U + (-W) S                       B operand: S as fragments along K
//   S'    = Diag(gamma) S + Ktilde^T Delta   B operand: Delta as fragments along the tokens
//   O^T   = S^T Qe^T + Delta^T P^T           A operands: the same S and Delta fragments
//   U = T'V of the next chunk                V through LDS and the transposing read
// so the state path has no workgroup barrier and no LDS round trip. A chunk is NF matrix-core
// operations, each consuming one record fragment; the fragments stream through a ring of D
// registers, each load issued D operations ahead of its use. V and gamma pass through this
// wave's own LDS (the transposing read and the per-lane gamma layout need it).
template <int K, typename MT>
struct StateShape {
  static constexpr int KS = Mma<MT>::KS;
  static constexpr int NKT = K / 16;      // key-channel tiles of S
  static constexpr int NKS = K / KS;      // reduction steps over K
  static constexpr int NTT = CHUNK / 16;  // token tiles
  static constexpr int NTS = CHUNK / KS;  // reduction steps over tokens
  // fragment (tile t, step s) of a lower-triangular CHUNK x CHUNK matrix may be nonzero
  static constexpr bool tri_nz(int t, int s) { return KS * s < 16 * (t + 1); }
  static constexpr int NTRI = [] {
    int n = 0;
    for (int s = 0; s < NTS; ++s)
      for (int t = 0; t < NTT; ++t) n += tri_nz(t, s) ? 1 : 0;
    return n;
  }();
  // i-th nonzero fragment, steps outer: tile and step
  static constexpr int tri_t(int i) {
    for (int s = 0; s < NTS; ++s)
      for (int t = 0; t < NTT; ++t)
        if (tri_nz(t, s) && i-- == 0) return t;
    return 0;
  }
  static constexpr int tri_s(int i) {
    for (int s = 0; s < NTS; ++s)
      for (int t = 0; t < NTT; ++t)
        if (tri_nz(t, s) && i-- == 0) return s;
    return 0;
  }
  // the chunk's operations in issue order: -W and Qe interleaved per K step (2*NTT per step),
  // Ktilde^T (steps outer), T' of the next chunk, then P of this chunk
  static constexpr int NA = 2 * NTT * NKS;
  static constexpr int NB = NKT * NTS;
  static constexpr int NF = NA + NB + 2 * NTRI;
  static constexpr int DMAX = 60;  // ring length limit (4 registers per fragment)
  static constexpr int D = [] {
    for (int d = DMAX; d > 1; --d)
      if (NF % d == 0) return d;
    return 1;
  }();
  static constexpr int LDV = 16 + 16 / (int)sizeof(MT);  // LDS row of V (16-byte aligned)
};

struct StateParams {
  const void* v;
  void* o;
  const float* init_state;
  float* state;  // running and final state [N][H][K][V]
  const Entry* entries;
  const int32_t* header;
  const int32_t* basetab;    // base[d] of the chunk table (depth-major order)
  const int32_t* seg_first;  // this segment's list
  const int32_t* seg_count;  // this segment's count
  int64_t seg_begin, E;
  int H, V, n_slices;
  int64_t chains;  // slots * H
  const char* rec;
  uint32_t rec_bytes;
  uint32_t rec_buf_bytes;  // the whole record buffer (addressed with 32-bit offsets)
  int seq_major;           // the chunk table's order
  float* ckpt;             // checkpoint states (ChunkArgs::ckpt; sequence-major tables only)
};

constexpr int STATE_THREADS = 64;

// Raw buffer access (gfx9 descriptor: byte-addressed, range-checked against num_records: loads
// past the end return zero and stores past the end are dropped).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ T buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  static_assert(sizeof(T) == 16, "16-byte load");
  return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, bf16x4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, x), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, x), r, (int)voff, (int)soff, 0);
}
template <typename MT>
__device__ __forceinline__ auto to_mt4(f32x4 x) {
  if constexpr (std::is_same_v<MT, bf16>) return __builtin_convertvector(x, bf16x4);
  else return x;
}

template <int K, typename MT>
__global__ __launch_bounds__(STATE_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void state_kernel(StateParams p) {
  using SH = StateShape<K, MT>;
  using R = Rec<K, MT>;
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int KS = SH::KS, NKT = SH::NKT, NKS = SH::NKS, NTT = SH::NTT, NTS = SH::NTS;
  constexpr int NA = SH::NA, NB = SH::NB, NTRI = SH::NTRI, NF = SH::NF, D = SH::D;
  constexpr int LDV = SH::LDV;
  constexpr int VL = 16 / (int)sizeof(MT);  // V elements per 16-byte load
  constexpr int NVL = 16 / VL;              // 16-byte loads per token row of the slice
  using vload = typename VecN<MT, VL>::vec;
  static_assert(K % KS == 0 && K % 16 == 0, "K tiling");
  __shared__ __align__(16) MT sV[CHUNK * LDV];
  __shared__ __align__(16) float sG[K];
  __shared__ int32_t sRun[SEG_CHUNK_HEADS + 16];
  __shared__ int32_t sLen;

  // XCD-aware decode: all slices of a chain share blockIdx % 8 (the same XCD / L2).
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
  const int col0 = slice * 16;
  const int lane = lane_id();
  const int m = lane & 15;
  const int g = lane >> 4;

  // This wave's run: chunks d0, d0+1, ... of sequence en.seq inside the segment. Chunk d0+k is
  // entry base[d0+k] + rank; the run ends at the sequence's end or the segment's end.
  const int seq_start = en.tok - CHUNK * en.depth;
  const int nc = (en.end - seq_start + CHUNK - 1) / CHUNK;
  const int64_t rank = p.seq_major ? 0 : e0 - p.basetab[en.depth];
  const int kmax = (int)min((int64_t)(nc - en.depth), p.E);
  if (lane == 0) sLen = kmax;
  __syncthreads();
  for (int k = lane; k < kmax; k += STATE_THREADS) {
    const int64_t ek = p.seq_major ? e0 + k : p.basetab[en.depth + k] + rank;
    sRun[k] = (int32_t)(ek - p.seg_begin);
    if (ek >= seg_end) atomicMin(&sLen, k);
  }
  __syncthreads();
  const int run = sLen;

  // state tile kt: lane (m, g) holds S[16kt + 4g + i][col0 + m], i = 0..3
  const size_t sbase = ((size_t)en.seq * H + h) * (size_t)K * V + col0;
  const float* src = (en.depth == 0) ? p.init_state : p.state;
  f32x4 S[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (src != nullptr) {
      const float* ps = src + sbase + (size_t)(16 * kt + 4 * g) * V + m;
      x = f32x4{ps[0], ps[V], ps[2 * V], ps[3 * V]};
    }
    S[kt] = x;
  }

  // Per-chunk descriptors cover the chunk's valid rows of V and of the output, so rows past
  // the end load as zero (T' is zero in those columns anyway) and are never stored.
  const uint32_t rowb = (uint32_t)(H * V * (int)sizeof(MT));  // bytes between token rows
  MT* go = reinterpret_cast<MT*>(p.o) + (int64_t)h * V + col0;
  auto tok_of = [&](int k) { return seq_start + CHUNK * (en.depth + k); };
  auto len_of = [&](int k) { return min(CHUNK, en.end - tok_of(k)); };
  auto rows_rsrc = [&](const MT* base, int k) {
    const int kk = min(k, run - 1);
    return make_rsrc(base + (int64_t)tok_of(kk) * (H * V), (uint32_t)len_of(kk) * rowb);
  };
  const uint32_t o_voff = (uint32_t)m * rowb + 4u * g * (uint32_t)sizeof(MT);  // token m of a tile

  // records: one descriptor over the buffer, 32-bit offsets; chunk k of the run (clamped to the
  // run's last chunk -- a load past the end is never used)
  const rsrc_t rrec = make_rsrc(p.rec, p.rec_buf_bytes);
  const uint32_t rec_h = (uint32_t)h * p.rec_bytes;
  const uint32_t rec_stride = (uint32_t)H * p.rec_bytes;
  auto rec_off = [&](int ri) { return rec_h + (uint32_t)ri * rec_stride; };
  const uint32_t lo = 16u * (uint32_t)lane;  // a fragment slot is 64 lanes x 16 bytes
  auto ldf = [&](uint32_t rc, uint32_t off) -> frag {
    return buf_load16<frag>(rrec, lo + (off & 4095u), rc + (off & ~4095u));
  };

  // operation j reads the next chunk's record (T') or this chunk's (everything else)
  auto next_rec = [](int j) constexpr { return j >= NA + NB && j < NA + NB + NTRI; };
  // byte offset (without the lane part) of operation j's fragment in its record
  auto frag_off = [](auto J) constexpr -> uint32_t {
    constexpr int j = decltype(J)::value;
    constexpr uint32_t SLOT = 64 * 16;
    if constexpr (j < NA) {
      constexpr int s = j / (2 * NTT), r = j % (2 * NTT), tt = r % NTT;
      constexpr size_t base = (r < NTT ? R::oW : R::oQ) * sizeof(MT);
      return (uint32_t)(base + (size_t)(tt * NKS + s) * SLOT);
    } else if constexpr (j < NA + NB) {
      constexpr int jj = j - NA, s = jj / NKT, kt = jj % NKT;
      return (uint32_t)(R::oKt * sizeof(MT) + (size_t)(kt * NTS + s) * SLOT);
    } else {
      constexpr int jj = (j - NA - NB) % NTRI;
      constexpr size_t base = (j - NA - NB < NTRI ? R::oTb : R::oPb) * sizeof(MT);
      return (uint32_t)(base + (size_t)(SH::tri_t(jj) * NTS + SH::tri_s(jj)) * SLOT);
    }
  };

  // this slice's V rows of the chunk whose record starts at rc (lane = token), and gamma
  const uint32_t vslice_off = (uint32_t)(R::oVBytes + (size_t)slice * R::vslice_bytes);
  auto load_v = [&](uint32_t rc, vload (&x)[NVL]) {
#pragma unroll
    for (int i = 0; i < NVL; ++i)
      x[i] = buf_load16<vload>(rrec, (uint32_t)lane * 16u * sizeof(MT) + 16u * i, rc + vslice_off);
  };
  auto stage_v = [&](const vload (&x)[NVL]) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) *reinterpret_cast<vload*>(sV + lane * LDV + VL * i) = x[i];
  };
  constexpr int GPL = (K + 63) / 64;  // gamma values per lane (1 or 2)
  using gvec = std::conditional_t<GPL == 2, f32x2, float>;
  const uint32_t g_voff = 4u * (uint32_t)min(GPL * lane, K - GPL);
  auto load_g = [&](uint32_t rc) -> gvec {
    if constexpr (GPL == 2)
      return __builtin_bit_cast(gvec, __builtin_amdgcn_raw_buffer_load_b64(rrec, (int)(g_voff + R::oGamBytes % 4096), (int)(rc + R::oGamBytes / 4096 * 4096), 0));
    else
      return __builtin_bit_cast(gvec, __builtin_amdgcn_raw_buffer_load_b32(rrec, (int)(g_voff + R::oGamBytes % 4096), (int)(rc + R::oGamBytes / 4096 * 4096), 0));
  };
  auto stage_g = [&](gvec x) {
    if (GPL * lane < K) *reinterpret_cast<gvec*>(sG + GPL * lane) = x;
  };
  auto rec_index = [&](int k) { return __builtin_amdgcn_readfirstlane(sRun[min(k, run - 1)]); };

  // ---- prologue: U of chunk 0, the ring for chunk 0, gamma of chunk 0
  uint32_t rc0 = rec_off(rec_index(0));
  uint32_t rc1 = rec_off(rec_index(1));
  uint32_t rc2 = rec_off(rec_index(2));
  f32x4 U[NTT], O[NTT];
  frag Vf[NTS];
  {
    vload vx[NVL];
    load_v(rc0, vx);
    stage_v(vx);
#pragma unroll
    for (int s = 0; s < NTS; ++s) Vf[s] = frag_t(sV, LDV, 0, s, lane);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) U[tt] = O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, NTRI>([&](auto I) {
      constexpr int i = decltype(I)::value, tt = SH::tri_t(i), s = SH::tri_s(i);
      U[tt] = M::mma(ldf(rc0, frag_off(std::integral_constant<int, NA + NB + i>())), Vf[s], U[tt]);
    });
  }
  // gamma first, then the ring: in the loop gamma is waited for long after the loads behind it
  gvec gnext = load_g(rc0);
  __builtin_amdgcn_sched_barrier(0);
  frag ring[D];
  static_for<0, D>([&](auto J) {
    constexpr int j = decltype(J)::value;
    ring[j] = ldf(next_rec(j) ? rc1 : rc0, frag_off(J));
  });
  __builtin_amdgcn_sched_barrier(0);
  int ri_pre = sRun[min(3, run - 1)];  // record index of chunk k + 3, read one chunk ahead
  vload vx[NVL];                         // V rows of chunk k + 1, loaded a chunk ahead
  load_v(rc1, vx);

  for (int k = 0; k < run; ++k) {
    // records of chunks k, k+1, k+2 (rc0 .. rc2 on entry), and k+3 for the next iteration
    const uint32_t rc3 = rec_off(__builtin_amdgcn_readfirstlane(ri_pre));
    ri_pre = sRun[min(k + 4, run - 1)];
    const rsrc_t ro = rows_rsrc(go, k);
    const gvec gcur = gnext;
    gnext = load_g(rc1);
    __builtin_amdgcn_sched_barrier(0);

    frag Sb[NKS], Db[NTS];
    f32x4 gam[NKT];
    static_for<0, NF>([&](auto J) {
      constexpr int j = decltype(J)::value;
      // --- work placed before operation j
      if constexpr (j < NA && j % (2 * NTT) == 0) {
        constexpr int s = j / (2 * NTT);
        if constexpr (KS == 32) Sb[s] = frag_from_acc(S[2 * s], S[2 * s + 1], MT());
        else Sb[s] = S[s];
      }
      // gamma of chunk k into LDS, then per key-channel tile: read gamma GLEAD operations ahead
      // and scale S (every S fragment is formed by then) as the update's accumulator
      constexpr int GLEAD = 6;
      static_assert(NA > GLEAD, "gamma lead");
      if constexpr (j == NA - GLEAD - 1) stage_g(gcur);
      static_for<0, NKT>([&](auto KT) {
        constexpr int kt = decltype(KT)::value;
        if constexpr (j == NA + kt - GLEAD) gam[kt] = *reinterpret_cast<const f32x4*>(sG + 16 * kt + 4 * g);
        if constexpr (j == NA + kt) S[kt] *= gam[kt];
      });
      if constexpr (j == NA) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
          if constexpr (KS == 32) Db[s] = frag_from_acc(U[2 * s], U[2 * s + 1], MT());
          else Db[s] = U[s];
        }
      }
      if constexpr (j == NA + NB / 2) {
        // V of chunk k+1 into LDS and its fragments
        stage_v(vx);
#pragma unroll
        for (int s = 0; s < NTS; ++s) Vf[s] = frag_t(sV, LDV, 0, s, lane);
      }
      if constexpr (j == NA + NB) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) U[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        load_v(rc2, vx);
      }
      // --- operation j
      const frag f = ring[j % D];
      if constexpr (j < NA) {
        constexpr int s = j / (2 * NTT), r = j % (2 * NTT), tt = r % NTT;
        if constexpr (r < NTT) U[tt] = M::mma(f, Sb[s], U[tt]);  // U - W S
        else O[tt] = M::mma(Sb[s], f, O[tt]);                    // S^T Qe^T
      } else if constexpr (j < NA + NB) {
        constexpr int jj = j - NA, s = jj / NKT, kt = jj % NKT;
        S[kt] = M::mma(f, Db[s], S[kt]);  // + Ktilde^T Delta
      } else if constexpr (j < NA + NB + NTRI) {
        constexpr int i = j - NA - NB;
        U[SH::tri_t(i)] = M::mma(f, Vf[SH::tri_s(i)], U[SH::tri_t(i)]);  // T'V, next chunk
      } else {
        constexpr int i = j - NA - NB - NTRI;
        O[SH::tri_t(i)] = M::mma(Db[SH::tri_s(i)], f, O[SH::tri_t(i)]);  // + Delta^T P^T
      }
      // --- refill: operation j + D of the stream
      {
        constexpr int jn = j + D;
        if constexpr (jn < NF) {
          ring[j % D] = ldf(next_rec(jn) ? rc1 : rc0, frag_off(std::integral_constant<int, jn>()));
        } else {
          constexpr int jw = jn - NF;
          ring[j % D] = ldf(next_rec(jw) ? rc2 : rc1, frag_off(std::integral_constant<int, jw>()));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // output rows of chunk k; the accumulators restart for chunk k+1
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      buf_store(ro, o_voff, (uint32_t)(16 * tt) * rowb, to_mt4<MT>(O[tt]));
      O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    rc0 = rc1;
    rc1 = rc2;
    rc2 = rc3;
  }

#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    float* ps = p.state + sbase + (size_t)(16 * kt + 4 * g) * V + m;
    ps[0] = S[kt][0];
    ps[V] = S[kt][1];
    ps[2 * V] = S[kt][2];
    ps[3 * V] = S[kt][3];
  }
  // a sequence that goes on past the segment: its state before chunk seg_end, the checkpoint
  // of boundary seg_end / E (sequence-major table: entry index = chunk index in token order)
  if (p.ckpt != nullptr && en.depth + run < nc) {
    float* pc = p.ckpt + ((size_t)(seg_end / p.E - 1) * H + h) * (size_t)K * V + col0;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      float* ps = pc + (size_t)(16 * kt + 4 * g) * V + m;
      ps[0] = S[kt][0];
      ps[V] = S[kt][1];
      ps[2 * V] = S[kt][2];
      ps[3 * V] = S[kt][3];
    }
  }
}

// ---------------------------------------------------------------------- two-wave state kernel
// The chain of one (sequence run, head, 16-column slice) split by key channels over the two
// waves of a workgroup: wave w holds rows [w K/2, (w+1) K/2) of S and streams only the record
// fragments of its half -- -W and Qe over its reduction steps, Ktilde^T over its rows -- plus
// T' of the next chunk (wave 0; in the record's U form that chunk's U instead) or P (wave 1).
// Per chunk:
//   Delta_w = [U] + (-W_w) S_w       partial over this wave's half of K (wave 0 starts from U)
//   exchange Delta_w through LDS, Delta = Delta_0 + Delta_1 (fp32), one barrier
//   S_w' = Diag(gamma_w) S_w + Ktilde_w^T Delta
//   O^T = S_0^T Qe_0^T + S_1^T Qe_1^T + Delta^T P^T     (partials; summed at the next exchange)
// Each wave issues half of the chunk's matrix-core and vector work and keeps one chunk (or two:
// a ring of 2 NF registers, for which the loop handles chunks in pairs so that every ring slot
// has a fixed register) of its fragments in flight. The two halves of the output meet at the next chunk's
// exchange: each wave keeps half of the token tiles of O and receives the partner's partial
// for them. Exchange buffers alternate by chunk parity, so a write never meets the partner's
// read of the previous chunk. Measured on the long prefill this is a few percent faster than
// one wave per chain: the chain stays bound by the fragments' round trips through L2 (the
// CU's L1 reports stalls on pending L2 data for about 40% of the kernel's time either way).
// NW waves per slice, each holding K / NW key channels of S: two up to K = 128, four at
// K = 256 (so that each wave's share of S and of the chunk's fragments stays that of K = 128)
template <int K>
constexpr int split_threads() { return K > 128 ? 256 : 128; }
template <int K, typename MT>
struct SplitShape {
  using SH = StateShape<K, MT>;
  static constexpr int NW = K > 128 ? 4 : 2;
  static constexpr int THREADS = 64 * NW;
  static constexpr int KS = SH::KS, NKT = SH::NKT, NKS = SH::NKS, NTT = SH::NTT, NTS = SH::NTS;
  static constexpr int NTRI = SH::NTRI;
  static constexpr bool OK = NKS % NW == 0 && NTT % NW == 0;
  static constexpr int HKS = NKS / NW;  // reduction steps over K per wave
  static constexpr int HKT = NKT / NW;  // key-channel tiles of S per wave
  static constexpr int HT = NTT / NW;   // output token tiles each wave stores
  static constexpr int NA = 2 * NTT * HKS;      // -W and Qe, interleaved per step
  static constexpr int NB = HKT * NTS;          // Ktilde^T over this wave's rows
  static constexpr int NF = NA + NB + NTRI;     // + T' (wave 0) or P (wave 1); NA + NB for the rest
  // chunks of fragments in flight (1 or 2): the same time on the long prefill (2.24 ms per
  // call), and one chunk needs 120 fewer registers
  static constexpr int RING_CHUNKS = 1;
  static_assert(THREADS == split_threads<K>(), "one thread count per K");
};

// UREC: the record's U form (bf16, 128 value columns): wave 0 takes U from the record instead of
// forming T'V, and V is not staged.
template <int K, typename MT, bool UREC = false>
__global__ __launch_bounds__(split_threads<K>()) __attribute__((amdgpu_waves_per_eu(K > 128 ? 2 : 1, K > 128 ? 2 : 1))) void state_split_kernel(StateParams p) {
  using SH = StateShape<K, MT>;
  using SS = SplitShape<K, MT>;
  constexpr int NW = SS::NW;
  using R = Rec<K, MT>;
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int KS = SS::KS, NKS = SS::NKS, NTT = SS::NTT, NTS = SS::NTS, NTRI = SS::NTRI;
  constexpr int HKS = SS::HKS, HKT = SS::HKT, HT = SS::HT, NA = SS::NA, NB = SS::NB, NF = SS::NF;
  constexpr int LDV = SH::LDV;
  constexpr int VL = 16 / (int)sizeof(MT);
  constexpr int NVL = 16 / VL;
  using vload = typename VecN<MT, VL>::vec;
  static_assert(SS::OK, "two-wave split needs an even number of K steps and token tiles");
  static_assert(HKT == HKS * (KS / 16), "a wave's K steps cover its key tiles");
  __shared__ __align__(16) f32x4 sX[2][NW][NTT][64];  // [parity][wave][token tile][lane]: Delta partials
  __shared__ __align__(16) f32x4 sO[2][NW][NTT][64];  // [parity][wave][tile][lane]: O partials for the tile's owner
  __shared__ __align__(16) MT sV[CHUNK * LDV];       // wave 0: V of the next chunk
  __shared__ int32_t sRun[SEG_CHUNK_HEADS + 16];
  __shared__ int32_t sLen;

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
  const int col0 = slice * 16;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int m = lane & 15;
  const int g = lane >> 4;

  const int seq_start = en.tok - CHUNK * en.depth;
  const int nc = (en.end - seq_start + CHUNK - 1) / CHUNK;
  const int64_t rank = p.seq_major ? 0 : e0 - p.basetab[en.depth];
  const int kmax = (int)min((int64_t)(nc - en.depth), p.E);
  if (tid == 0) sLen = kmax;
  __syncthreads();
  for (int k = tid; k < kmax; k += SS::THREADS) {
    const int64_t ek = p.seq_major ? e0 + k : p.basetab[en.depth + k] + rank;
    sRun[k] = (int32_t)(ek - p.seg_begin);
    if (ek >= seg_end) atomicMin(&sLen, k);
  }
  __syncthreads();
  const int run = sLen;

  const size_t sbase = ((size_t)en.seq * H + h) * (size_t)K * V + col0;
  const float* src = (en.depth == 0) ? p.init_state : p.state;
  const uint32_t rowb = (uint32_t)(H * V * (int)sizeof(MT));
  MT* go = reinterpret_cast<MT*>(p.o) + (int64_t)h * V + col0;
  auto tok_of = [&](int k) { return seq_start + CHUNK * (en.depth + k); };
  auto len_of = [&](int k) { return min(CHUNK, en.end - tok_of(k)); };
  auto rows_rsrc = [&](const MT* base, int k) {
    const int kk = min(k, run - 1);
    return make_rsrc(base + (int64_t)tok_of(kk) * (H * V), (uint32_t)len_of(kk) * rowb);
  };
  const uint32_t o_voff = (uint32_t)m * rowb + 4u * g * (uint32_t)sizeof(MT);
  const rsrc_t rrec = make_rsrc(p.rec, p.rec_buf_bytes);
  const uint32_t rec_h = (uint32_t)h * p.rec_bytes;
  const uint32_t rec_stride = (uint32_t)H * p.rec_bytes;
  auto rec_off = [&](int ri) { return rec_h + (uint32_t)ri * rec_stride; };
  const uint32_t lo = 16u * (uint32_t)lane;
  auto ldf = [&](uint32_t rc, uint32_t off) -> frag {
    return buf_load16<frag>(rrec, lo + (off & 4095u), rc + (off & ~4095u));
  };
  auto rec_index = [&](int k) { return __builtin_amdgcn_readfirstlane(sRun[min(k, run - 1)]); };

  auto body = [&](auto WVc) {
    constexpr int WV = decltype(WVc)::value;
    constexpr int NFW = (WV == 1 || (WV == 0 && !UREC)) ? NF : NA + NB;  // operations per chunk
    // operation j of this wave's stream reads the next chunk's record (wave 0's T') or this one's
    auto next_rec = [](int j) constexpr { return WV == 0 && j >= NA + NB; };
    auto frag_off = [](auto J) constexpr -> uint32_t {
      constexpr int j = decltype(J)::value;
      constexpr uint32_t SLOT = 64 * 16;
      if constexpr (j < NA) {
        constexpr int s = WV * HKS + j / (2 * NTT), r = j % (2 * NTT), tt = r % NTT;
        constexpr size_t base = (r < NTT ? R::oW : R::oQ) * sizeof(MT);
        return (uint32_t)(base + (size_t)(tt * NKS + s) * SLOT);
      } else if constexpr (j < NA + NB) {
        constexpr int jj = j - NA, s = jj / HKT, kt = WV * HKT + jj % HKT;
        return (uint32_t)(R::oKt * sizeof(MT) + (size_t)(kt * NTS + s) * SLOT);
      } else {
        constexpr int i = j - NA - NB;
        constexpr size_t base = (WV == 0 ? R::oTb : R::oPb) * sizeof(MT);
        return (uint32_t)(base + (size_t)(SH::tri_t(i) * NTS + SH::tri_s(i)) * SLOT);
      }
    };
    // gamma of this wave's rows: lane (m, g) needs rows 16 kt + 4g .. +3 of its tiles
    auto load_gam = [&](uint32_t rc, f32x4 (&x)[HKT]) {
#pragma unroll
      for (int i = 0; i < HKT; ++i) {
        const uint32_t off = (uint32_t)R::oGamBytes + 64u * (uint32_t)(WV * HKT + i);
        x[i] = buf_load16<f32x4>(rrec, 16u * (uint32_t)g + (off & 4095u), rc + (off & ~4095u));
      }
    };
    // this slice's V rows of the chunk whose record starts at rc (lane = token)
    const uint32_t vslice_off = (uint32_t)(R::oVBytes + (size_t)slice * R::vslice_bytes);
    auto load_v = [&](uint32_t rc, vload (&x)[NVL]) {
#pragma unroll
      for (int i = 0; i < NVL; ++i)
        x[i] = buf_load16<vload>(rrec, (uint32_t)lane * 16u * sizeof(MT) + 16u * i, rc + vslice_off);
    };
    auto stage_v = [&](const vload (&x)[NVL]) {
#pragma unroll
      for (int i = 0; i < NVL; ++i) *reinterpret_cast<vload*>(sV + lane * LDV + VL * i) = x[i];
    };

    // this wave's rows of S: local tile i is key tile WV * HKT + i
    f32x4 S[HKT];
#pragma unroll
    for (int i = 0; i < HKT; ++i) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (src != nullptr) {
        const float* ps = src + sbase + (size_t)(16 * (WV * HKT + i) + 4 * g) * V + m;
        x = f32x4{ps[0], ps[V], ps[2 * V], ps[3 * V]};
      }
      S[i] = x;
    }

    uint32_t rc0 = rec_off(rec_index(0));
    uint32_t rc1 = rec_off(rec_index(1));
    uint32_t rc2 = rec_off(rec_index(2));
    f32x4 U[NTT], O[NTT], Okeep[HT];
    frag Vf[NTS];
    vload vx[NVL];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) U[tt] = O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the U form: this slice's four U tiles of the chunk whose record starts at rc, as two
    // 16-byte pieces per lane (tiles 2p and 2p + 1)
    constexpr bool UW0 = UREC && WV == 0;
    const uint32_t uslice_off = (uint32_t)(R::oVBytes + (size_t)slice * R::vslice_bytes);
    auto load_u = [&](uint32_t rc, bf16x8 (&x)[2]) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        x[pp] = buf_load16<bf16x8>(rrec, (uint32_t)(pp * 64 + lane) * 16u, rc + uslice_off);
    };
    auto set_u = [&](const bf16x8 (&x)[2]) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        U[2 * pp] = __builtin_convertvector(__builtin_shufflevector(x[pp], x[pp], 0, 1, 2, 3), f32x4);
        U[2 * pp + 1] = __builtin_convertvector(__builtin_shufflevector(x[pp], x[pp], 4, 5, 6, 7), f32x4);
      }
    };
    bf16x8 unext[2];  // the U form: the next chunk's U, loaded a chunk ahead
    if constexpr (UW0) {
      load_u(rc0, unext);
      set_u(unext);
    } else if constexpr (WV == 0) {
      load_v(rc0, vx);
      stage_v(vx);
#pragma unroll
      for (int s = 0; s < NTS; ++s) Vf[s] = frag_t(sV, LDV, 0, s, lane);
      static_for<0, NTRI>([&](auto I) {
        constexpr int i = decltype(I)::value, tt = SH::tri_t(i), s = SH::tri_s(i);
        constexpr uint32_t off = (uint32_t)(R::oTb * sizeof(MT) + (size_t)(tt * NTS + s) * 64 * 16);
        U[tt] = M::mma(ldf(rc0, off), Vf[s], U[tt]);
      });
    }
    // gamma of this wave's rows: a chunk ahead, or (four waves, whose registers are scarcer) at
    // the chunk's start, NA operations before its first use
    constexpr bool GAHEAD = NW == 2;
    f32x4 gnext[GAHEAD ? HKT : 1], gcur[HKT];
    if constexpr (GAHEAD) load_gam(rc0, gnext);
    __builtin_amdgcn_sched_barrier(0);
    // ring slot P * NF + j holds operation j of the next chunk of parity P (two chunks in
    // flight), or slot j operation j of the next chunk (one chunk in flight)
    constexpr int RC = SS::RING_CHUNKS;
    static_assert(RC == 1 || RC == 2, "ring depth");
    frag ring[RC * NFW];
    static_for<0, NFW>([&](auto J) {
      constexpr int j = decltype(J)::value;
      ring[j] = ldf(next_rec(j) ? rc1 : rc0, frag_off(J));
    });
    if constexpr (RC == 2)
      static_for<0, NFW>([&](auto J) {
        constexpr int j = decltype(J)::value;
        ring[NFW + j] = ldf(next_rec(j) ? rc2 : rc1, frag_off(J));
      });
    __builtin_amdgcn_sched_barrier(0);
    uint32_t rc3 = rec_off(rec_index(3));
    int ri_pre = sRun[min(4, run - 1)];  // record index of chunk k + 4, read a chunk ahead
    if constexpr (WV == 0 && !UREC) load_v(rc1, vx);
    rsrc_t ro_prev = rows_rsrc(go, 0);

    // one chunk; PAR = k & 1 selects the ring half and the exchange buffers
    auto chunk = [&](auto PARc, const int k) {
      constexpr int par = decltype(PARc)::value;
      const rsrc_t ro = rows_rsrc(go, k);
      if constexpr (GAHEAD) {
#pragma unroll
        for (int i = 0; i < HKT; ++i) gcur[i] = gnext[i];
        load_gam(rc1, gnext);
      } else {
        load_gam(rc0, gcur);
      }
      if constexpr (UW0) load_u(rc1, unext);  // the next chunk's U
      __builtin_amdgcn_sched_barrier(0);

      frag Sb[HKS], Db[NTS];
      static_for<0, NFW>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (j < NA && j % (2 * NTT) == 0) {
          constexpr int s = j / (2 * NTT);
          if constexpr (KS == 32) Sb[s] = frag_from_acc(S[2 * s], S[2 * s + 1], MT());
          else Sb[s] = S[s];
        }
        if constexpr (j == NA) {
          // exchange the Delta partials (and the previous chunk's output partials)
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) sX[par][WV][tt][lane] = U[tt];
          lds_barrier();
          if constexpr (NW == 2) {
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) U[tt] += sX[par][1 - WV][tt][lane];
          } else {
            // every wave sums the partials in wave order, so all hold the same Delta
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
              f32x4 x = sX[par][0][tt][lane];
#pragma unroll
              for (int v = 1; v < NW; ++v) x += sX[par][v][tt][lane];
              U[tt] = x;
            }
          }
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            if constexpr (KS == 32) Db[s] = frag_from_acc(U[2 * s], U[2 * s + 1], MT());
            else Db[s] = U[s];
          }
          if (k > 0) {
#pragma unroll
            for (int i = 0; i < HT; ++i) {
              f32x4 o = Okeep[i];
#pragma unroll
              for (int v = 0; v < NW; ++v)
                if (v != WV) o += sO[par][v][WV * HT + i][lane];
              buf_store(ro_prev, o_voff, (uint32_t)(16 * (WV * HT + i)) * rowb, to_mt4<MT>(o));
            }
          }
        }
        if constexpr (j >= NA && j < NA + HKT) S[j - NA] *= gcur[j - NA];
        if constexpr (WV == 0 && !UREC && j == NA + NB / 2) {
          stage_v(vx);
#pragma unroll
          for (int s = 0; s < NTS; ++s) Vf[s] = frag_t(sV, LDV, 0, s, lane);
        }
        if constexpr (j == NA + NB) {
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) U[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (WV == 0 && !UREC) load_v(rc2, vx);
        }
        constexpr int slot = (RC == 2 ? par * NFW : 0) + j;
        const frag f = ring[slot];
        if constexpr (j < NA) {
          constexpr int s = j / (2 * NTT), r = j % (2 * NTT), tt = r % NTT;
          if constexpr (r < NTT) U[tt] = M::mma(f, Sb[s], U[tt]);  // [U] - W S, this half
          else O[tt] = M::mma(Sb[s], f, O[tt]);                    // S^T Qe^T, this half
        } else if constexpr (j < NA + NB) {
          constexpr int jj = j - NA, s = jj / HKT, i = jj % HKT;
          S[i] = M::mma(f, Db[s], S[i]);  // + Ktilde^T Delta, this wave's rows
        } else {
          constexpr int i = j - NA - NB;
          if constexpr (WV == 0) U[SH::tri_t(i)] = M::mma(f, Vf[SH::tri_s(i)], U[SH::tri_t(i)]);  // T'V, next chunk
          else O[SH::tri_t(i)] = M::mma(Db[SH::tri_s(i)], f, O[SH::tri_t(i)]);               // + Delta^T P^T
        }
        // refill: the same operation RC chunks on
        if constexpr (RC == 2) ring[slot] = ldf(next_rec(j) ? rc3 : rc2, frag_off(J));
        else ring[slot] = ldf(next_rec(j) ? rc2 : rc1, frag_off(J));
        __builtin_amdgcn_sched_barrier(0);
      });
      // waves without the T'V / P Delta operations never reach the reset at NA + NB: their next
      // Delta partial starts from zero here
      if constexpr (UW0) {
        set_u(unext);  // the U form: the next chunk's Delta partial starts from its U
      } else if constexpr (NFW == NA + NB) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) U[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // output partials: keep this wave's tiles, hand the other tiles to their owners
#pragma unroll
      for (int i = 0; i < HT; ++i) Okeep[i] = O[WV * HT + i];
#pragma unroll
      for (int t = 0; t < NTT; ++t)
        if (t / HT != WV) sO[par ^ 1][WV][t][lane] = O[t];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      ro_prev = ro;
      // records of chunks k + 1 .. k + 4 for the next chunk
      rc0 = rc1;
      rc1 = rc2;
      rc2 = rc3;
      rc3 = rec_off(__builtin_amdgcn_readfirstlane(ri_pre));
      ri_pre = sRun[min(k + 5, run - 1)];
    };
    for (int k = 0; k < run; k += 2) {
      chunk(std::integral_constant<int, 0>(), k);
      if (k + 1 < run) chunk(std::integral_constant<int, 1>(), k + 1);
    }
    // the last chunk's output
    lds_barrier();
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      f32x4 o = Okeep[i];
#pragma unroll
      for (int v = 0; v < NW; ++v)
        if (v != WV) o += sO[run & 1][v][WV * HT + i][lane];
      buf_store(ro_prev, o_voff, (uint32_t)(16 * (WV * HT + i)) * rowb, to_mt4<MT>(o));
    }
#pragma unroll
    for (int i = 0; i < HKT; ++i) {
      float* ps = p.state + sbase + (size_t)(16 * (WV * HKT + i) + 4 * g) * V + m;
      ps[0] = S[i][0];
      ps[V] = S[i][1];
      ps[2 * V] = S[i][2];
      ps[3 * V] = S[i][3];
    }
    // a sequence that goes on past the segment: its state before chunk seg_end, the checkpoint
    // of boundary seg_end / E (sequence-major table: entry index = chunk index in token order)
    if (p.ckpt != nullptr && en.depth + run < nc) {
      float* pc = p.ckpt + ((size_t)(seg_end / p.E - 1) * H + h) * (size_t)K * V + col0;
#pragma unroll
      for (int i = 0; i < HKT; ++i) {
        float* ps = pc + (size_t)(16 * (WV * HKT + i) + 4 * g) * V + m;
        ps[0] = S[i][0];
        ps[V] = S[i][1];
        ps[2 * V] = S[i][2];
        ps[3 * V] = S[i][3];
      }
    }
  };
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  if (wv == 0) body(std::integral_constant<int, 0>());
  else if (wv == 1) body(std::integral_constant<int, 1>());
  if constexpr (NW == 4) {
    if (wv == 2) body(std::integral_constant<int, 2>());
    else if (wv == 3) body(std::integral_constant<int, 3>());
  }
}

// ====================================================================== host side
// Compute units of the current device, queried once per device and cached (256 if the query
// fails).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool make_chunk_plan(int N, int64_t T, int H, int K, int V, bool bf16, ChunkPlan* p,
                     size_t max_rec_buf_bytes, bool running_state) {
  if (N <= 0 || H <= 0 || T < 0 || K <= 0 || V <= 0) return false;
  const int64_t es = bf16 ? 2 : 4;
  int64_t ub = (T + (int64_t)N * (CHUNK - 1)) / CHUNK;
  if (ub > T) ub = T;
  p->ub_entries = ub;
  // the fixed part (a multiple of 1 KB), then the chunk's V (CHUNK x V, a multiple of 1 KB)
  p->rec_bytes = ((3LL * CHUNK * K + 2LL * CHUNK * CHUNK) * es + 4LL * K + 1023) / 1024 * 1024 +
                 (int64_t)CHUNK * V * es;
  int64_t E = SEG_CHUNK_HEADS / H;
  if (max_rec_buf_bytes > 0) {  // a cap on the record buffer: fewer chunks per segment
    const int64_t cap = (int64_t)(max_rec_buf_bytes / ((size_t)H * p->rec_bytes));
    if (cap < E) E = cap;
    if (E < 1) return false;
  }
  if (E < 1) E = 1;
  if (ub > 0 && E > ub) E = ub;
  p->seg_entries = E;
  p->num_segs = ub > 0 ? (ub + E - 1) / E : 0;
  p->slots = N < E ? N : E;
  // V split: slices of 16 columns, one wave each
  p->n_slices = V / 16;
  p->vs = 16;
  // sequence-major once one sequence's chains at V = 128 (H heads x 8 slices) cover 256 CUs;
  // a function of H alone, so that calls on the same packing with other V (the scan's two
  // passes over one set of records) order the table alike
  p->seq_major = (int64_t)H * 8 >= 256 ? 1 : 0;
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
  if (running_state) off += al((size_t)N * H * K * V * 4);
  p->off_rec = off;
  p->rec_buf_bytes = (size_t)E * H * p->rec_bytes;
  off += p->rec_buf_bytes;
  // the state kernel addresses the record buffer and a chunk's rows with 32-bit offsets
  if (p->rec_buf_bytes >= (1ull << 31) || (int64_t)CHUNK * H * V * es >= (1ll << 31)) return false;
  p->total_bytes = off;
  return true;
}

template <int K, typename MT>
static hipError_t launch_chunk_t(const ChunkArgs& a, const ChunkPlan& pl, const RecordRegion* rr) {
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = reinterpret_cast<char*>(a.workspace);
  Entry* entries = reinterpret_cast<Entry*>(ws + pl.off_entries);
  int32_t* header = reinterpret_cast<int32_t*>(ws + pl.off_header);
  int32_t* basetab = reinterpret_cast<int32_t*>(ws + pl.off_basetab);
  int32_t* seg_first = reinterpret_cast<int32_t*>(ws + pl.off_seg_first);
  int32_t* seg_count = reinterpret_cast<int32_t*>(ws + pl.off_seg_count);
  float* run_state = a.final_state ? a.final_state : reinterpret_cast<float*>(ws + pl.off_state);
  // records: the plan's buffer, reused by every segment, or the caller's region with one slot
  // per segment; a region filled by an earlier call with more value columns serves a call
  // with fewer (the value slices lead the record's V part, the rest is never read)
  const int64_t need = (int64_t)(Rec<K, MT>::bytes + (size_t)CHUNK * a.dv * sizeof(MT));
  const int64_t rb = rr ? rr->rec_bytes : pl.rec_bytes;
  if (rr ? (rb < need || (rr->prep && rb != need) || rb % 1024 != 0) : rb != need)
    return hipErrorInvalidValue;
  const size_t seg_buf = (size_t)pl.seg_entries * a.num_heads * rb;
  if (seg_buf >= (1ull << 31)) return hipErrorInvalidValue;
  auto seg_rec = [&](int64_t s) -> char* {
    return rr ? rr->base + (size_t)s * seg_buf : ws + pl.off_rec;
  };

  SeqView sv{a.cu_seqlens, a.num_seqs, a.total_tokens};
  hipLaunchKernelGGL(table_kernel, dim3(a.num_seqs), dim3(256), 0, st, sv, a.num_heads,
                     (int64_t)a.dk * a.dv, pl.ub_entries, a.init_state, a.final_state, entries,
                     header, basetab, pl.seq_major);
  if (pl.num_segs == 0) return hipGetLastError();
  hipLaunchKernelGGL(segment_kernel, dim3(pl.num_segs), dim3(256), 0, st, entries, header,
                     pl.seg_entries, pl.slots, seg_first, seg_count);

  // The record's U form (U = T'V in place of T' and V): bf16, 128 value columns, the two-wave
  // chain, and records made and used in this call (the scan's second pass reads the first
  // pass's records, which carry V).
  constexpr bool UFORM_OK = sizeof(MT) == 2 && K <= 128 && SplitShape<K, MT>::OK;
  const bool urec = UFORM_OK && a.dv == 128 && rr == nullptr;
  const int64_t chains = pl.slots * a.num_heads;
  const int64_t chains8 = (chains + 7) / 8 * 8;
  const dim3 sgrid((unsigned)(chains8 * pl.n_slices));
  // prep: persistent workgroups, two per CU (its LDS and register budget), looping over tasks
  const int ncu = device_cu_count();
  const int64_t ptasks = pl.seg_entries * a.num_heads;
  const dim3 pgrid((unsigned)min(ptasks, (int64_t)2 * ncu));
  auto prep = [&](int64_t s, hipStream_t q) {
    if constexpr (K == 256) {  // the fp32 record kernel of 256 key channels
      const Rec256Params rp{a.q, a.k, a.v, a.g, a.beta, entries, header, a.num_heads, a.dv,
                            s * pl.seg_entries, pl.seg_entries, seg_rec(s), rb, a.options};
      launch_rec256(rp, q);
    } else {
      PrepParams pp{a.q, a.k, a.g, a.beta, entries, header, a.num_heads, s * pl.seg_entries,
                    pl.seg_entries, seg_rec(s), rb, a.options, a.v, a.dv};
      const bool v256 = (size_t)a.dv * sizeof(MT) == 256;
      if constexpr (UFORM_OK) {
        if (urec) {
          if (a.options == 0)
            hipLaunchKernelGGL((prep_kernel<K, MT, false, true, true>), pgrid, dim3(PREP_THREADS), 0, q, pp);
          else
            hipLaunchKernelGGL((prep_kernel<K, MT, true, true, true>), pgrid, dim3(PREP_THREADS), 0, q, pp);
          return;
        }
      }
      if (a.options == 0 && v256)
        hipLaunchKernelGGL((prep_kernel<K, MT, false, true>), pgrid, dim3(PREP_THREADS), 0, q, pp);
      else if (a.options == 0)
        hipLaunchKernelGGL((prep_kernel<K, MT, false, false>), pgrid, dim3(PREP_THREADS), 0, q, pp);
      else if (v256)
        hipLaunchKernelGGL((prep_kernel<K, MT, true, true>), pgrid, dim3(PREP_THREADS), 0, q, pp);
      else
        hipLaunchKernelGGL((prep_kernel<K, MT, true, false>), pgrid, dim3(PREP_THREADS), 0, q, pp);
    }
  };
  auto state = [&](int64_t s, hipStream_t q) -> bool {
    StateParams sp{a.v, a.o, a.init_state, run_state, entries, header, basetab,
                   seg_first + s * pl.slots, seg_count + s, s * pl.seg_entries, pl.seg_entries,
                   a.num_heads, a.dv, pl.n_slices, chains, seg_rec(s), (uint32_t)rb,
                   (uint32_t)seg_buf, pl.seq_major, pl.seq_major ? a.ckpt : nullptr};
    if (pl.vs != 16) return false;
    if constexpr (UFORM_OK) {
      if (urec) {
        hipLaunchKernelGGL((state_split_kernel<K, MT, true>), sgrid, dim3(SplitShape<K, MT>::THREADS), 0, q, sp);
        return true;
      }
    }
    if constexpr (SplitShape<K, MT>::OK)
      hipLaunchKernelGGL((state_split_kernel<K, MT>), sgrid, dim3(SplitShape<K, MT>::THREADS), 0, q, sp);
    else
      hipLaunchKernelGGL((state_kernel<K, MT>), sgrid, dim3(STATE_THREADS), 0, q, sp);
    return true;
  };

  // Segments run in order on the caller's stream, each kernel with the whole device: the
  // prep kernel fills the record buffer, then the state kernel consumes it.
  const bool run_prep = !rr || rr->prep;
  for (int64_t s = 0; s < pl.num_segs; ++s) {
    if (run_prep) prep(s, st);
    if (!state(s, st)) return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, const ChunkPlan& pl, const RecordRegion* rr) {
  if (a.dtype_bf16) {
    if (a.dk == 32) return launch_chunk_t<32, bf16>(a, pl, rr);
    if (a.dk == 64) return launch_chunk_t<64, bf16>(a, pl, rr);
    if (a.dk == 128) return launch_chunk_t<128, bf16>(a, pl, rr);
    if (a.dk == 256) return launch_chunk_t<256, bf16>(a, pl, rr);
  } else {
    if (a.dk == 32) return launch_chunk_t<32, float>(a, pl, rr);
    if (a.dk == 64) return launch_chunk_t<64, float>(a, pl, rr);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
