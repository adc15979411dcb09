/*
 * KDA oracle: plain, slow, token-by-token fp64 reference of Kimi Delta Attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link, load or
 * call this file: only the test-suite, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code, header, table or constant with the HIP path.
 *
 * Sources (cited by page title and section; no page prints code that is copied here):
 *  [TB]  "Kimi Linear's Hybrid Linear Attention Architecture: A Technical Breakdown",
 *        section 3.3 "The Combined Form: Fine-Grained Gating": the update
 *        S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + (write of v_t along k_t), and the
 *        note in the same section that decay is applied to the old memory first, erasure
 *        and writing after.
 *  [WP]  "Kimi Linear: How Moonshot AI Built a Hybrid Attention Architecture That Beats
 *        Full Attention", the update-rule code block: S_t = (I - b k k^T) Diag(a) S + b k v^T,
 *        which fixes the orientation: S is (key dim K) x (value dim V), rows are key channels.
 *  [KX]  "Kimi Linear" explainer, "Step 4: Query": the output is read from the state after
 *        the token's write.
 *
 * Readings (see the design notes): alpha = exp(log_alpha) per key channel; beta is one
 * scalar per token and head; no query scaling; no normalisation of q or k; o_t = S_t^T q_t
 * with S_t the state after token t; state never crosses a sequence boundary. Inputs arrive
 * in fp64: the exact values the GPU received, or the fp64 result of the input options
 * (gate and beta activations, q/k normalisation), which the Python wrapper applies first.
 *
 * Step for one token (all in fp64):
 *   1. S[c][:] *= exp(g[c])                   decay first            [TB] 3.3
 *   2. u = S^T k                              current prediction for key k
 *   3. S += beta * k (v - u)^T                erase along k, then write  [TB] 3.3, [WP]
 *      (equal to (I - beta k k^T) S' + beta k v^T with S' the decayed state)
 *   4. o = S^T q                              read after write       [KX] Step 4
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of one (sequence, head). S is K x V row-major, fp64. */
static void oracle_token(double* S, int K, int V, const double* q, const double* k,
                         const double* v, const double* g, double beta, double* o,
                         double* u /* scratch, V */) {
  /* 1. per-channel decay of the old memory */
  for (int c = 0; c < K; ++c) {
    const double a = exp(g[c]);
    double* row = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) row[j] *= a;
  }
  /* 2. prediction of the decayed memory along k */
  for (int j = 0; j < V; ++j) u[j] = 0.0;
  for (int c = 0; c < K; ++c) {
    const double kc = k[c];
    const double* row = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) u[j] += row[j] * kc;
  }
  /* 3. erase along k and write v (delta correction) */
  for (int c = 0; c < K; ++c) {
    const double bk = beta * k[c];
    double* row = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) row[j] += bk * (v[j] - u[j]);
  }
  /* 4. read with the query after the write */
  for (int j = 0; j < V; ++j) o[j] = 0.0;
  for (int c = 0; c < K; ++c) {
    const double qc = q[c];
    const double* row = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) o[j] += row[j] * qc;
  }
}

static int pick_threads(int32_t requested) {
#ifdef _OPENMP
  if (requested > 0) return requested;
  return omp_get_max_threads();
#else
  (void)requested;
  return 1;
#endif
}

/*
 * Full forward over packed variable-length sequences.
 *   q, k, g : [T_total][H][K]  double
 *   v       : [T_total][H][V]
 *   beta    : [T_total][H]
 *   cu_seqlens : [N+1] int64, sequence n is tokens cu[n] .. cu[n+1]-1
 *   init_state : [N][H][K][V] fp64 or NULL (zeros)
 *   heads, num_sel : optional subset of heads to compute (NULL = all H, in order)
 *   o           : [T_total][num_sel][V] fp64 out
 *   final_state : [N][num_sel][K][V] fp64 out (may be NULL)
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_fwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const int64_t* cu_seqlens, int32_t num_seqs,
                   int32_t num_heads, int32_t dk, int32_t dv, const double* init_state,
                   const int32_t* heads, int32_t num_sel, double* o, double* final_state,
                   int32_t num_threads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return -1;
  if (num_seqs <= 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!heads) num_sel = num_heads;
  if (num_sel <= 0) return -1;
  const int K = dk, V = dv, H = num_heads;
  const int64_t pairs = (int64_t)num_seqs * num_sel;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(num_threads)) reduction(| : bad)
  for (int64_t p = 0; p < pairs; ++p) {
    const int n = (int)(p / num_sel);
    const int hs = (int)(p % num_sel);
    const int h = heads ? heads[hs] : hs;
    if (h < 0 || h >= H) { bad = 1; continue; }
    double* S = (double*)malloc(sizeof(double) * ((size_t)K * V + V));
    if (!S) { bad = 1; continue; }
    double* u = S + (size_t)K * V;
    if (init_state)
      memcpy(S, init_state + ((size_t)n * H + h) * K * V, sizeof(double) * K * V);
    else
      memset(S, 0, sizeof(double) * K * V);
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      const size_t th = (size_t)t * H + h;
      oracle_token(S, K, V, q + th * K, k + th * K, v + th * V, g + th * K,
                   beta[th], o + ((size_t)t * num_sel + hs) * V, u);
    }
    if (final_state)
      memcpy(final_state + ((size_t)n * num_sel + hs) * K * V, S, sizeof(double) * K * V);
    free(S);
  }
  return bad ? -1 : 0;
}

/*
 * One recurrent decode step for N sequences x H heads, state updated in place.
 *   q, k, g : [N][H][K], v : [N][H][V], beta : [N][H]  (double)
 *   state   : [N][H][K][V] fp64, in/out
 *   o       : [N][H][V] fp64 out
 */
int kda_oracle_step(const double* q, const double* k, const double* v, const double* g,
                    const double* beta, int32_t num_seqs, int32_t num_heads, int32_t dk,
                    int32_t dv, double* state, double* o, int32_t num_threads) {
  if (!q || !k || !v || !g || !beta || !state || !o) return -1;
  if (num_seqs <= 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return -1;
  const int K = dk, V = dv;
  const int64_t pairs = (int64_t)num_seqs * num_heads;
  int bad = 0;
#pragma omp parallel for schedule(static) num_threads(pick_threads(num_threads)) reduction(| : bad)
  for (int64_t p = 0; p < pairs; ++p) {
    double* u = (double*)malloc(sizeof(double) * V);
    if (!u) { bad = 1; continue; }
    oracle_token(state + (size_t)p * K * V, K, V, q + (size_t)p * K, k + (size_t)p * K,
                 v + (size_t)p * V, g + (size_t)p * K, beta[p], o + (size_t)p * V, u);
    free(u);
  }
  return bad ? -1 : 0;
}

/*
 * Gradients of the forward above (reverse mode, written from the four steps of one token).
 * With the loss L = sum(do * o) + sum(dfinal * S_final), L_t = dL/dS_t accumulates backwards
 * from dfinal. For token t, with S' = Diag(a) S_{t-1}, u = S'^T k, r = v - u:
 *   L_t  += q do^T                       (o = S_t^T q)
 *   dq    = S_t do
 *   dbeta = k^T L_t r,   dk = beta L_t r,   dv = beta L_t^T k,   du = -dv
 *   dS'   = L_t + k du^T,   dk += S' du  (u = S'^T k)
 *   dlog_a[c] = a[c] sum_j S_{t-1}[c][j] dS'[c][j],   L_{t-1} = Diag(a) dS'
 * and d init_state = L before the sequence's first token. The states S_t are recomputed by a
 * forward pass over the sequence and kept (one K x V matrix per token).
 *   dout  : [T_total][H][V]      dfinal : [N][H][K][V] or NULL (zero)
 *   dq, dk, dg : [T_total][H][K]   dv : [T_total][H][V]   dbeta : [T_total][H]
 *   dinit : [N][H][K][V] (may be NULL)
 */
int kda_oracle_bwd(const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const int64_t* cu_seqlens, int32_t num_seqs,
                   int32_t num_heads, int32_t dk_, int32_t dv_, const double* init_state,
                   const double* dout, const double* dfinal, double* dq, double* dk, double* dv,
                   double* dg, double* dbeta, double* dinit, int32_t num_threads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !dout || !dq || !dk || !dv || !dg || !dbeta)
    return -1;
  if (num_seqs <= 0 || num_heads <= 0 || dk_ <= 0 || dv_ <= 0) return -1;
  const int K = dk_, V = dv_, H = num_heads;
  const int64_t pairs = (int64_t)num_seqs * H;
  const size_t KV = (size_t)K * V;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(num_threads)) reduction(| : bad)
  for (int64_t p = 0; p < pairs; ++p) {
    const int n = (int)(p / H), h = (int)(p % H);
    const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1], L = t1 - t0;
    double* St = (double*)malloc(sizeof(double) * ((size_t)(L + 1) * KV + 2 * KV + 4 * (size_t)(K + V)));
    if (!St) { bad = 1; continue; }
    double* Lam = St + (size_t)(L + 1) * KV;  /* dL/dS_t */
    double* dS1 = Lam + KV;
    double* u = dS1 + KV;
    double* r = u + V;
    double* dr = r + V;
    double* tmpk = dr + V;
    /* forward: St[i] = state after token t0 + i - 1 (St[0] = initial state) */
    if (init_state) memcpy(St, init_state + ((size_t)n * H + h) * KV, sizeof(double) * KV);
    else memset(St, 0, sizeof(double) * KV);
    for (int64_t i = 0; i < L; ++i) {
      const size_t th = (size_t)(t0 + i) * H + h;
      double* S = St + (size_t)(i + 1) * KV;
      memcpy(S, St + (size_t)i * KV, sizeof(double) * KV);
      double* o_unused = tmpk;  /* the forward output is not needed here */
      oracle_token(S, K, V, q + th * K, k + th * K, v + th * V, g + th * K, beta[th], o_unused, u);
    }
    /* backward */
    if (dfinal) memcpy(Lam, dfinal + ((size_t)n * H + h) * KV, sizeof(double) * KV);
    else memset(Lam, 0, sizeof(double) * KV);
    for (int64_t i = L - 1; i >= 0; --i) {
      const size_t th = (size_t)(t0 + i) * H + h;
      const double* qt = q + th * K;
      const double* kt = k + th * K;
      const double* vt = v + th * V;
      const double* gt = g + th * K;
      const double* dot = dout + th * V;
      const double b = beta[th];
      const double* Sprev = St + (size_t)i * KV;
      const double* Scur = St + (size_t)(i + 1) * KV;
      /* L_t += q do^T; dq = S_t do */
      for (int c = 0; c < K; ++c)
        for (int j = 0; j < V; ++j) Lam[(size_t)c * V + j] += qt[c] * dot[j];
      for (int c = 0; c < K; ++c) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) acc += Scur[(size_t)c * V + j] * dot[j];
        dq[th * K + c] = acc;
      }
      /* u = (Diag(a) S_{t-1})^T k, r = v - u */
      for (int j = 0; j < V; ++j) u[j] = 0.0;
      for (int c = 0; c < K; ++c) {
        const double a = exp(gt[c]);
        for (int j = 0; j < V; ++j) u[j] += a * Sprev[(size_t)c * V + j] * kt[c];
      }
      for (int j = 0; j < V; ++j) r[j] = vt[j] - u[j];
      /* dbeta = k^T L r; dk = beta L r; dr = beta L^T k */
      double db = 0.0;
      for (int c = 0; c < K; ++c) {
        double lr = 0.0;
        for (int j = 0; j < V; ++j) lr += Lam[(size_t)c * V + j] * r[j];
        db += kt[c] * lr;
        dk[th * K + c] = b * lr;
      }
      dbeta[th] = db;
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c) acc += Lam[(size_t)c * V + j] * kt[c];
        dr[j] = b * acc;
        dv[th * V + j] = dr[j];
      }
      /* dS' = L + k du^T with du = -dr; dk += S' du */
      for (int c = 0; c < K; ++c) {
        const double a = exp(gt[c]);
        double acc = 0.0;
        for (int j = 0; j < V; ++j) {
          dS1[(size_t)c * V + j] = Lam[(size_t)c * V + j] - kt[c] * dr[j];
          acc -= a * Sprev[(size_t)c * V + j] * dr[j];
        }
        dk[th * K + c] += acc;
      }
      /* dlog a and L_{t-1} = Diag(a) dS' */
      for (int c = 0; c < K; ++c) {
        const double a = exp(gt[c]);
        double acc = 0.0;
        for (int j = 0; j < V; ++j) acc += Sprev[(size_t)c * V + j] * dS1[(size_t)c * V + j];
        dg[th * K + c] = a * acc;
        for (int j = 0; j < V; ++j) Lam[(size_t)c * V + j] = a * dS1[(size_t)c * V + j];
      }
    }
    if (dinit) memcpy(dinit + ((size_t)n * H + h) * KV, Lam, sizeof(double) * KV);
    free(St);
  }
  return bad ? -1 : 0;
}

int kda_oracle_max_threads(void) { return pick_threads(0); }
