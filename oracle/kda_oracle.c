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

int kda_oracle_max_threads(void) { return pick_threads(0); }
