/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library, libkda.so.
 *
 * The operator (per sequence and head, state S in R^{K x V}, rows = key channels):
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t
 * Update rule: "Kimi Linear's Hybrid Linear Attention Architecture: A Technical Breakdown",
 * section 3.3 (per-channel decay first, then directional erase and write); orientation from
 * the update-rule code block of "Kimi Linear: How Moonshot AI Built a Hybrid Attention
 * Architecture That Beats Full Attention"; the query reads the state after the token's write
 * ("Kimi Linear" explainer, "Step 4: Query").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library never allocates
 *    or frees device memory and keeps no per-call state. Tensor pointers must be 16-byte
 *    aligned, except beta, cu_seqlens and a scalar gate (KDA_OPT_SCALAR_GATE), which need
 *    only their element alignment.
 *  - Layouts are row-major and token-major. q, k, log_alpha: [rows][H][K]; v: [rows][H][V];
 *    beta: [rows][H]; o: [rows][H][V]; states: [N][H][K][V] fp32 (element (c, j) of S at
 *    c*V + j, c = key channel, j = value channel).
 *  - dtype selects the element type of q, k, v, log_alpha, beta and o (fp32 or bf16). States
 *    are always fp32. Outputs are rounded to nearest even when dtype is bf16.
 *  - log_alpha is the natural log of the per-channel decay alpha (expected <= 0); no query
 *    scale is applied and q, k are used as given (no normalisation inside). The _ex entry
 *    points take options that change how these inputs are read (KDA_OPT_* below).
 *  - Supported head dims: kda_chunk_fwd K in {32, 64, 128, 256}, V in {32, 64, 128, 256};
 *    K = 256, and fp32 inputs at K = 128, run the wide-key path below (no input options);
 *    kda_decode_step K, V in {32, 64, 128, 256}. Other values give KDA_ERROR_NOT_SUPPORTED.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *    returns without waiting. Argument errors are reported synchronously before anything is
 *    enqueued; a failed launch gives KDA_ERROR_LAUNCH. Values are not checked on the device:
 *    NaN/Inf propagate. No exception crosses the ABI.
 *  - Calls on different streams are independent; calls that share a workspace or a state
 *    buffer must be ordered by the caller.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_SUCCESS = 0,
  KDA_ERROR_INVALID_VALUE = 1,       /* NULL pointer, misaligned pointer, bad size/count */
  KDA_ERROR_NOT_SUPPORTED = 2,       /* unsupported head dims, dtype or option bits */
  KDA_ERROR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below kda_chunk_fwd_workspace_size */
  KDA_ERROR_LAUNCH = 4               /* a kernel launch or stream operation failed */
} kda_status;

typedef enum {
  KDA_DTYPE_F32 = 0,  /* IEEE fp32 */
  KDA_DTYPE_BF16 = 1  /* bfloat16 */
} kda_dtype;

/*
 * Input options of kda_chunk_fwd_ex and kda_decode_step_ex: a bitwise OR of these values, 0 for
 * the operator exactly as above. They fold the elementwise steps that produce the operator's
 * inputs into the kernels, so that the raw tensors are read once. Unknown bits give
 * KDA_ERROR_NOT_SUPPORTED.
 *  KDA_OPT_SCALAR_GATE  log_alpha holds one value per token and head, [rows][H], and every key
 *                       channel of the head decays by it: the gated delta rule, whose gate scales
 *                       the whole memory ("A Technical Breakdown", section 3.2).
 *  KDA_OPT_GATE_LOGITS  log_alpha holds the pre-activation z of alpha = sigmoid(z) (the gate of
 *                       the "Kimi Linear" explainer, "Step 2: Per-Channel Decay"); the kernels
 *                       form log alpha = -log(1 + e^{-z}) without overflow for any finite z.
 *  KDA_OPT_BETA_LOGITS  beta holds x and the write strength is sigmoid(x).
 *  KDA_OPT_L2NORM_QK    q and k are each scaled to unit L2 norm over the K key channels, per
 *                       token and head: x / sqrt(sum_c x_c^2 + 1e-6).
 * The options combine freely (e.g. SCALAR_GATE | GATE_LOGITS: one logit per token and head).
 */
enum {
  KDA_OPT_SCALAR_GATE = 1u,
  KDA_OPT_GATE_LOGITS = 2u,
  KDA_OPT_BETA_LOGITS = 4u,
  KDA_OPT_L2NORM_QK = 8u
};

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status s);

/*
 * Workspace bytes kda_chunk_fwd needs for this shape (0 if the arguments are invalid).
 * The value depends only on the arguments; it covers the device chunk table, a running state
 * and one chunk-record buffer, and is bounded (about 170 MB at H=32, K=V=128, bf16) plus
 * 32 bytes per chunk and 4*N*H*K*V bytes, whatever the sequence length. On the wide-key path
 * (K = 256) it holds an fp32 record for every chunk and head instead: 214 KB + 256 V
 * bytes per 64 tokens and head (e.g. 9.2 GB at H = 32, V = 256 and 65,536 tokens).
 */
size_t kda_chunk_fwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype);

/*
 * Chunkwise KDA forward (prefill / training forward) over packed variable-length sequences.
 * Method: "A Technical Breakdown", section 4 "Hardware-Friendly Chunkwise Computation"
 * (in-chunk cumulative decay, WY / UT representation of the chunk's rank-1 updates through
 * a triangular solve, state passing between chunks, masked intra-chunk output).
 *
 *   q, k, log_alpha : [T_total][H][K]   dtype
 *   v               : [T_total][H][V]   dtype
 *   beta            : [T_total][H]      dtype
 *   init_state      : [N][H][K][V] fp32, or NULL for zero initial states
 *   cu_seqlens      : device int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = T_total;
 *                     sequence n is tokens cu[n] .. cu[n+1]-1. NULL means N sequences of
 *                     equal length T_total / N (T_total must then be divisible by N).
 *                     A malformed cu_seqlens is undefined behaviour (it is not read on the host).
 *   o               : [T_total][H][V]   dtype, written for every token
 *   final_state     : [N][H][K][V] fp32 out, or NULL. May be the same pointer as init_state
 *                     (then updated in place); other partial overlaps are not allowed.
 *   workspace       : device buffer of at least kda_chunk_fwd_workspace_size(...) bytes,
 *                     256-byte aligned, contents need not be initialised; used only during
 *                     the call's stream work.
 * A sequence of length 0 gets final = init (or zero). T_total = 0 is a no-op apart from that.
 * States never cross sequence boundaries.
 * Numerical domain: the in-chunk factorisation keeps every factor within fp32 range when the
 * decay of any key channel over 16 consecutive tokens is at most e^80 (e.g. log_alpha >= -5
 * everywhere); stronger decays can overflow to Inf/NaN.
 * K = 256, and fp32 inputs at K = 128, run a separate path in fp32 (the chunk's products over
 * the key channels in parts of 64, every decay factor formed pairwise within the chunk, so any
 * decay is in range); it takes options = 0 only (other options give KDA_ERROR_NOT_SUPPORTED).
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* init_state, const int32_t* cu_seqlens,
                         int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                         int32_t dv, kda_dtype dtype, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd with input options (KDA_OPT_*); options = 0 is kda_chunk_fwd. With
 * KDA_OPT_SCALAR_GATE, log_alpha is [T_total][H]. The workspace size does not depend on the
 * options.
 */
kda_status kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                            const void* beta, const float* init_state, const int32_t* cu_seqlens,
                            int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                            int32_t dv, kda_dtype dtype, uint32_t options, void* o,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Chunk-parallel scan variant of kda_chunk_fwd_ex for long sequences over few heads. Each of the
 * num_seqs sequences (equal lengths total_tokens / num_seqs, no cu_seqlens) splits into
 * num_groups groups of whole 64-token chunks; one chunked pass over all groups with the values
 * [v | 0] and the initial state [0 | I] yields each group's end state from zero, B_g, and its
 * state transition, M_g (K x K); a combine forms every group's initial state
 * S_in(g + 1) = M_g S_in(g) + B_g; a second pass runs all groups from those states ("Kimi Linear"
 * explainer, "DPLR Chunked Parallel"); it reads the records the first pass built. Results
 * equal kda_chunk_fwd_ex's up to rounding. It runs the sequential state sweep twice (the first
 * time with dv + dk columns) and pays off when num_seqs * num_heads * dv / 16 is far below the
 * GPU's 256 CUs (e.g. one sequence of 64k tokens over 1 to 4 heads with num_groups = 16).
 * Requires dk == dv in {32, 64, 128}; other shapes give KDA_ERROR_NOT_SUPPORTED.
 * total_tokens must be divisible by num_seqs and num_groups >= 1 (else
 * KDA_ERROR_INVALID_VALUE). The workspace needs kda_chunk_fwd_scan_workspace_size bytes
 * (it holds every (chunk, head) record of the first pass, about 100 KB per 64 tokens and head
 * at dk = dv = 128 bf16, plus [v | 0], a scratch output and the groups' states). Other
 * arguments as for kda_chunk_fwd_ex.
 */
size_t kda_chunk_fwd_scan_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                         int32_t num_heads, int32_t dk, int32_t dv,
                                         kda_dtype dtype, int32_t num_groups);
kda_status kda_chunk_fwd_scan(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, const float* init_state, int32_t num_seqs,
                              int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                              kda_dtype dtype, uint32_t options, int32_t num_groups, void* o,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Training backward of kda_chunk_fwd (options = 0): the gradients of
 *     L = sum(d_o * o) + sum(d_final_state * final_state)
 * with respect to q, k, v, log_alpha, beta and init_state, for the forward on the same inputs
 * (same q, k, v, log_alpha, beta, init_state, cu_seqlens and shapes), by reverse mode through
 * the chunk form ("A Technical Breakdown", section 4; "Kimi Linear" explainer, "WY
 * Representation"): the chunk-start states are recomputed, the state gradient is carried
 * backwards chunk by chunk, and the per-token gradients of each chunk follow from it. All of
 * it runs in fp32.
 *   d_o            : [rows][H][V], dtype
 *   d_final_state  : [N][H][K][V] fp32, or NULL (zero)
 *   grad_q, grad_k, grad_log_alpha : [rows][H][K] fp32 (written)
 *   grad_v         : [rows][H][V] fp32 (written)
 *   grad_beta      : [rows][H] fp32 (written; 4-byte aligned)
 *   grad_init_state: [N][H][K][V] fp32 (written), or NULL (not needed); with a NULL init_state
 *                    it is still the gradient with respect to the zero initial state.
 * Gradients of rows past the end of every sequence are not written (there are none: cu_seqlens
 * covers all rows). No gradient buffer may overlap an input or another gradient
 * (KDA_ERROR_INVALID_VALUE). Head dims K, V in {32, 64, 128}, both dtypes; others give
 * KDA_ERROR_NOT_SUPPORTED. The workspace (kda_chunk_bwd_workspace_size bytes, 256-byte aligned)
 * holds, for every (chunk, head), an fp32 record, the chunk-start state and the chunk-end state
 * gradient and scratch: about 500 KB per 64 tokens and head at K = V = 128.
 */
size_t kda_chunk_bwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype);
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* init_state, const int32_t* cu_seqlens,
                         int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                         int32_t dv, kda_dtype dtype, const void* d_o,
                         const float* d_final_state, float* grad_q, float* grad_k, float* grad_v,
                         float* grad_log_alpha, float* grad_beta, float* grad_init_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent KDA token step per (sequence, head), state updated in place (decode).
 * The decay, prediction u = (Diag(alpha) S)^T k, erase-and-write and read are fused into one
 * pass that streams each fp32 state once from HBM and writes it once.
 *   q, k, log_alpha : [N][H][K] dtype;  v : [N][H][V] dtype;  beta : [N][H] dtype
 *   state           : [N][H][K][V] fp32, read and overwritten
 *   o               : [N][H][V] dtype out (must not overlap the other buffers)
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* beta, float* state, void* o, int32_t num_seqs,
                           int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                           void* stream);

/*
 * kda_decode_step with input options (KDA_OPT_*); options = 0 is kda_decode_step. With
 * KDA_OPT_SCALAR_GATE, log_alpha is [N][H].
 */
kda_status kda_decode_step_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, float* state, void* o, int32_t num_seqs,
                              int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                              uint32_t options, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
