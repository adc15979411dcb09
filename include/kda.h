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
 *    fp32 inputs at K >= 128 run the wide-key path below;
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
 * The value depends only on the arguments. On the main path (bf16 inputs, and fp32 inputs at
 * K <= 64) it covers the device chunk table, a running state and one chunk-record buffer
 * reused by every segment of the call: about 170 MB at H=32, K=V=128, bf16 (300 MB at
 * K=V=256), plus 32 bytes per chunk and 4*N*H*K*V bytes, whatever the sequence length.
 * The wide-key path (fp32 inputs at K >= 128) forms fp32 records one segment of 512 MiB at a
 * time: under about 1 GB at H = 32 whatever the length.
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
 * Numerical domain: every log_alpha <= 0 gives finite results. In-chunk decay factors are
 * formed relative to 16-token sub-block references so that each is at most 1; a diagonal
 * sub-block whose decay exceeds 2^96 on some channel is formed from running products of the
 * per-token decays instead (exact up to rounding; vanishing terms underflow to zero).
 * Positive log_alpha values are accepted but lie outside this guarantee.
 * bf16 inputs at K = 256 run the main path with an fp32 record kernel: the chunk's sums over
 * the key channels in parts of 64, the off-diagonal 16 x 16 blocks of A and P on the fp32
 * matrix cores with the decay split at a block boundary (both factors at most 1), the diagonal
 * blocks pairwise, then the bf16 chain with four waves per 16 value columns (input options are
 * applied in fp32 as that kernel reads the raw inputs). fp32 inputs at K >= 128 run a separate
 * path in fp32 (the same record arithmetic, the chain on the fp32 matrix cores) that forms the
 * chunks' records one segment of chunks at a time (512 MiB of records), so its workspace stays
 * under about 1 GB at 32 heads whatever the length; with input options a separate pass forms
 * the processed q, k, log alpha and beta of each segment's tokens in fp32 first. Every decay
 * factor on either path is at most 1, so any log_alpha <= 0 is in range.
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
 * kda_chunk_fwd_ex without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It calls no allocating routine. Its scratch is one fixed array of 128 MiB inside the library,
 * held on each device the entry point runs on until the process ends; it holds the chunk
 * table and one record buffer, which is capped to fit, so a call runs in more (shorter)
 * segments than kda_chunk_fwd_ex. Results are the same as kda_chunk_fwd_ex's.
 * Differences from kda_chunk_fwd_ex:
 *  - final_state is required (KDA_ERROR_INVALID_VALUE if NULL): it carries the running state;
 *  - shapes on the wide-key path (fp32 inputs at K >= 128) give KDA_ERROR_NOT_SUPPORTED;
 *  - a shape whose chunk table plus one chunk record per head exceeds the scratch gives
 *    KDA_ERROR_WORKSPACE_TOO_SMALL (e.g. more than about 2^24 chunks in total);
 *  - every call on a device shares that device's scratch: calls that overlap in time on one
 *    device (different streams, or different host threads without ordering) race and must be
 *    serialised by the caller.
 * Other arguments, layouts and errors as for kda_chunk_fwd_ex.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta, const float* init_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                                 uint32_t options, void* o, float* final_state, void* stream);

/*
 * Chunk-parallel scan variant of kda_chunk_fwd_ex for long sequences over few heads. Each of the
 * num_seqs sequences (equal lengths total_tokens / num_seqs; kda_chunk_fwd_scan_ex below takes
 * cu_seqlens) splits into num_groups groups of whole 64-token chunks (its length over
 * num_groups, rounded up to whole chunks, per group; trailing groups may be short or empty); one chunked pass over all groups with the values
 * [v | 0] and the initial state [0 | I] yields each group's end state from zero, B_g, and its
 * state transition, M_g (K x K); a combine forms every group's initial state
 * S_in(g + 1) = M_g S_in(g) + B_g; a second pass runs all groups from those states ("Kimi Linear"
 * explainer, "DPLR Chunked Parallel"); it reads the records the first pass built. Results
 * equal kda_chunk_fwd_ex's up to rounding. It runs the sequential state sweep twice (the first
 * time with dv + dk columns, rounded up to a power of two) and pays off when
 * num_seqs * num_heads * dv / 16 is far below the GPU's 256 CUs (e.g. one sequence of 64k
 * tokens over 1 to 4 heads with num_groups = 16). Requires dk in {32, 64, 128} and
 * dk + dv <= 256 (fp32 inputs: dk <= 64); other shapes give KDA_ERROR_NOT_SUPPORTED.
 * total_tokens must be divisible by num_seqs and num_groups >= 1 (else
 * KDA_ERROR_INVALID_VALUE). The workspace needs kda_chunk_fwd_scan_workspace_size bytes (the
 * same for any split of total_tokens into num_seqs sequences)
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
 * kda_chunk_fwd_scan over packed variable-length sequences: cu_seqlens ([num_seqs + 1] int32,
 * device, 4-byte aligned, non-decreasing from 0 to total_tokens) gives each sequence's tokens,
 * and each splits into num_groups groups of its own; NULL is kda_chunk_fwd_scan. The workspace
 * size is kda_chunk_fwd_scan_workspace_size's.
 */
kda_status kda_chunk_fwd_scan_ex(const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta, const float* init_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                 kda_dtype dtype, uint32_t options, int32_t num_groups, void* o,
                                 float* final_state, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Training backward of kda_chunk_fwd (options = 0; kda_chunk_bwd_ex below takes input options):
 * the gradients of
 *     L = sum(d_o * o) + sum(d_final_state * final_state)
 * with respect to q, k, v, log_alpha, beta and init_state, for the forward on the same inputs
 * (same q, k, v, log_alpha, beta, init_state, cu_seqlens and shapes), by reverse mode through
 * the chunk form ("A Technical Breakdown", section 4; "Kimi Linear" explainer, "WY
 * Representation"): the chunk-start states are recomputed, the state gradient is carried
 * backwards chunk by chunk, and the per-token gradients of each chunk follow from it. Every
 * stored value and every sum is fp32; the products of the two state chains and of S and X
 * with the chunk's rows run on the bf16 matrix cores with each fp32 operand split into two
 * bf16 parts (about 2^-16 relative error per product), the rest on the fp32 matrix cores.
 *   d_o            : [rows][H][V], dtype
 *   d_final_state  : [N][H][K][V] fp32, or NULL (zero)
 *   grad_q, grad_k, grad_log_alpha : [rows][H][K] fp32 (written)
 *   grad_v         : [rows][H][V] fp32 (written)
 *   grad_beta      : [rows][H] fp32 (written; 4-byte aligned)
 *   grad_init_state: [N][H][K][V] fp32 (written), or NULL (not needed); with a NULL init_state
 *                    it is still the gradient with respect to the zero initial state.
 * Gradients of rows past the end of every sequence are not written (there are none: cu_seqlens
 * covers all rows). No gradient buffer may overlap an input or another gradient
 * (KDA_ERROR_INVALID_VALUE). Head dims K in {32, 64, 128}, V in {32, 64, 128, 256}, both
 * dtypes; others give KDA_ERROR_NOT_SUPPORTED. Every gradient is the same bit for bit on every
 * run (no atomics; sums in a fixed order).
 *
 * Workspace (256-byte aligned): the chunks are taken in segments, processed from the last
 * backwards; each segment holds, per (chunk, head), an fp32 record, the chunk-start state, the
 * chunk-end state gradient and scratch (about 500 KB per 64 tokens and head at K = V = 128).
 * With more than one segment, a forward pass over the records first keeps the state at every
 * segment boundary (H * K * V fp32 each), and each segment's record and states are formed again
 * on the way back: the workspace stays near one segment's size for any T, at the cost of that
 * second pass. kda_chunk_bwd takes the longest segments that workspace_bytes holds (one segment,
 * no second pass, when it holds every chunk) and returns KDA_ERROR_WORKSPACE_TOO_SMALL when not
 * even one chunk per segment fits. The gradients do not depend on the segment length.
 *   kda_chunk_bwd_workspace_size    : the default, segments of about 4 GiB, no input options
 *   kda_chunk_bwd_workspace_size_ex : for kda_chunk_bwd_ex with these options, segments of
 *                                     segment_tokens tokens (rounded up to 64; 0: one segment
 *                                     over every chunk; < 0: the default segments)
 * Both return 0 for shapes (or option bits) the backward does not support.
 */
size_t kda_chunk_bwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                    int32_t dk, int32_t dv, kda_dtype dtype);
size_t kda_chunk_bwd_workspace_size_ex(int32_t num_seqs, int64_t total_tokens,
                                       int32_t num_heads, int32_t dk, int32_t dv,
                                       kda_dtype dtype, uint32_t options, int64_t segment_tokens);
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* init_state, const int32_t* cu_seqlens,
                         int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                         int32_t dv, kda_dtype dtype, const void* d_o,
                         const float* d_final_state, float* grad_q, float* grad_k, float* grad_v,
                         float* grad_log_alpha, float* grad_beta, float* grad_init_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_bwd for kda_chunk_fwd_ex with input options (KDA_OPT_*; options = 0 is
 * kda_chunk_bwd): the gradients are those of the raw inputs, through the options' prologue
 * (unit-norm q and k, log alpha = log sigmoid(z), one gate per head, beta = sigmoid(x)). With
 * KDA_OPT_SCALAR_GATE, log_alpha and grad_log_alpha are [rows][H] and need only their element
 * alignment. The workspace (kda_chunk_bwd_workspace_size_ex with the same options) also holds
 * the processed q, k, log alpha and beta in fp32 for every token (and, with the scalar gate,
 * the per-channel gradient of log alpha): about 12 K + 4 bytes per token and head more.
 */
kda_status kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                            const void* beta, const float* init_state, const int32_t* cu_seqlens,
                            int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                            int32_t dk, int32_t dv, kda_dtype dtype, uint32_t options,
                            const void* d_o, const float* d_final_state, float* grad_q,
                            float* grad_k, float* grad_v, float* grad_log_alpha,
                            float* grad_beta, float* grad_init_state, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Checkpoints for training: the forward keeps the state at the start of every E-th chunk
 * (E = kda_chunk_fwd_ckpt_interval, its segment length: 2048 / H chunks of 64 tokens, at
 * most the chunk count), and the backward starts its segments from those states instead of
 * forming them with a pass of its own ("A Technical Breakdown", section 4: the state passed
 * from chunk to chunk is all that links the chunks).
 * Chunks are numbered in token order over the packed sequences (sequence n's chunks follow
 * sequence n - 1's; a sequence's last chunk may be partial). Slot j of checkpoints
 * ([slots][H][K][V] fp32, slots = kda_chunk_fwd_ckpt_bytes / (4 H K V)) holds, for every
 * head, the state of the sequence that chunk (j + 1) E belongs to, just before that chunk,
 * when that chunk is not the sequence's first; other slots are not written (the backward
 * starts such a sequence from its initial state).
 * kda_chunk_fwd_ckpt is kda_chunk_fwd_ex with this output (same results bit for bit; the
 * chunk table is in token order whatever H); it supports the shapes of the training backward
 * on the chunk path: K in {32, 64, 128}, V in {32, 64, 128, 256}, bf16 inputs, or fp32 inputs at
 * K <= 64
 * (KDA_ERROR_NOT_SUPPORTED otherwise). checkpoints may be NULL when there are no slots, must
 * be 16-byte aligned and must not overlap another buffer of the call.
 * kda_chunk_bwd_ckpt is kda_chunk_bwd_ex starting from the checkpoints of a
 * kda_chunk_fwd_ckpt call on the same inputs and options; its segments are multiples of E
 * chunks (the longest that workspace_bytes holds; KDA_ERROR_WORKSPACE_TOO_SMALL when not even E
 * chunks fit), and no boundary pass runs. The gradients then carry the forward's rounding of
 * the states at the segment boundaries (the bf16 forward's states are within its 2e-2
 * tolerance; the backward's own boundary pass keeps fp32 records); with one segment the result
 * equals kda_chunk_bwd_ex's. checkpoints may be NULL only when there are no slots.
 */
int64_t kda_chunk_fwd_ckpt_interval(int32_t num_seqs, int64_t total_tokens, int32_t num_heads);
size_t kda_chunk_fwd_ckpt_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                int32_t dk, int32_t dv);
kda_status kda_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, const float* init_state,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                              uint32_t options, void* o, float* final_state, float* checkpoints,
                              void* workspace, size_t workspace_bytes, void* stream);
kda_status kda_chunk_bwd_ckpt(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, const float* init_state,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                              uint32_t options, const void* d_o, const float* d_final_state,
                              const float* checkpoints, float* grad_q, float* grad_k,
                              float* grad_v, float* grad_log_alpha, float* grad_beta,
                              float* grad_init_state, void* workspace, size_t workspace_bytes,
                              void* stream);

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
