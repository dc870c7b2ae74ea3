/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA gated delta-rule core.
 *
 * The core is the per-head gated delta-rule recurrence over an FP32
 * [heads, 128, 128] key-major state (config page, config.rs:
 * Glm5NextKdaConfig::recurrent_state_elems; head_dim is fixed at 128 by
 * Glm5NextKdaConfig::validate).  For every token t of a sequence and every
 * head, with gate the per-channel log-decay (workspace page, field "gate")
 * and beta already passed through a sigmoid (workspace page, field "beta"):
 *
 *     S <- diag(exp(gate_t)) S                 decay, one factor per key row
 *     delta = beta_t (v_t - S^T k_t)
 *     S <- S + k_t delta^T
 *     out_t = S^T q_t                          post-update state, no scale
 *
 * The decay comes before the delta correction: the recurrent kernels of the
 * kernel-table page (Glm5NextKdaKernels, fields recurrent / recurrent_smem)
 * share the *decayed* state column between their two passes.  q and k are
 * expected L2-normalised and v raw (module page, pipeline line); the core
 * itself normalises nothing.  A caller that wants a 1/sqrt(d) attention scale
 * pre-scales q.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * All tensor pointers are DEVICE pointers to contiguous memory owned by
 *    the caller, FP32 unless a declaration says BF16, and 16-byte aligned
 *    (beta: 4-byte aligned); a misaligned pointer is refused.  The library allocates nothing and keeps no state between
 *    calls (module page: the forward calls allocate nothing and write only
 *    into the caller's workspace and sequence state).
 *  * Layouts (token-major, heads inside, D = 128):
 *        q, k, v, gate, out : [batch][rows][heads][D]
 *        beta               : [batch][rows][heads]
 *        state              : [batch][heads][D key][D value]  (value index contiguous)
 *        snapshots          : [n_snapshots][batch][heads][D][D]
 *    rows = T_pad = ceil(T / chunk) * chunk for kda_chunk_prefill (the
 *    workspace page pads prefill buffers to whole chunks), rows = T for
 *    kda_recurrent_k and rows = 1 for kda_recurrent_step.  The packed
 *    (varlen) prefill, the decode and prefill front ends, the BF16 decode
 *    forms and the gated RMSNorm state their own layouts at their
 *    declarations.
 *  * Inputs are read-only.  state is read and updated in place (layer page:
 *    decode updates the state in place).  out rows >= T are never written.
 *  * out, state, snapshots and workspace must not overlap each other or any
 *    input; an overlap of the ranges implied by the sizes is refused.
 *  * stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    are asynchronous on that stream: a return of KDA_OK means the work was
 *    validated and enqueued.  Faults during execution surface at the caller's
 *    next synchronisation, as for any HIP launch.
 *  * Every argument check runs on the host before anything is enqueued; on any
 *    error nothing is launched and no buffer is touched (config page:
 *    validate refuses a bad geometry instead of running it).
 *  * Calls are reentrant; concurrent calls on different streams are safe as
 *    long as their buffers do not overlap.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
/* Largest head count kda_chunk_prefill accepts (byte offsets inside one chunk
 * of a sequence stay below 2^31). */
#define KDA_PREFILL_MAX_HEADS 16384
/* Most sequences one kda_chunk_prefill_varlen call takes. */
#define KDA_VARLEN_MAX_SEQS (1 << 20)
/* Smallest eps kda_gated_rmsnorm and the front ends accept. */
#define KDA_GATED_RMSNORM_MIN_EPS 1e-30f
/* Largest conv_kernel the front ends accept: the config page's validation
 * caps the window at four taps, and the kernels here hold the window of
 * every channel in four registers. */
#define KDA_FRONT_END_MAX_CONV_KERNEL 4

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, size < 1, bad n_snapshots / eps, overlap, overflow */
    KDA_ERR_UNSUPPORTED = -2, /* chunk not in {16, 32, 64}; conv_kernel above 4                          */
    KDA_ERR_WORKSPACE = -3,   /* workspace smaller than the matching *_workspace_bytes() query        */
    KDA_ERR_HIP = -4          /* the HIP runtime refused a launch                                     */
} kda_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* kda_status_string(int status);

/*
 * Workspace bytes kda_chunk_prefill needs for (batch, heads, T, chunk), or 0
 * when the arguments are invalid (batch/heads/T < 1, unsupported chunk, size
 * overflow).  The workspace holds, per (sequence, head, chunk), the chunk's
 * WY/UT intermediates written by the prepare kernel and read by the scan
 * kernel (kernel-table page, fields chunk_prepare / chunk_scan).  Contents
 * on entry are ignored.  On exit it holds the call's chunk records, from
 * which kda_chunk_scan can run the scan again.
 */
size_t kda_chunk_prefill_workspace_bytes(int batch, int heads, int T, int chunk);

/*
 * The chunked prefill: T tokens of each sequence continue its recurrent
 * state from wherever the previous call left it (layer page,
 * Glm5NextKdaLayer::prefill; kernel-table page, chunk_prepare + chunk_scan).
 *
 *   q, k, v, gate : [batch][T_pad][heads][128], T_pad = ceil(T/chunk)*chunk
 *   beta          : [batch][T_pad][heads]
 *   state         : [batch][heads][128][128], in: carried state, out: state after token T-1
 *   out           : [batch][T_pad][heads][128]; rows t < T receive the core output
 *   chunk         : 16, 32 or 64 (changes rounding only, never the result beyond it)
 *   workspace     : device scratch of at least kda_chunk_prefill_workspace_bytes() bytes
 *   heads         : at most KDA_PREFILL_MAX_HEADS (else KDA_ERR_INVALID_ARG)
 *   batch * heads * T_pad / chunk (the number of chunk records) at most 2^30
 *                   (else KDA_ERR_INVALID_ARG)
 *
 * Rows t >= T of every input may hold anything, NaN and inf included: the
 * kernels select them away before any arithmetic (the layer page's
 * prefill_with_pad_fill fills the padded tails with a test value for exactly
 * this property).
 * Gate domain: any gate <= 0, -inf included (config page, gate_lower_bound
 * bounds it from below without printing the value).  Chunks whose gates are
 * all >= about -8.3 (-12 in log2 units) factor each pairwise decay
 * exp(G_r - G_s) inside a 16-token block into two FP32 factors about the
 * block's eighth row; a chunk with a steeper gate takes a second path whose
 * factors are explicit exponentials of exponent sums <= 0, with two products
 * on the diagonal blocks, so no factor leaves the FP32 range.  On that path
 * a gate below about -19.4 (-28 in log2 units) counts as that value: its
 * decay factor is 2^-28 instead of a smaller one, which moves the state by
 * less than 2^-28 of its decayed part.  Results agree with the decode entry
 * points within the stated tolerance for every gate (tested down to -60 and
 * -inf).  Gates > 0 (growth) are computed as given but are outside this
 * statement.
 */
int kda_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                      float* state, float* out, int batch, int heads, int T, int chunk, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The chunk records live in a static device array the library
 * owns, KDA_STATIC_WORKSPACE_BYTES per GPU (held from the first call on that
 * GPU until the process ends), instead of a caller workspace.  Nothing is
 * allocated: the first call on a device looks the array's address up once
 * (hipGetSymbolAddress) and keeps it; later calls reuse it.
 *
 *   q, k, v, gate, beta, state, out, batch, heads, T, chunk : as kda_chunk_prefill
 *
 * The result equals kda_chunk_prefill's bit for bit (same kernels).  Calls
 * whose records would exceed the array, i.e. kda_chunk_prefill_workspace_bytes
 * (batch, heads, T, chunk) > KDA_STATIC_WORKSPACE_BYTES, are refused with
 * KDA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's array, and the array keeps the last call's records (nothing in
 * it needs to start at zero): two calls that can run at the same time on one
 * GPU (different streams, no ordering between them) race on it and give
 * undefined results; calls ordered on one stream are safe.  Other refusals as
 * kda_chunk_prefill; KDA_ERR_HIP if the array's address cannot be looked up.
 */
#define KDA_STATIC_WORKSPACE_BYTES (256u << 20)
int kda_chunk_prefill_noalloc(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                              float* state, float* out, int batch, int heads, int T, int chunk, void* stream);

/*
 * kda_chunk_prefill with the block's gate and beta steps inside the prefill's
 * prepare kernel: the gate comes from kda_gate of its projection g_raw and
 * beta from the sigmoid of its logit, both computed while a chunk is staged,
 * so neither the FP32 gate nor beta travels through HBM (workspace page,
 * field gate: the bounded log-decay kda_gate makes from g_raw; field beta:
 * already passed through a sigmoid; module page, pipeline line: beta =
 * sigmoid(b_proj(h)); config page, Glm5NextKdaWeights::dt_bias, a_log and
 * Glm5NextKdaConfig::gate_lower_bound).  The pages name kda_gate's inputs but
 * print no formula; the reading implemented is
 *
 *     gate[b][t][h][i] = gate_lower_bound * sigmoid(exp(a_log[h]) * (g_raw[b][t][h][i] + dt_bias[h][i]))
 *     beta[b][t][h]    = sigmoid(beta_logit[b][t][h])
 *
 * in FP32 (hardware exp2 and reciprocal, each within about one unit in the
 * last place), a log-decay in [gate_lower_bound, 0].
 *
 *   q, k, v, state, out, workspace : as kda_chunk_prefill
 *   g_raw            : [batch][T_pad][heads][128] BF16 (raw 16-bit patterns), 8-byte aligned
 *   beta_logit       : [batch][T_pad][heads] FP32
 *   dt_bias          : [heads][128] FP32 (the config page's [heads * head_dim]), 16-byte aligned
 *   a_log            : [heads] FP32
 *   gate_lower_bound : finite and <= 0 (else KDA_ERR_INVALID_ARG)
 *
 * Rows t >= T of every input are ignored, as for kda_chunk_prefill.  The
 * result equals kda_chunk_prefill fed with the gate and beta above within
 * the stated tolerance (the same kernels after the staging).  Refusals as
 * kda_chunk_prefill, plus a null, misaligned or overlapping gate input.
 */
int kda_chunk_prefill_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                            const float* beta_logit, const float* dt_bias, const float* a_log, float gate_lower_bound,
                            float* state, float* out, int batch, int heads, int T, int chunk, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill on BF16 q, k and v packed per token, the row layout of the
 * decode path's BF16 forms with the prefill's padding.  The pages keep the
 * prefill's q, k, v in FP32 (workspace page, fields q_f32 / k_f32 / v_f32);
 * this form is for callers that hold them in BF16 (module page: the block's
 * projections run in BF16), and it halves what the prefill reads for them.
 *
 *   qkv                            : [batch][T_pad][3][heads][128] BF16 (raw 16-bit patterns): q, then k,
 *                                    then v of every head for each token, 16-byte aligned
 *   gate, beta, state, out, workspace : as kda_chunk_prefill
 *
 * BF16 widens to FP32 exactly where a chunk is staged and the arithmetic is
 * that of kda_chunk_prefill, so the results equal kda_chunk_prefill on the
 * widened q, k, v bit for bit (rows t >= T ignored alike, the same gate
 * domain).  Refusals are those of kda_chunk_prefill, with qkv in place of q,
 * k and v.
 */
int kda_chunk_prefill_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                           int batch, int heads, int T, int chunk, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Chunked prefill of a packed batch of sequences of their own lengths
 * (varlen).  Same computation as kda_chunk_prefill for every sequence, with
 * the sequences stored back to back instead of padded to a common length (the
 * workspace page sizes its prefill buffers in whole chunks; here each
 * sequence's last chunk is cut at its end instead).
 *
 *   q, k, v, gate, out : [total_tokens][heads][128];  beta : [total_tokens][heads]
 *   state              : [n_seqs][heads][128][128], read and updated in place
 *   cu_seqlens         : DEVICE int32 [n_seqs + 1]; sequence s holds tokens
 *                        cu_seqlens[s] .. cu_seqlens[s + 1] - 1.  Expected
 *                        0 = cu_seqlens[0] <= ... <= cu_seqlens[n_seqs] <=
 *                        total_tokens.  The values are read on the device only:
 *                        each is clamped to [0, total_tokens] and raised to the
 *                        largest before it, so any content stays inside the
 *                        buffers (an empty sequence leaves its state as is).
 *   workspace          : >= kda_chunk_prefill_varlen_workspace_bytes(n_seqs,
 *                        heads, total_tokens, chunk) bytes (records for up to
 *                        heads * (total_tokens / chunk + n_seqs) chunks, then
 *                        the clamped offsets)
 *
 * out rows outside every sequence are not written.  Each sequence's result
 * equals the bits of kda_chunk_prefill on that sequence alone.  Refusals as
 * kda_chunk_prefill, plus n_seqs outside [1, KDA_VARLEN_MAX_SEQS] or
 * total_tokens < 1 (KDA_ERR_INVALID_ARG).
 */
size_t kda_chunk_prefill_varlen_workspace_bytes(int n_seqs, int heads, int total_tokens, int chunk);
int kda_chunk_prefill_varlen(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                             float* state, float* out, const int* cu_seqlens, int n_seqs, int heads, int total_tokens,
                             int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_varlen on BF16 q, k and v packed per token, as
 * kda_chunk_prefill_bf16 is to kda_chunk_prefill.
 *
 *   qkv : [total_tokens][3][heads][128] BF16 (raw 16-bit patterns), 16-byte aligned
 *   gate, beta, state, out, cu_seqlens, workspace : as kda_chunk_prefill_varlen
 *
 * The results equal kda_chunk_prefill_varlen on the widened q, k, v bit for
 * bit.  Refusals are those of kda_chunk_prefill_varlen, with qkv in place of
 * q, k and v.
 */
int kda_chunk_prefill_varlen_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                                  const int* cu_seqlens, int n_seqs, int heads, int total_tokens, int chunk,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_prefill_front_end followed by kda_chunk_prefill, fused: the front end
 * (causal conv1d + SiLU, L2 on q and k; module page, pipeline line) runs
 * inside the prefill's prepare kernel, which reads the BF16 projections
 * instead of FP32 q, k, v rows, so those rows never travel through HBM
 * (workspace page, fields q_f32 / k_f32 / v_f32: unused on this path).
 *
 *   qkv        : [batch][T][3 * heads * 128] BF16; each token's row holds its q, then k, then v channels (no padding)
 *   conv_w     : [3 * heads * 128][conv_kernel] BF16
 *   conv_state : [batch][3 * heads * 128][conv_kernel], read, then advanced by the T inputs
 *   gate, beta, state, out, workspace : as kda_chunk_prefill
 *   conv_kernel: 4 (others KDA_ERR_UNSUPPORTED; kda_prefill_front_end takes 1..4)
 *   l2_eps     : as kda_prefill_front_end
 *
 * The result agrees with kda_prefill_front_end + kda_chunk_prefill within
 * the stated tolerance, not bit for bit: the sum of squares of each q and k
 * row is taken in another order.  The conv state ends as kda_prefill_front_end
 * leaves it (bit for bit).  Refusals as the two calls, plus T * 3 * heads *
 * 256 above 2^31 - 1 (KDA_ERR_INVALID_ARG).
 */
int kda_chunk_prefill_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                            const float* beta, float* state, float* out, int batch, int heads, int T, int chunk,
                            int conv_kernel, float l2_eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_fused with the gate and beta steps inside the prepare as
 * well (as kda_chunk_prefill_gated forms them): the prefill of the block from
 * its raw projections, q | k | v, the gate's projection and beta's logits.
 *
 *   g_raw, beta_logit, dt_bias, a_log, gate_lower_bound : as
 *            kda_chunk_prefill_gated (rows [batch][T_pad])
 *   everything else : as kda_chunk_prefill_fused
 *
 * The result agrees with kda_prefill_front_end + kda_chunk_prefill_gated
 * within the stated tolerance (the q and k sums of squares in another order);
 * the conv state ends bit for bit as there.  Refusals: those of
 * kda_chunk_prefill_fused and kda_chunk_prefill_gated.
 */
int kda_chunk_prefill_fused_gated(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                  const uint16_t* g_raw, const float* beta_logit, const float* dt_bias,
                                  const float* a_log, float gate_lower_bound, float* state, float* out, int batch,
                                  int heads, int T, int chunk, int conv_kernel, float l2_eps, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * The varlen form of kda_chunk_prefill_fused: kda_prefill_front_end_varlen
 * followed by kda_chunk_prefill_varlen, with the front end inside the
 * prefill's prepare kernel.
 *
 *   qkv        : [total_tokens][3 * heads * 128] BF16, the sequences back to back
 *   conv_state : [n_seqs][3 * heads * 128][conv_kernel], one per sequence, advanced by its inputs
 *   conv_w, conv_kernel (4), l2_eps : as kda_chunk_prefill_fused
 *   gate, beta, state, out, cu_seqlens, workspace : as kda_chunk_prefill_varlen
 *
 * Each sequence's conv window starts from its own conv state.  Agreement with
 * the separate calls, and refusals, as kda_chunk_prefill_fused and
 * kda_chunk_prefill_varlen, plus total_tokens * 3 * heads * 256 above
 * 2^31 - 1 (KDA_ERR_INVALID_ARG).
 */
int kda_chunk_prefill_varlen_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                                   const float* beta, float* state, float* out, const int* cu_seqlens, int n_seqs,
                                   int heads, int total_tokens, int chunk, int conv_kernel, float l2_eps,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Segment transition of a prefill: the final state of kda_chunk_prefill over
 * these T tokens as an affine function of its initial state (layer page,
 * Glm5NextKdaLayer::prefill; kernel-table page, chunk_scan, whose per-chunk
 * update is linear in the incoming state plus a term from the chunk's
 * values).  Not an operation of the pages: it is the per-device piece of
 * splitting one long sequence across devices by token segments.  Each device
 * computes its segment's (P, Q); the pairs are folded in segment order with
 * kda_state_transition_apply to give every segment its true initial state;
 * then each device runs kda_chunk_scan on the records this call left in the
 * workspace (or kda_chunk_prefill) from that state.
 *
 *   q, k, v, gate, beta : as kda_chunk_prefill (rows t >= T ignored)
 *   trans_p             : [batch][heads][128][128] out, P[i][j] over key indices
 *   trans_q             : [batch][heads][128 key][128 value] out
 *   workspace           : >= kda_chunk_prefill_workspace_bytes(batch, heads, T, chunk)
 *
 * For every initial state S [128 key][128 value] the prefill's final state is
 * P S + Q, up to FP32 rounding.  Q is the final state from S = 0; P is the
 * product over the tokens, later ones on the left, of
 * (I - beta k k^T) diag(exp(gate)), computed chunk by chunk from the identity.
 * Both are written whole.  No output rows are produced.  The workspace is left
 * holding the chunk records, as after kda_chunk_prefill.  Refusals and accuracy
 * as kda_chunk_prefill, with trans_p and trans_q taking the place of state and
 * out in the overlap checks.
 */
int kda_chunk_prefill_transition(const float* q, const float* k, const float* v, const float* gate,
                                 const float* beta, float* trans_p, float* trans_q, int batch, int heads, int T,
                                 int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The scan half of kda_chunk_prefill alone (kernel-table page, chunk_scan),
 * from the chunk records a preceding kda_chunk_prefill or
 * kda_chunk_prefill_transition with the same batch, heads, T and chunk left
 * in the workspace.  It runs the prefill again from another initial state
 * without recomputing the records.  After a segment's transition and the fold
 * of the segments before it, this gives the segment's outputs from its true
 * initial state.
 *
 *   state     : [batch][heads][128][128], in: initial state, out: state after token T-1
 *   out       : [batch][T_pad][heads][128]; rows t < T written, as kda_chunk_prefill
 *   workspace : the records, at least kda_chunk_prefill_workspace_bytes(batch,
 *               heads, T, chunk) bytes; read only
 *
 * The result equals the bits of kda_chunk_prefill on the inputs the records
 * were made from, started from `state`.  Records made with other sizes, or
 * never made, give unspecified values; every access stays inside the
 * workspace size checked here.  Refusals as kda_chunk_prefill (a null or
 * short workspace is KDA_ERR_WORKSPACE; out, state and workspace must not
 * overlap).
 */
int kda_chunk_scan(float* state, float* out, int batch, int heads, int T, int chunk, const void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * state <- trans_p state + trans_q for batch * heads states of 128 x 128 FP32,
 * in place (trans_q NULL: state <- trans_p state).  The fold step of the
 * segment transitions above: applied to a state it gives the state after the
 * segment; applied to another segment's Q it composes two segments (P2 Q1 +
 * Q2), and with trans_q NULL to its P it gives P2 P1.
 *
 *   trans_p, trans_q, state : [batch][heads][128][128], 16-byte aligned
 *
 * state must not overlap trans_p or trans_q (KDA_ERR_INVALID_ARG); batch *
 * heads above 2^22 - 8 (the launch's grid limit) is refused the same way.
 * The products accumulate in FP32 over the 128 key indices.
 */
int kda_state_transition_apply(const float* trans_p, const float* trans_q, float* state, int batch, int heads,
                               void* stream);

/*
 * One recurrent decode step: one token per sequence (layer page,
 * Glm5NextKdaLayer::decode; kernel-table page, recurrent_smem).  Each head
 * state is read from HBM once and written once; the decayed state stays in
 * registers between the read-out and the update.
 *
 *   q, k, v, gate, out : [batch][1][heads][128];  beta : [batch][1][heads]
 *   state              : [batch][heads][128][128], updated in place
 *
 * Bit-for-bit equal to kda_recurrent_k with T = 1.
 */
int kda_recurrent_step(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                       float* state, float* out, int batch, int heads, void* stream);

/*
 * T rows of each sequence walked one at a time with the state held on chip
 * (layer page, Glm5NextKdaLayer::decode_k: speculative verify and prefill
 * sub-chunks; the row-serial walker stateful_row).
 *
 *   q, k, v, gate, out : [batch][T][heads][128];  beta : [batch][T][heads]
 *   state              : [batch][heads][128][128]; out: state after row T-1
 *   snapshots          : [n_snapshots][batch][heads][128][128]; slot t holds
 *                        the state as row t left it, for t < n_snapshots
 *                        (rows past n_snapshots take none); may be NULL when
 *                        n_snapshots == 0
 *   n_snapshots        : 0 <= n_snapshots <= T
 *
 * T == 0 is refused (the layer page refuses k == 0).  out, the final state
 * and every snapshot are bitwise the results of T successive
 * kda_recurrent_step calls.
 */
int kda_recurrent_k(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                    float* state, float* out, float* snapshots, int n_snapshots, int batch, int heads, int T,
                    void* stream);

/*
 * The two decode entry points above with the gate and beta steps inside the
 * decode kernel's row loads: gate = kda_gate(g_raw) and beta =
 * sigmoid(beta_logit), the reading and arguments of kda_chunk_prefill_gated
 * (g_raw [batch][T][heads][128] BF16, beta_logit [batch][T][heads] FP32,
 * dt_bias [heads][128], a_log [heads], gate_lower_bound finite and <= 0).
 * Everything else as kda_recurrent_k / kda_recurrent_step; T rows of
 * kda_recurrent_k_gated equal T successive kda_recurrent_step_gated calls
 * bit for bit (the same kernel).
 */
int kda_recurrent_k_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                          const float* beta_logit, const float* dt_bias, const float* a_log, float gate_lower_bound,
                          float* state, float* out, float* snapshots, int n_snapshots, int batch, int heads, int T,
                          void* stream);
int kda_recurrent_step_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                             const float* beta_logit, const float* dt_bias, const float* a_log,
                             float gate_lower_bound, float* state, float* out, int batch, int heads, void* stream);

/*
 * The two decode entry points above with BF16 q, k, v packed per token, as
 * the decode front end leaves them (workspace page, conv_out: [T, conv_dim]
 * BF16 after conv and SiLU, with L2 already applied on the decode path;
 * module page: every projection of the block runs in BF16).  gate, beta,
 * state, out and snapshots are as above (FP32).
 *
 *   qkv : [batch][T][3][heads][128] BF16 (raw 16-bit patterns): q, then k,
 *         then v of every head for each token, i.e. the [batch][T][conv_dim]
 *         conv_out of kda_decode_front_end_bf16
 *
 * BF16 widens to FP32 exactly and the arithmetic is that of the FP32 entry
 * points, so the results equal kda_recurrent_k / kda_recurrent_step on the
 * widened q, k, v bit for bit; kda_recurrent_step_bf16 equals
 * kda_recurrent_k_bf16 with T = 1, and T rows of kda_recurrent_k_bf16 equal T
 * successive kda_recurrent_step_bf16 calls bit for bit.  Refusals are those of
 * kda_recurrent_k, with qkv in place of q, k and v.
 */
int kda_recurrent_k_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                         float* snapshots, int n_snapshots, int batch, int heads, int T, void* stream);
int kda_recurrent_step_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                            int batch, int heads, void* stream);

/*
 * The BF16 decode forms above with the block's next step fused in: the
 * sigmoid-gated RMSNorm of every output row (see kda_gated_rmsnorm) is done
 * by the decode kernel itself, so the core's FP32 rows need not travel
 * through HBM to a second kernel (module page, pipeline line; workspace page,
 * fields core, out_gate and o_norm_out).  One workgroup holds a whole head
 * here, so the 128 channels of a row meet in one wave.
 *
 *   qkv, gate, beta, state, snapshots, n_snapshots : as kda_recurrent_k_bf16
 *   out      : [batch][T][heads][128] FP32 core rows, or NULL (then not stored)
 *   out_gate : [batch][T][heads][128] BF16, the output gate
 *   o_norm   : [128] BF16;  eps: as kda_gated_rmsnorm
 *   y        : [batch][T][heads][128] BF16, the normalised rows (o_norm_out)
 *
 * y is within one BF16 unit in the last place of the exact norm of the core
 * rows the call computes (the scale is formed in FP64 over the 128 squares
 * in another order than kda_gated_rmsnorm's, so the two agree bit for bit
 * except where that order moves the scale by its last bit).  The core rows,
 * state and snapshots are within the stated tolerance of kda_recurrent_k_bf16
 * (another reduction tree: a whole-head workgroup); T rows of
 * kda_recurrent_k_bf16_norm equal T successive kda_recurrent_step_bf16_norm
 * calls bit for bit.  Refusals as kda_recurrent_k_bf16 and kda_gated_rmsnorm.
 */
int kda_recurrent_k_bf16_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                              const uint16_t* out_gate, const uint16_t* o_norm, float eps, uint16_t* y,
                              float* snapshots, int n_snapshots, int batch, int heads, int T, void* stream);
int kda_recurrent_step_bf16_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                                 const uint16_t* out_gate, const uint16_t* o_norm, float eps, uint16_t* y, int batch,
                                 int heads, void* stream);

/*
 * The step after the core: sigmoid-gated RMSNorm of the core's output (module
 * page, pipeline line: the core output goes through a sigmoid-gated RMSNorm
 * with weight o_norm and gate g_b(g_a(h)) before o_proj; the gate goes
 * through the logistic sigmoid there, unlike the SiLU-gated norm the page
 * also names).  Independently for every row r and
 * head h, over the 128 value channels j of x = core[r][h]:
 *
 *     out[r][h][j] = x_j / sqrt(mean_i x_i^2 + eps) * o_norm[j] * sigmoid(out_gate[r][h][j])
 *
 *   core     : [rows][heads][128] FP32, e.g. the out of the entry points
 *              above with rows = batch * their row count
 *   out_gate : [rows][heads][128] BF16 (raw 16-bit patterns), the output gate
 *              (workspace page, field out_gate: [T, qkv] BF16)
 *   o_norm   : [128] BF16, one weight per channel shared by every head (config
 *              page, Glm5NextKdaWeights::o_norm: [head_dim] BF16)
 *   out      : [rows][heads][128] BF16 (workspace page, field o_norm_out)
 *   eps      : rms_norm_eps (config page), finite and
 *              >= KDA_GATED_RMSNORM_MIN_EPS
 *
 * Rows are independent; padded prefill rows (t >= T) are processed like any
 * other and give whatever their core holds.  The scale is formed in FP64, so
 * any finite core is handled without overflow; the products are FP32 and the
 * result is rounded to nearest even, within one BF16 unit in the last place
 * of the exact value.  out must not overlap an input.  Refusals
 * (KDA_ERR_INVALID_ARG): a null pointer, rows or heads < 1, eps out of range,
 * rows * heads above 2^34 - 8, overlap.
 */
int kda_gated_rmsnorm(const float* core, const uint16_t* out_gate, const uint16_t* o_norm, uint16_t* out,
                      int rows, int heads, float eps, void* stream);

/*
 * The step before the core on the decode path: the depthwise causal conv1d
 * update, SiLU and L2 on q and k in one call (module page, pipeline line:
 * conv1d and SiLU on q, k, v, then L2 on q and k alone, so v is never
 * normalised; the decode form there is a single kernel too; the conv state
 * holds conv_kernel slots that move one place toward the oldest before each
 * convolution).  T rows of each sequence are walked in
 * order (T = 1 for a decode step, T = k for decode_k).  For every row and
 * every channel c of conv_dim = 3 * heads * 128 (q | k | v, in that order):
 *
 *     slots <- (slots[1], ..., slots[K-1], qkv[c])      K = conv_kernel
 *     y      = sum_k conv_w[c][k] * slots[k]            slot K-1 holds the newest input
 *     y      = y * sigmoid(y)
 *     q, k  : each head's 128 values scaled by 1 / sqrt(sum y^2 + l2_eps); v as is
 *
 *   qkv            : [batch][T][conv_dim] BF16 (workspace page, qkv_proj:
 *                    [T, conv_dim] BF16, one row of q, k and v channels a token)
 *   conv_w         : [conv_dim][conv_kernel] BF16, no bias (config page,
 *                    Glm5NextKdaWeights::conv)
 *   conv_state     : [batch][conv_dim][conv_kernel] FP32, read and updated in
 *                    place (config page, conv_state_elems)
 *   q, k, v        : [batch][T][heads][128] FP32, the inputs of
 *                    kda_recurrent_step / kda_recurrent_k
 *   conv_snapshots : [n_snapshots][batch][conv_dim][conv_kernel] FP32, the
 *                    conv state after row t for t < n_snapshots (the conv half
 *                    of decode_k's snapshots, layer page); NULL when
 *                    n_snapshots == 0
 *   conv_kernel    : 1..4 (KDA_ERR_UNSUPPORTED above 4)
 *   l2_eps         : finite, >= KDA_GATED_RMSNORM_MIN_EPS, added inside the
 *                    square root (config page, l2_eps)
 *
 * The conv state only ever holds inputs, so it is exact; q, k, v carry the
 * FP32 rounding of the conv sum and a few units of 2^-24 from the SiLU (the
 * hardware exp2 and reciprocal); the L2 sum of squares and scale are formed
 * in FP64, so no finite input overflows or flushes them.
 * Outputs, conv_state and conv_snapshots must not overlap each other or an
 * input.  Refusals (KDA_ERR_INVALID_ARG): a null pointer, batch, heads or T
 * < 1, heads > KDA_PREFILL_MAX_HEADS, n_snapshots outside [0, T], conv_kernel
 * < 1, l2_eps out of range, overlap.
 */
int kda_decode_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                         float* v, float* conv_snapshots, int n_snapshots, int batch, int heads, int T,
                         int conv_kernel, float l2_eps, void* stream);

/*
 * kda_decode_front_end with its output in BF16, in the input's own layout
 * (workspace page, conv_out: [T, conv_dim] BF16 after conv + SiLU, L2 fused
 * in on the decode path), ready for kda_recurrent_step_bf16 /
 * kda_recurrent_k_bf16:
 *
 *   conv_out : [batch][T][conv_dim] BF16 = [batch][T][3][heads][128]
 *
 * Every value is the FP32 result kda_decode_front_end writes, rounded to the
 * nearest BF16 (ties to even); conv_state and conv_snapshots are updated
 * exactly as there.  All other arguments, conventions and refusals are those
 * of kda_decode_front_end; conv_out must not overlap any other buffer.
 */
int kda_decode_front_end_bf16(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, uint16_t* conv_out,
                              float* conv_snapshots, int n_snapshots, int batch, int heads, int T, int conv_kernel,
                              float l2_eps, void* stream);

/*
 * The whole decode step of the block between its projections, in one kernel:
 * the decode front end (conv1d update, SiLU, L2 on q and k), the recurrence,
 * and the sigmoid-gated RMSNorm of every output row (module page, pipeline
 * line, from the conv to the norm; workspace page, fields qkv_proj, conv_out,
 * core and o_norm_out).  One workgroup holds a whole head: three of its waves
 * run the front end of the head's q, k and v vectors with the code of
 * kda_decode_front_end, so the FP32 q, k, v never leave the chip, and the
 * core's rows go through the norm where the workgroup has them.
 *
 *   qkv_proj, conv_w, conv_state, conv_snapshots, conv_kernel, l2_eps :
 *            as kda_decode_front_end (qkv_proj its qkv)
 *   gate, beta, state, snapshots, n_snapshots : as kda_recurrent_k; one
 *            n_snapshots counts both kinds of snapshot (both pointers
 *            non-NULL when it is > 0)
 *   out_gate, o_norm, norm_eps, y : as kda_recurrent_k_bf16_norm (its eps)
 *   out    : [batch][T][heads][128] FP32 core rows, or NULL (then not stored)
 *
 * conv_state and conv_snapshots equal kda_decode_front_end's bit for bit, and
 * so do the q, k, v the recurrence consumes; the core rows, state and
 * snapshots are within the stated tolerance of kda_decode_front_end followed
 * by kda_recurrent_k (a whole-head reduction tree here, unrounded q, k, v
 * rather than kda_decode_front_end_bf16's BF16 ones); y is within one BF16
 * unit in the last place of the norm of the call's own core rows.  T rows of
 * kda_decode_fused_k equal T successive kda_decode_fused_step calls bit for
 * bit.  Refusals: those of kda_decode_front_end and kda_recurrent_k_bf16_norm.
 */
int kda_decode_fused_k(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state, float* conv_snapshots,
                       const float* gate, const float* beta, float* state, float* snapshots, int n_snapshots,
                       const uint16_t* out_gate, const uint16_t* o_norm, float norm_eps, float l2_eps, uint16_t* y,
                       float* out, int batch, int heads, int T, int conv_kernel, void* stream);
int kda_decode_fused_step(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state, const float* gate,
                          const float* beta, float* state, const uint16_t* out_gate, const uint16_t* o_norm,
                          float norm_eps, float l2_eps, uint16_t* y, float* out, int batch, int heads,
                          int conv_kernel, void* stream);

/*
 * kda_decode_fused_k / kda_decode_fused_step with the gate and beta formed in
 * the kernel from the gate's projection and beta's logits, as
 * kda_recurrent_k_gated forms them (g_raw, beta_logit, dt_bias, a_log,
 * gate_lower_bound as there; gate and beta are not taken).  Everything else as
 * kda_decode_fused_k; refusals also those of kda_recurrent_k_gated.
 */
int kda_decode_fused_k_gated(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                             float* conv_snapshots, const uint16_t* g_raw, const float* beta_logit,
                             const float* dt_bias, const float* a_log, float gate_lower_bound, float* state,
                             float* snapshots, int n_snapshots, const uint16_t* out_gate, const uint16_t* o_norm,
                             float norm_eps, float l2_eps, uint16_t* y, float* out, int batch, int heads, int T,
                             int conv_kernel, void* stream);
int kda_decode_fused_step_gated(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                                const uint16_t* g_raw, const float* beta_logit, const float* dt_bias,
                                const float* a_log, float gate_lower_bound, float* state, const uint16_t* out_gate,
                                const uint16_t* o_norm, float norm_eps, float l2_eps, uint16_t* y, float* out,
                                int batch, int heads, int conv_kernel, void* stream);

/*
 * The step before the core on the prefill path: the same conv1d update, SiLU
 * and L2 on q and k as kda_decode_front_end, over the T tokens of a prefill,
 * written into the chunk-padded FP32 inputs kda_chunk_prefill reads
 * (workspace page, fields q_f32 / k_f32 / v_f32: the FP32 padded prefill
 * inputs, q and k after their L2 step and v as convolved; module page,
 * pipeline line).  The pages
 * round the conv output to BF16 (conv_out) before the L2; here conv, SiLU
 * and L2 are one pass and the values stay FP32 throughout.
 *
 *   qkv        : [batch][T][conv_dim] BF16, a token's q, k, v channels in one row (qkv_proj)
 *   conv_w     : [conv_dim][conv_kernel] BF16
 *   conv_state : [batch][conv_dim][conv_kernel] FP32, read, then advanced in
 *                place by the T inputs (afterwards it holds the inputs of the
 *                last conv_kernel tokens, older slots first, as T single
 *                decode front-end rows would leave it)
 *   q, k, v    : [batch][T_pad][heads][128] FP32, T_pad = ceil(T / chunk) *
 *                chunk: the q, k, v of kda_chunk_prefill for the same T and
 *                chunk.  Rows >= T are not written.
 *   chunk      : 16, 32 or 64 (KDA_ERR_UNSUPPORTED otherwise)
 *
 * Every row equals, bit for bit, the row kda_decode_front_end computes when
 * it walks the same T tokens from the same conv state.  All other arguments,
 * conventions and refusals are those of kda_decode_front_end (no snapshots).
 * The work is two launches on the stream (the outputs, then the conv state).
 */
int kda_prefill_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                          float* v, int batch, int heads, int T, int chunk, int conv_kernel, float l2_eps,
                          void* stream);

/*
 * kda_prefill_front_end for sequences of their own lengths packed back to
 * back, producing the inputs of kda_chunk_prefill_varlen.
 *
 *   qkv        : [total_tokens][conv_dim] BF16
 *   conv_state : [n_seqs][conv_dim][conv_kernel] FP32, one per sequence, each
 *                advanced in place by its own tokens (an empty sequence keeps
 *                its state)
 *   q, k, v    : [total_tokens][heads][128] FP32; rows of sequence s are
 *                cu_seqlens[s] .. cu_seqlens[s + 1] - 1; rows from
 *                cu_seqlens[n_seqs] on belong to no sequence and are not
 *                written
 *   cu_seqlens : DEVICE int32 [n_seqs + 1], expected 0 = cu_seqlens[0] <= ...
 *                <= cu_seqlens[n_seqs] <= total_tokens (as for
 *                kda_chunk_prefill_varlen)
 *
 * No conv window reaches across a sequence boundary: the first row of each
 * sequence starts from that sequence's conv state.  Every row equals, bit
 * for bit, what kda_decode_front_end computes walking its sequence alone.
 * The offsets are read clamped to [0, total_tokens], so no content moves an
 * access outside the buffers; offsets that break the expected order give
 * unspecified values.  n_seqs at most KDA_VARLEN_MAX_SEQS; other arguments
 * and refusals as for kda_prefill_front_end (no chunk).
 */
int kda_prefill_front_end_varlen(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                                 float* v, const int* cu_seqlens, int n_seqs, int heads, int total_tokens,
                                 int conv_kernel, float l2_eps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
