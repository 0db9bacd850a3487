/*
 * spec_verify.h -- C ABI of libspecverify.so: batched speculative-sampling
 * verification over full-vocabulary bf16 logits on AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page and section:
 *   [LT] "Speculative Decoding 为什么是 Lossless 的 -- 详细证明教程" (restates
 *        Leviathan et al. 2023 App. A.1 and Chen et al. 2023 Thm 1; p = target,
 *        q = draft).
 *   [NB] Paper note "Not-a-Bandit: Provably No-Regret Drafter Selection in
 *        Speculative Decoding for LLMs" (HedgeSpec), Key designs 1-4.
 *   [CA] Paper note "Cactus: Accelerating Auto-Regressive Decoding with
 *        Constrained Acceptance Speculative Sampling", Key designs 1-3.
 *   [NH] Chaudhuri, Freund, Hsu, "A parameter-free hedging algorithm" (2009).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every array pointer is a DEVICE pointer owned by the caller.  The
 *   library allocates nothing and keeps no pointer after a call returns; its
 *   only memory between calls is a per-device cache of the resident-workgroup
 *   count.  The only memory it writes besides the outputs is the caller's
 *   workspace.
 * Streams.  Calls enqueue kernels on `stream` and return at once.  A non-zero
 *   return means nothing was launched (argument error) or the launch itself
 *   failed (SPEC_ERR_HIP); device faults surface at the caller's next
 *   synchronisation.
 * Logits.  Rows are bf16 (raw bit patterns), V-contiguous.  A row stride is in
 *   elements, must be >= V and a multiple of 8, and every base pointer must be
 *   16-byte aligned (rows are streamed with 128-bit loads).  When V is not a
 *   multiple of 8 the elements of a row from V up to the next multiple of 8 are
 *   read and ignored, so each row's storage must extend that far.  Logits must
 *   be finite or -inf, with at least one finite logit per row and
 *   |logit| / T < 6e8; anything else gives unspecified (but in-bounds) results.
 * Temperature.  One T > 0 scales every row, target and draft alike ([LT] §8 Q4:
 *   shaping is folded into both distributions before any ratio is formed).
 * Uniforms.  r and u are float32 in [0, 1), drawn by the caller: the library
 *   draws no random numbers.
 * Workspace.  `workspace` holds the values the kernel's workgroups hand to
 *   one another.  Size it with spec_workspace_bytes(B, K, N) (enough for any V
 *   up to SPEC_MAX_V) and zero it with spec_workspace_init() (or any zero fill)
 *   before its first use.  Every completed call leaves it all zero again, so
 *   back-to-back calls need no clearing, whatever their shapes, as long as
 *   each fits.  The 32-bit word at byte offset 12 is a fault word: a call sets
 *   it non-zero when a wait between its workgroups times out (after 2 s; this
 *   needs the device to be shared with work that keeps part of the grid from
 *   running, or a workspace that was not zero at launch).  The outputs of that
 *   call are then unspecified and the workspace must be zeroed again.  Calls
 *   that run concurrently must use different workspaces.
 * Residency.  The verification and gamma kernels launch exactly as many
 *   workgroups as the device holds at once, and their workgroups wait for
 *   values other workgroups publish.  Precondition: no other kernel occupies
 *   the device's compute units while such a call runs (no concurrent kernels
 *   on other streams).  If one does, part of the grid may not be resident, a
 *   wait times out after 2 s, the fault word is set and that call's outputs are
 *   unspecified; the Python binding's synchronisation points (Launcher.check,
 *   HedgeSpecLoop.check) raise WorkspaceFault then and zero the workspace.
 * Bad token ids.  A drafted or trajectory token outside [0, V) is reported in
 *   the outputs (see each call), never by a fault.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t spec_bf16;      /* raw bf16 bits */
struct ihipStream_t;             /* hipStream_t == struct ihipStream_t* */
typedef struct ihipStream_t* spec_stream_t;

enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = -1,      /* a required pointer is NULL */
  SPEC_ERR_SHAPE = -2,     /* B, K, N, V out of range or stride < V / not a multiple of 8 */
  SPEC_ERR_PARAM = -3,     /* temperature, delta or loss_scale not finite / out of range */
  SPEC_ERR_ALIGN = -4,     /* a logits base pointer is not 16-byte aligned */
  SPEC_ERR_WORKSPACE = -5, /* workspace NULL, misaligned or smaller than spec_workspace_bytes() */
  SPEC_ERR_HIP = -6,       /* the HIP launch failed */
  SPEC_ERR_TOO_LARGE = -7  /* spec_verify_noalloc: the call needs more than SPEC_NOALLOC_MAX_BYTES of scratch */
};

/* Learners of hedge_censored_update. */
enum { SPEC_LEARNER_NORMALHEDGE = 0, SPEC_LEARNER_HEDGE = 1 };

/* Limits checked by every call. */
#define SPEC_MAX_B 65536       /* sequences per call */
#define SPEC_MAX_V (1 << 20)   /* vocabulary size */
#define SPEC_MAX_K 64          /* draft positions per sequence */
#define SPEC_MAX_N 64          /* drafters */
#define SPEC_NOALLOC_MAX_BYTES (16u << 20)  /* scratch of spec_verify_noalloc, per device */

/* Human-readable text for a status code (static storage). */
const char* spec_status_str(int status);

/* Bytes of workspace one call with these B, K, N needs (N = 1 for the
 * verify calls), for any V up to SPEC_MAX_V; 0 when B, K or N is out of range.
 * A workspace must be 256-byte aligned. */
size_t spec_workspace_bytes(int B, int K, int N);

/* Zero `bytes` of workspace on `stream` with a fill kernel (no memset node). */
int spec_workspace_init(void* workspace, size_t bytes, spec_stream_t stream);

/*
 * spec_verify -- lossless speculative sampling, K drafts per sequence.
 *
 * Computes, for every sequence b, the standard draft-then-verify round of [LT]
 * §5.1 (SpecSampleOne) chained over K positions as in [LT] §9.1:
 *   pt_k = softmax(target[b][k] / T), pd_k = softmax(draft[b][k] / T);
 *   position k accepts its drafted token t iff r[b][k] < pt_k(t) / pd_k(t)
 *   (strict; [LT] §2.2 and §5.1);
 *   A = the first rejected position, or K if every position accepts;
 *   if A < K: out_token = inverse CDF of (pt_A - pd_A)+ at u[b][A] * Z, with
 *     Z = sum (pt_A - pd_A)+  ([LT] §2.2, §6.4 Step 3a); if Z is exactly 0
 *     the token is drawn from pt_A instead;
 *   if A == K: out_token = inverse CDF of pt_K at u[b][K] (the bonus token of
 *     the (K+1)-th target position).
 * The inverse CDF is over ascending token ids: the smallest j with C_j > x.
 *
 * target        [B][K+1] rows, row (b,k) at target + (b*(K+1)+k)*target_row_stride
 * draft         [B][K] rows,   row (b,k) at draft + (b*K+k)*draft_row_stride
 * draft_tokens  [B][K] int32 drafted ids
 * r_accept      [B][K] float32 accept uniforms
 * u_resample    [B][K+1] float32 resample / bonus uniforms
 * accepted_len  [B] int32 out: A in [0, K], or -1 if any drafted id of the
 *               sequence is outside [0, V)
 * out_token     [B] int32 out: the resampled or bonus token, -1 as above
 * accept_mask   [B][K] uint8 out or NULL: each position's own test (1 accept),
 *               evaluated at every position, including after the first
 *               rejection; 0 for an invalid id
 * Limits: 1 <= B <= SPEC_MAX_B, 1 <= K <= SPEC_MAX_K, 1 <= V <= SPEC_MAX_V,
 * T > 0 finite.
 */
int spec_verify(const spec_bf16* target, int64_t target_row_stride,
                const spec_bf16* draft, int64_t draft_row_stride,
                const int32_t* draft_tokens, const float* r_accept, const float* u_resample,
                int B, int K, int V, float temperature,
                int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                void* workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory: code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same computation, arguments, outputs and status codes as
 * spec_verify, without the workspace: the call uses a device array inside the
 * library (SPEC_NOALLOC_MAX_BYTES, one per device, held until the process ends)
 * and calls no allocating routine.  Its first call on a device looks up that
 * device's copy (hipGetSymbolAddress): make it outside graph capture.  Every
 * call clears the part of the array it uses with a fill kernel on `stream`, then
 * verifies.  A call whose layout (spec_workspace_bytes(B, K, 1)) exceeds the
 * array returns SPEC_ERR_TOO_LARGE and launches nothing.  All calls on one
 * device share the array: calls that overlap on one device (different streams
 * or threads without ordering) race and give unspecified results.
 */
int spec_verify_noalloc(const spec_bf16* target, int64_t target_row_stride,
                        const spec_bf16* draft, int64_t draft_row_stride,
                        const int32_t* draft_tokens, const float* r_accept, const float* u_resample,
                        int B, int K, int V, float temperature,
                        int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                        spec_stream_t stream);

/*
 * spec_cactus_verify -- Cactus constrained acceptance, m drafts per sequence.
 *
 * [CA] Key designs 1-3 with Cactus's q = the verifier softmax pt and p = the
 * draft softmax pd.  At position k with candidate n = draft_tokens[b][k]:
 *   c = pt_k(n); gamma* = min(c + sqrt(2 delta c (1 - c)), 1)   (Key design 3);
 *   accept iff r[b][k] < gamma* / pd_k(n)  (acceptance min(1, h_n / pd(n)));
 * at the first rejection A the token is drawn from g = (h - pd_A)+ / Z with the
 * closed-form target h of Key design 2: h_n = gamma*, h_x = s * pt_A(x) for
 * x != n, s = (1 - gamma*) / (1 - c) (s = 0 when c = 1); if Z is exactly 0
 * the token is drawn from h.  If all m accept, the bonus is drawn from pt_m.
 * delta = 0 runs exactly the spec_verify arithmetic (h == pt), so both calls
 * return bit-identical results on the same inputs.
 *
 * Layout and outputs as spec_verify with K = m, plus
 * gamma_star    [B][m] float32 out or NULL: gamma* at every position.
 * delta >= 0 and finite.
 */
int spec_cactus_verify(const spec_bf16* verifier, int64_t verifier_row_stride,
                       const spec_bf16* draft, int64_t draft_row_stride,
                       const int32_t* draft_tokens, const float* r_accept, const float* u_resample,
                       int B, int m, int V, float delta, float temperature,
                       int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                       float* gamma_star,
                       void* workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_cactus_kl_verify -- Cactus with gamma* the exact root of the KL budget.
 *
 * [CA] Key designs 1-2 with the KL divergence, without the second-order Taylor
 * step of Key design 3 (which the note derives because the equation has no
 * closed form).  gamma* is the largest g in [c, 1] whose target h (h_n = g,
 * h_x = (1 - g) / (1 - c) * pt(x) otherwise) keeps KL(h || pt) <= delta; for
 * that h the divergence is g ln(g / c) + (1 - g) ln((1 - g) / (1 - c)).
 * gamma* = 1 when -ln c <= delta, and c when delta = 0 or c = 0.  It is found
 * in float64 (bracketed Newton steps, at most 100, to a few ulps).  Everything
 * else -- the acceptance test, the recovery draw, the bonus, the layout, the
 * outputs, the workspace and the status codes -- is spec_cactus_verify's, and
 * delta = 0 again returns exactly the spec_verify results.  The Taylor value
 * never exceeds this gamma* where it is <= 0.5 (Corollary 6), so this call
 * accepts at least as often there.
 */
int spec_cactus_kl_verify(const spec_bf16* verifier, int64_t verifier_row_stride,
                          const spec_bf16* draft, int64_t draft_row_stride,
                          const int32_t* draft_tokens, const float* r_accept, const float* u_resample,
                          int B, int m, int V, float delta, float temperature,
                          int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                          float* gamma_star,
                          void* workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_counterfactual_gamma -- HedgeSpec full-information evaluation of N drafters.
 *
 * For every sequence b, position k < K and drafter i ([NB] Key design 1, and
 * [LT] §6.3 for the identity with the acceptance probability):
 *   gamma[b][k][i] = sum_x min(pt_k(x), pd_{i,k}(x)) = 1 - TV(pt_k, pd_{i,k}).
 * With the realised trajectory tokens x_k = traj_tokens[b][k] and
 *   a_k = min(1, pd_{i,k}(x_k) / pt_k(x_k)),
 * the one-step acceptance-length estimator ([NB] Key design 2; the printed
 * formula was lost, this is the reading that is unbiased with range [1, K+1])
 *   est_len[b][i] = 1 + sum_{k<K} gamma[b][k][i] * prod_{j<k} a_j
 * and the loss ([NB] Key design 3, length objective)
 *   loss[b][i] = (K + 1) - est_len[b][i].
 * Only traj_tokens[b][0..K-2] enter; an id outside [0, V) there makes
 * est_len and loss of that sequence NaN (gamma is still written).
 *
 * target        rows (b,k) at target + (b*target_rows_per_seq + k)*target_row_stride,
 *               k < K (k = K also used by the fused verify below)
 * drafts        row (i,b,k) at drafts + i*drafter_stride + (b*K+k)*draft_row_stride
 * gamma [B][K][N], est_len [B][N], loss [B][N]  float32 out.
 *
 * Fused verify (one launch for evaluation and verification): when sel is not
 * NULL, every sequence b is also verified exactly as spec_verify does, using
 * drafter sel[b]'s rows as the draft, draft_tokens / r_accept / u_resample as
 * in spec_verify, and target row K of the sequence for the bonus (so
 * target_rows_per_seq must be K+1); results go to accepted_len / out_token /
 * accept_mask (accept_mask may be NULL).  A sel[b] outside [0, N) makes that
 * sequence's accepted_len and out_token -1.
 * Limits: 1 <= N <= SPEC_MAX_N, target_rows_per_seq >= K (K+1 when fused).
 * Workspace: spec_workspace_bytes(B, K, N).
 */
int spec_counterfactual_gamma(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                              const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                              const int32_t* traj_tokens,
                              int B, int K, int N, int V, float temperature,
                              float* gamma, float* est_len, float* loss,
                              const int32_t* sel, const int32_t* draft_tokens,
                              const float* r_accept, const float* u_resample,
                              int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                              void* workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_tree_gamma -- HedgeSpec acceptance probabilities under a greedy draft tree.
 *
 * [NB] Key design 1, the draft-tree case (its Theorem 2): at the node of
 * position k the acceptance probability of drafter i is the total target
 * probability of the children drafter i keeps there.  Here the children are the
 * drafter's topk most likely tokens (the topk largest logits of its row k, ties
 * to the smaller token id; its softmax keeps that order at any temperature):
 *   gamma[b][k][i] = sum over those tokens x of pt_k(x),
 * with pt_k = softmax(target row k / temperature) of sequence b.
 *
 * target  [B][target_rows_per_seq][V] bf16 (rows 0..K-1 are read), row stride
 *         target_row_stride elements; drafts [N][B][K][V] bf16, row stride
 *         draft_row_stride, drafter stride drafter_stride elements (as
 *         spec_counterfactual_gamma);  gamma [B][K][N] float32 out.
 * Limits: 1 <= N <= SPEC_MAX_N, 1 <= topk <= 64 (SPEC_ERR_PARAM otherwise; a
 * topk of V or more keeps every token, gamma = 1), target_rows_per_seq >= K.
 * Workspace: spec_tree_workspace_bytes(B, K, N, V, topk) bytes (a workspace
 * sized for V serves every smaller V), zeroed once (spec_workspace_init); every
 * call leaves it zero.  Other conventions
 * (alignment, strides, status codes, asynchrony) as spec_verify.
 */
int spec_tree_gamma(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                    const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                    int B, int K, int N, int V, int topk, float temperature,
                    float* gamma, void* workspace, size_t workspace_bytes, spec_stream_t stream);

/* Workspace bytes of spec_tree_gamma for vocabularies up to V; 0 for sizes out of range. */
size_t spec_tree_workspace_bytes(int B, int K, int N, int V, int topk);

/*
 * hedge_update -- one NormalHedge round per sequence ([NH]; named by [NB] Key
 * design 3 as the full-information learner; one learner per sequence).
 *
 * For every b with has_loss[b] != 0 (or every b if has_loss is NULL), with
 * l_i = loss[b][i] * loss_scale and w = weights[b]:
 *   lhat = sum_i w_i l_i;  cum_regret[b][i] += lhat - l_i;
 *   if no cum_regret[b][i] > 0: weights[b] = uniform; otherwise find c > 0 with
 *   (1/N) sum_i exp([R_i]+^2 / (2c)) = e (fp64 Newton steps from the left end of
 *   [M^2 / (2(1 + ln N)), M^2 / 2], M = max [R]+, to 1e-15 of c) and set
 *   weights[b][i] proportional to ([R_i]+ / c) exp([R_i]+^2 / (2c)).
 * Then, if v_select is not NULL, sel_out[b] = the inverse CDF of weights[b]
 * at v_select[b] (the next drafter, drawn from the weights).
 *
 * cum_regret, weights  [B][N] float64 in/out, caller-owned learner state
 *                      (initialise to 0 and 1/N)
 * loss [B][N] float32; has_loss [B] uint8 or NULL; loss_scale finite >= 0
 * (1/K maps the length loss in [0, K] onto [0, 1]); v_select [B] float32 or
 * NULL; sel_out [B] int32 (required when v_select is given).
 */
int hedge_update(double* cum_regret, double* weights,
                 const float* loss, const uint8_t* has_loss, float loss_scale,
                 const float* v_select, int32_t* sel_out,
                 int B, int N, spec_stream_t stream);

/*
 * hedge_exp_update -- one exponential-weights Hedge round per sequence ([NB]
 * Key design 3 names Hedge beside NormalHedge as the full-information learner).
 *
 * For every b with has_loss[b] != 0 (or every b if has_loss is NULL):
 *   cum_loss[b][i] += loss[b][i] * loss_scale;
 *   weights[b][i] = exp(-eta cum_loss[b][i]) / sum_j exp(-eta cum_loss[b][j])
 * (fp64, evaluated against min_j cum_loss[b][j]).  Then, if v_select is not
 * NULL, sel_out[b] = the inverse CDF of weights[b] at v_select[b], as
 * hedge_update.
 *
 * cum_loss, weights  [B][N] float64 in/out, caller-owned learner state
 *                    (initialise to 0 and 1/N)
 * loss [B][N] float32; has_loss [B] uint8 or NULL; loss_scale and eta finite
 * and >= 0 (SPEC_ERR_PARAM otherwise); v_select [B] float32 or NULL; sel_out
 * [B] int32 (required when v_select is given).  1 <= N <= SPEC_MAX_N.
 */
int hedge_exp_update(double* cum_loss, double* weights, const float* loss, const uint8_t* has_loss,
                     float loss_scale, float eta, const float* v_select, int32_t* sel_out,
                     int B, int N, spec_stream_t stream);

/*
 * hedge_queue_update -- one round of per-sequence NormalHedge under delayed
 * feedback, with the feedback queue resident on the device ([NB] Key design 3:
 * the stochastic-setting reduction keeps a queue of losses and applies each as it
 * becomes available), so that rounds can follow each other without the host
 * (e.g. in a captured graph).  Sequence b's call at round t = round[b]:
 *   1. if t > 0, queues round t-1's loss[b][*] * loss_scale, usable at round
 *      t + delays[(t-1) B + b] (a delay of -1 never arrives);
 *   2. applies every queued loss usable at round t, one NormalHedge step each
 *      (as hedge_update), in order of (usable round, origin round);
 *   3. draws round t's drafter: sel_out[b] = inverse CDF of weights[b] at
 *      v_select[t B + b]; sel_hist[t B + b] = sel_out[b];
 *   4. round[b] = t + 1.  Calls with round[b] >= T do nothing.
 * This is the schedule of hedge_update applied as the host-side queue does
 * (losses of round s usable at round s + 1 + d_s).
 *
 * cum_regret, weights [B][N] float64 state (0 and 1/N to start);
 * queue_loss [B][Q][N] float64 and queue_due [B][Q] int32 the queue (queue_due
 * all -1 to start); round [B] int32 (0 to start); loss [B][N] float32 (round
 * t-1's); delays [T][B] int32 in [-1, Q-2]; v_select [T][B] float32; sel_out
 * [B], sel_hist [T][B] int32.  2 <= Q <= 256, 1 <= N <= SPEC_MAX_N.
 */
int hedge_queue_update(double* cum_regret, double* weights, double* queue_loss, int32_t* queue_due, int32_t* round,
                       const float* loss, const int32_t* delays, float loss_scale, const float* v_select,
                       int32_t* sel_out, int32_t* sel_hist, int B, int N, int Q, int T, spec_stream_t stream);

/*
 * hedge_censored_update -- one round of per-sequence learning under the delay that
 * censoring causes ([NB] Key design 3: a round's loss can only be scored once the
 * chunk after it is verified, so feedback arrives late; the learner keeps a queue
 * and applies each loss once it is complete).  Round s's loss is usable once K
 * more tokens have been verified after round s, each round verifying its
 * accepted drafts plus one token; the tokens are counted on the device, from the
 * accepted lengths the rounds produce, so no schedule is needed in advance.
 * Sequence b's call at round t = round[b] (< T; later calls do nothing):
 *   1. if t > 0, adds accepted_len[b] + 1 (round t-1's tokens; 0 if negative) to
 *      the token count of every queued loss;
 *   2. applies every queued loss whose count has reached K, oldest round first,
 *      one learner step each (as hedge_update / hedge_exp_update), and frees it;
 *   3. if t > 0, queues round t-1's loss[b][*] * loss_scale with count 0 in slot
 *      (t-1) % Q; a loss still queued in that slot (from round t-1-Q, possible
 *      only after rounds that verified nothing) is dropped: it never arrives;
 *   4. draws round t's drafter: sel_out[b] = inverse CDF of weights[b] at
 *      v_select[t B + b]; sel_hist[t B + b] = sel_out[b]; round[b] = t + 1.
 * learner: SPEC_LEARNER_NORMALHEDGE (state = cumulative regret, as hedge_update)
 * or SPEC_LEARNER_HEDGE (state = cumulative loss, weights exp(-eta L), as
 * hedge_exp_update).
 *
 * state, weights [B][N] float64 (0 and 1/N to start); queue_loss [B][Q][N]
 * float64 and queue_tokens [B][Q] int32 (all -1 to start); round [B] int32 (0 to
 * start); loss [B][N] float32 and accepted_len [B] int32 (round t-1's, e.g. the
 * outputs of a fused spec_counterfactual_gamma); v_select [T][B] float32;
 * sel_out [B], sel_hist [T][B] int32.  1 <= K <= SPEC_MAX_K, K + 1 <= Q <= 256,
 * 1 <= N <= SPEC_MAX_N; loss_scale and eta finite and >= 0.
 */
int hedge_censored_update(double* state, double* weights, double* queue_loss, int32_t* queue_tokens, int32_t* round,
                          const float* loss, const int32_t* accepted_len, int K, int learner, float eta,
                          float loss_scale, const float* v_select, int32_t* sel_out, int32_t* sel_hist, int B, int N,
                          int Q, int T, spec_stream_t stream);

/*
 * spec_hedgespec_round -- one whole HedgeSpec round in one launch ([NB] overall
 * framework: the learner selects a drafter per sequence, that drafter's chunk is
 * verified, and every drafter is evaluated on the verified trajectory; Key
 * designs 1-3).  It computes exactly what hedge_censored_update (steps 1-4 above,
 * with these state arguments) followed by the fused spec_counterfactual_gamma
 * with sel = this round's selections computes, but the learner step runs inside
 * the gamma launch: the waves of its first gamma slot take every sequence's step
 * at the kernel's start (that slot then takes no gamma rows) and hand each
 * sequence's drafter to its draw units, so a round is one kernel and no node gap.
 * Like the other verification calls, it assumes that no other kernel holds the
 * device's compute units while it runs (its waits between workgroups end after
 * 2 s otherwise, with the workspace's fault word set).
 *
 * loss [B][N] and accepted_len [B] are both the previous round's outputs, which
 * the learner reads, and this round's, which the launch writes (the estimator
 * waits for the learner before it overwrites loss).  sel [B] receives this
 * round's drafters.  Every other argument is as in spec_counterfactual_gamma
 * (fused form: draft_tokens, r_accept, u_resample, accepted_len and out_token
 * required) and hedge_censored_update; the workspace is a
 * spec_workspace_bytes(B, K, N) one.  Status codes as there.
 */
int spec_hedgespec_round(const spec_bf16* target, int64_t target_row_stride, int target_rows_per_seq,
                         const spec_bf16* drafts, int64_t draft_row_stride, int64_t drafter_stride,
                         const int32_t* traj_tokens, int B, int K, int N, int V, float temperature, float* gamma,
                         float* est_len, float* loss, const int32_t* draft_tokens, const float* r_accept,
                         const float* u_resample, int32_t* accepted_len, int32_t* out_token, uint8_t* accept_mask,
                         double* state, double* weights, double* queue_loss, int32_t* queue_tokens, int32_t* round,
                         int learner, float eta, float loss_scale, const float* v_select, int32_t* sel,
                         int32_t* sel_hist, int Q, int T, void* workspace, size_t workspace_bytes,
                         spec_stream_t stream);

/*
 * spec_acceptance_loss -- [NB] Key design 3's loss when the acceptance probability
 * is optimised: f = 1 - gamma at every position, a chunk's K positions summed:
 *   loss[b][i] = sum_k (1 - gamma[b][k][i])   (fp64 sum, stored as float32)
 * gamma [B][K][N] float32 (spec_counterfactual_gamma or spec_tree_gamma),
 * loss [B][N] float32 out, in [0, K].
 */
int spec_acceptance_loss(const float* gamma, float* loss, int B, int K, int N, spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
