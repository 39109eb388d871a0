/*
 * libdspark: the per-step sampling hot path of DSpark confidence-scheduled
 * speculative decoding, as hand-written HIP kernels for CDNA4 (gfx950).
 *
 * Sources (web pages on DSpark, cited by site and section):
 *   [weigao]   weigao.cc "DSpark 与 MTP：DeepSeek 投机解码调研", section
 *              "DSpark 的核心设计" parts 2-4.
 *   [billytse] billytse.dev "DSpark：DeepSeek 點樣「一次估多個、驗證前綴、
 *              錯咗即修正」", sections 1, 3.2, 3.3, 5, 6, 7.
 *   [xhh]      xhh.club "DeepSeek-V4.1 模型结构（6）：解码，DSpark", Q&A on
 *              the acceptance rule and the scheduler; note on
 *              non-anticipating truncation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array pointer is a DEVICE pointer owned by the caller; the
 *    library never frees or retains it.  Arrays are dense, row-major, and
 *    16-byte aligned.  Nothing is allocated by the library.
 *  - Calls are asynchronous on `stream` (NULL = the default stream), keep no
 *    state between calls (except the process-wide setting of
 *    dspark_set_draft_path and the scratch of dspark_schedule_noalloc), and
 *    may be issued from several host threads.
 *  - Arguments are validated on the host BEFORE anything is enqueued; on a
 *    validation error the call returns a negative status, enqueues nothing,
 *    and dspark_last_error() (thread-local) describes the problem.
 *  - Data errors found on the device never abort: they OR bit flags
 *    (DSPARK_DEV_*) into the optional int32 word `*status` (may be NULL),
 *    which the caller clears before the step, and the affected outputs stay
 *    in range (token ids within [0, V)).
 *  - dtype selects the element type of the large tensors (U, target, W1,
 *    W2, hidden): DSPARK_BF16 (bit patterns, round-to-nearest-even) or
 *    DSPARK_F32.  Accumulation is fp32 (bf16 inputs use MFMA), cross-tile
 *    sums and cumulative sums are fp64.
 *  - Shapes: V % 8 == 0 and V <= 262144 (larger: DSPARK_EUNSUPPORTED);
 *    rank in {32, 64, 128, 256} for bf16 (the matrix-core path keeps
 *    64 x rank tiles of W2 in LDS and registers), any multiple of 32 in
 *    [32, 512] for fp32; H % 8 == 0; 1 <= gamma <= 64; B >= 1.
 *  - Positions are 0-based: draft position k (0..gamma-1) is the pages'
 *    x_{k+1}.
 *  - uniforms [B, gamma+1, 2] fp32 in [0,1): uniforms[b,k,0] draws draft
 *    token k; uniforms[b,k,1] is the accept test of draft token k;
 *    uniforms[b,gamma,0] draws the one final token (residual or bonus);
 *    uniforms[b,gamma,1] is unused.
 *  - temperature [B] fp32: logits are divided by T; T <= 0 (or NaN) means
 *    greedy: lowest-index argmax, and q and p become one-hot.
 *  - Inverse-CDF convention: the drawn token is the lowest index whose
 *    cumulative probability exceeds u.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = -1,       /* bad size, count or NULL pointer            */
  DSPARK_EDTYPE = -2,       /* unknown dtype                              */
  DSPARK_EALIGN = -3,       /* pointer not 16-byte aligned                */
  DSPARK_EWORKSPACE = -4,   /* workspace missing or too small             */
  DSPARK_EUNSUPPORTED = -5, /* valid but outside what the kernels support */
  DSPARK_EHIP = -6          /* a HIP runtime call failed                  */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* device-side data-error flags ORed into *status */
#define DSPARK_DEV_BAD_TOKEN   1  /* anchor/token id outside [0,V); clamped     */
#define DSPARK_DEV_NONFINITE   2  /* NaN/Inf logits or stats; token 0 emitted   */
#define DSPARK_DEV_DEGENERATE  4  /* residual had no mass; drew from p instead  */
#define DSPARK_DEV_BAD_ELL     8  /* ell outside [0,gamma]; clamped             */
#define DSPARK_DEV_BAD_CONF   16  /* confidence NaN or outside [0,1]; clamped   */
#define DSPARK_DEV_TIMEOUT    32  /* a cross-work-group wait gave up; results of
                                     the call are undefined (never expected)   */

const char* dspark_status_str(int status);
const char* dspark_last_error(void);
/* library version, e.g. "libdspark 0.1 gfx950" */
const char* dspark_version(void);

/* ------------------------------------------------------------------------
 * dspark_draft_block: semi-autoregressive block drafting with the vanilla
 * Markov head ([billytse] 3.2-3.3; [weigao] part 2).
 *
 * For each request b, starting from prev = anchor[b], for k = 0..gamma-1:
 *     z      = U[b,k,:] + W1[prev,:] @ W2          (rank-r transition bias)
 *     x      = inverse-CDF draw from softmax(z / T_b) with uniforms[b,k,0]
 *     prev   = x
 * W2 is the rank -> V projection, [rank, V] row-major: bias[v] =
 * sum_i W1[prev,i] * W2[i,v].  The kernels transpose each 64-entry tile of
 * W2 on chip; no transposed copy is made in memory.
 *
 * in : U [B,gamma,V], W1 [V,rank], W2 [rank,V] (dtype); anchor [B] int32;
 *      temperature [B], uniforms [B,gamma+1,2] fp32
 * out: tokens [B,gamma] int32; q_tok [B,gamma] fp32 = q_k(x_k);
 *      row_max [B,gamma] = max_v z/T (max z when greedy);
 *      row_logZ [B,gamma] = log sum_v exp(z/T - row_max) (0 when greedy).
 * workspace: dspark_draft_block_workspace(...) bytes of device memory,
 *      zero-filled before its first use (e.g. one hipMemset after the
 *      allocation).  Every call leaves it ready for the next one (whatever
 *      its shape or dtype), so a workspace kept for later calls needs no
 *      clearing, except after a call that raised DSPARK_DEV_TIMEOUT: zero it
 *      again then.  Calls that share one workspace must not overlap.
 * No full probability row is ever written.
 * The single-launch (persistent) implementation synchronises its work-groups
 * with bounded waits and reports a wait that gave up (DSPARK_DEV_TIMEOUT)
 * through `status` only; with status NULL the per-position launches run
 * instead (same results, no waits), and the persistent-only settings of
 * dspark_set_draft_path make the call return DSPARK_EINVAL.
 * ---------------------------------------------------------------------- */
size_t dspark_draft_block_workspace(int B, int gamma, int V, int rank, int dtype);
int dspark_draft_block(int B, int gamma, int V, int rank, int dtype,
                       const void* U, const void* W1, const void* W2,
                       const int32_t* anchor, const float* temperature,
                       const float* uniforms,
                       int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                       int32_t* status, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_draft_block_conf: dspark_draft_block and the confidence head of the
 * drafted block in one call ([billytse] 3.3 and 5; [weigao] parts 2-3: the
 * head scores position k from its hidden state and the token drawn before
 * it, so each score is available as soon as that token is).  conf[b,k] is
 * bit for bit what dspark_confidence (temps NULL) or dspark_confidence_sts
 * (temps given) returns for the drafted tokens.  The single-launch kernel's
 * draw waves evaluate the head while they wait for each position's
 * statistics, which saves the head's launch; where that kernel does not run
 * the head's own kernel follows the draft (same results).
 * in : as dspark_draft_block, plus hidden [B,gamma,H] (dtype; H % 8 == 0),
 *      w [H+rank] fp32, bias, temps [gamma] fp32 or NULL
 * out: as dspark_draft_block, plus conf [B,gamma] fp32
 * workspace, status and errors as dspark_draft_block.
 * ---------------------------------------------------------------------- */
int dspark_draft_block_conf(int B, int gamma, int V, int rank, int H, int dtype,
                            const void* U, const void* W1, const void* W2,
                            const int32_t* anchor, const float* temperature,
                            const float* uniforms,
                            const void* hidden, const float* w, float bias,
                            const float* temps,
                            int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                            float* conf,
                            int32_t* status, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_draft_block_rnn: block drafting with the RNN head instead of the
 * Markov head ([weigao] part 2, the _rnn_step description; [billytse] 3.3:
 * a recurrent state lets each position see the whole block prefix).
 * For each request b, with s = 0 and prev = anchor[b], for k = 0..gamma-1:
 *     pre   = Wr . [s ; W1[prev,:] ; hidden[b,k,:]] + br     (3 rank outputs)
 *     gate  = sigmoid(pre[0:r]), cand = tanh(pre[r:2r]), out = tanh(pre[2r:3r])
 *     s     = gate * s + (1 - gate) * cand
 *     emb[b,k,:] = out                    (rounded to dtype: the bias operand)
 *     z     = U[b,k,:] + emb[b,k,:] @ W2
 *     x     = inverse-CDF draw from softmax(z / T_b) with uniforms[b,k,0]
 *     prev  = x
 * (r = rank.  The activations of gate and candidate, the state size, the
 * layer's column order and the zero initial state are this library's
 * readings; the pages give the split and the two formulas.)
 * in : U [B,gamma,V], W1 [V,rank], W2 [rank,V], hidden [B,gamma,H],
 *      Wr [3 rank, 2 rank + H] (dtype; rows gate | candidate | output,
 *      columns state | embedding | hidden); br [3 rank] fp32; anchor,
 *      temperature, uniforms as dspark_draft_block
 * out: tokens, q_tok, row_max, row_logZ as dspark_draft_block;
 *      emb [B,gamma,rank] (dtype): the vector each position projected
 *      (dspark_verify_rnn takes it); state [B,gamma,rank] fp32: s after each
 *      position (or NULL)
 * Arithmetic: the hidden part of the layer for all positions is one bf16
 * matrix-core GEMM (fp32 out); the recurrence is fp32 (the state enters the
 * matrix cores as two bf16 parts, ~2^-17 relative); sampling as
 * dspark_draft_block.  Per-position launches (the single-launch kernel
 * serves the Markov head only).
 * workspace: dspark_draft_block_rnn_workspace(...) bytes; H % 8 == 0.
 * ---------------------------------------------------------------------- */
size_t dspark_draft_block_rnn_workspace(int B, int gamma, int V, int rank, int H, int dtype);
int dspark_draft_block_rnn(int B, int gamma, int V, int rank, int H, int dtype,
                           const void* U, const void* W1, const void* W2, const void* hidden,
                           const void* Wr, const float* br,
                           const int32_t* anchor, const float* temperature,
                           const float* uniforms,
                           int32_t* tokens, float* q_tok, float* row_max, float* row_logZ,
                           void* emb, float* state,
                           int32_t* status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_confidence: the confidence head ([weigao] part 3; [billytse] 5):
 *     conf[b,k] = sigmoid( w[0:H] . hidden[b,k,:] + w[H:H+rank] . W1[prev_k,:]
 *                          + bias )
 * with prev_0 = anchor[b] and prev_k = tokens[b,k-1] -- the token BEFORE
 * position k, never position k's own token ([xhh], non-anticipation).
 * The Markov embedding of a token is its W1 row.
 * in : hidden [B,gamma,H], W1 [V,rank] (dtype); anchor [B], tokens [B,gamma]
 *      int32; w [H+rank] fp32; bias scalar
 * out: conf [B,gamma] fp32
 * ---------------------------------------------------------------------- */
int dspark_confidence(int B, int gamma, int H, int V, int rank, int dtype,
                      const void* hidden, const void* W1,
                      const int32_t* anchor, const int32_t* tokens,
                      const float* w, float bias, float* conf,
                      int32_t* status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_confidence_sts: the confidence head with sequential temperature
 * scaling ([billytse] 5.2: the raw head is overconfident, and STS calibrates
 * the cumulative probability from left to right; [weigao] part 3: the
 * scheduler needs absolute probabilities).  The pages give no formula; this
 * library's reading: one temperature per block position divides that
 * position's logit,
 *     conf[b,k] = sigmoid( (w . [hidden[b,k] ; W1[prev_k]] + bias) / temps[k] ),
 * and the scheduler's survival is the running product of these calibrated
 * conditionals (still non-increasing, so admitted sets stay prefixes).  The
 * temperatures are fitted offline, position by position from the left,
 * against the cumulative survival of calibration drafts.  temps [gamma] fp32
 * device array; temps[k] == 1 gives exactly dspark_confidence's value; a
 * temperature that is not finite and positive leaves the logit unchanged and
 * sets DSPARK_DEV_BAD_CONF.  Other arguments as dspark_confidence.
 * ---------------------------------------------------------------------- */
int dspark_confidence_sts(int B, int gamma, int H, int V, int rank, int dtype,
                          const void* hidden, const void* W1,
                          const int32_t* anchor, const int32_t* tokens,
                          const float* w, float bias, const float* temps, float* conf,
                          int32_t* status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_schedule: hardware-aware prefix scheduler ([weigao] part 4;
 * [billytse] 6-7; [xhh] scheduler Q&A).
 *     a[r,j]  = prod_{i<=j} conf[r,i]        (fp64, left to right)
 *     rank all (r,j) by a descending, ties by flat index r*gamma+j ascending
 *     Bt = R, tau = R, Theta = tau*sps[Bt]
 *     for each candidate in rank order: stop if Bt+1 >= sps_len or
 *       sps[Bt+1] <= 0; tau' = tau + a; Theta' = tau'*sps[Bt+1];
 *       admit iff Theta' > Theta (strict rise), else stop.
 *     tau is the exact sum of R and the admitted survivals rounded once to
 *     fp64 (double-double prefix sums on the device), so the result does
 *     not depend on a summation order.
 *     ell[r] = number of admitted positions of request r (always a prefix)
 * in : conf [R,gamma] fp32 (NaN / out of [0,1] clamped and flagged);
 *      sps [sps_len] fp64, steps per second at target batch Bt (entry Bt)
 * out: ell [R] int32; order [R*gamma] int32 flat ids in rank order (or
 *      NULL); stats [3] fp64 {n_admitted, tau, Theta} (or NULL)
 * Supports R*gamma <= 8192 (the keys live in one work-group's LDS).
 * workspace: dspark_schedule_workspace(R, gamma) bytes (the candidates'
 * ranks, int32, for R*gamma <= 4096; 0 beyond), 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t dspark_schedule_workspace(int R, int gamma);
int dspark_schedule(int R, int gamma, const float* conf,
                    const double* sps, int sps_len,
                    int32_t* ell, int32_t* order, double* stats,
                    int32_t* status, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_schedule_noalloc: dspark_schedule for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * device allocation): the same arguments and results without a workspace.
 * The candidates' ranks go to a scratch array of the library's own, 16 KB
 * (4096 int32) per device, held from the first call on a device until the
 * process ends; batches with R*gamma > 4096 need none.  The call allocates
 * nothing (it never calls the tracer either).  Every call on one device
 * shares that device's scratch: calls that overlap on one device (other
 * streams, other host threads) race and give undefined results; serialise
 * them.  R*gamma above what the scratch holds returns DSPARK_EUNSUPPORTED
 * (with the size limits of dspark_schedule no such batch exists).
 * ---------------------------------------------------------------------- */
int dspark_schedule_noalloc(int R, int gamma, const float* conf,
                            const double* sps, int sps_len,
                            int32_t* ell, int32_t* order, double* stats,
                            int32_t* status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_schedule_capacity: the two-step causal barrier ([billytse] 7;
 * [weigao] part 4, asynchronous scheduling).  The size of the next target
 * batch is fixed beforehand from older predictions; the current candidates
 * are still ranked by their latest survival, and the first K are verified:
 *     a[r,j] and the rank order exactly as dspark_schedule
 *     K = floor(*capacity) clamped to [0, R*gamma]; NaN or < 1 gives 0
 *     ell[r] = number of request r's candidates among the first K ranked
 *     (always a prefix; whether (r,j) is taken never reads conf[r, j+1..])
 * in : conf [R,gamma] fp32 (clamped and flagged as in dspark_schedule);
 *      capacity: DEVICE pointer to one fp64, read when the kernel runs (for
 *      example stats[0] written by a dspark_schedule call of an earlier
 *      step, so the chain needs no host round trip); 8-byte aligned
 * out: ell [R] int32; order [R*gamma] int32 (or NULL); stats [3] fp64
 *      {n_admitted, tau, NaN} (or NULL), tau as in dspark_schedule
 * workspace: dspark_schedule_workspace(R, gamma) bytes, as dspark_schedule.
 * ---------------------------------------------------------------------- */
int dspark_schedule_capacity(int R, int gamma, const float* conf,
                             const double* capacity,
                             int32_t* ell, int32_t* order, double* stats,
                             int32_t* status, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_schedule_threshold: fixed confidence threshold ([billytse] 8,
 * threshold sweep; [xhh] scheduler Q&A contrasts it with the load-dependent
 * rule).  Candidate (r,j) is verified iff a[r,j] >= threshold (fp64
 * comparison of the fp64 survival); a NaN threshold verifies nothing.
 * Survival never rises along a request, so ell[r] counts a prefix.
 * in/out and workspace as dspark_schedule_capacity; stats {n, tau, NaN}.
 * ---------------------------------------------------------------------- */
int dspark_schedule_threshold(int R, int gamma, const float* conf,
                              double threshold,
                              int32_t* ell, int32_t* order, double* stats,
                              int32_t* status, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_verify: lossless speculative rejection sampling ([billytse] 1;
 * [xhh] acceptance-rule Q&A).
 * For request b with verify length L = ell[b] (0..gamma):
 *   for k = 0..L-1: p = softmax(target[b,k,:]/T); accept draft token x_k iff
 *     uniforms[b,k,1] < p(x_k)/q_tok[b,k]; stop at the first reject j.
 *   reject at j: q_j is recomputed from U[b,j], W1, W2 and prev_j (bit-
 *     identical to the draft's logits; row_max/row_logZ normalise it), and
 *     one token is drawn from norm(max(0, p_j - q_j)) with uniforms[b,gamma,0].
 *   no reject : one bonus token is drawn from softmax(target[b,L,:]/T) with
 *     uniforms[b,gamma,0].
 * in : target [B,gamma+1,V] (slot gamma is the bonus slot when ell = gamma),
 *      U [B,gamma,V], W1 [V,rank], W2 [rank,V] (dtype); anchor, tokens int32; q_tok, row_max, row_logZ
 *      (outputs of dspark_draft_block); temperature, uniforms; ell [B]
 * out: out_tokens [B,gamma+1] int32: accepted prefix then the one drawn
 *      token, -1 padded; n_accepted [B] int32 (emitted = n_accepted + 1;
 *      the last emitted token is the next anchor); ratio [B,gamma] fp32 =
 *      p(x_k)/q(x_k) at tested positions, NaN elsewhere (or NULL).
 * workspace: dspark_verify_workspace(...) bytes.
 * ---------------------------------------------------------------------- */
size_t dspark_verify_workspace(int B, int gamma, int V, int rank, int dtype);
int dspark_verify(int B, int gamma, int V, int rank, int dtype,
                  const void* target, const void* U, const void* W1, const void* W2,
                  const int32_t* anchor, const int32_t* tokens, const float* q_tok,
                  const float* row_max, const float* row_logZ,
                  const float* temperature, const float* uniforms, const int32_t* ell,
                  int32_t* out_tokens, int32_t* n_accepted, float* ratio,
                  int32_t* status, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_verify_rnn: dspark_verify for drafts of dspark_draft_block_rnn.
 * Identical except that the q recompute at a rejected slot j takes its bias
 * from the drafter's own projected vector: z = U[b,j] + emb[b,j,:] @ W2
 * (bit-identical to the draft's logits), so the residual norm(max(0, p - q))
 * uses exactly the q the token was drawn from ([billytse] 1; [xhh]
 * acceptance-rule Q&A).  emb [B,gamma,rank] (dtype) replaces W1; every other
 * argument, output and the workspace are those of dspark_verify.
 * ---------------------------------------------------------------------- */
int dspark_verify_rnn(int B, int gamma, int V, int rank, int dtype,
                      const void* target, const void* U, const void* emb, const void* W2,
                      const int32_t* anchor, const int32_t* tokens, const float* q_tok,
                      const float* row_max, const float* row_logZ,
                      const float* temperature, const float* uniforms, const int32_t* ell,
                      int32_t* out_tokens, int32_t* n_accepted, float* ratio,
                      int32_t* status, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * dspark_tv_label: the confidence head's training label per drafted
 * position ([weigao] part 3; [billytse] 5.1):
 *     tv[b,k]    = 0.5 * sum_v |p_k(v) - q_k(v)|
 *     label[b,k] = 1 - tv[b,k]  (= the probability that the acceptance test
 *                                 of dspark_verify keeps drafted token k)
 *   q_k = softmax((U[b,k] + W1[prev] W2) / T), prev = anchor[b] (k = 0)
 *         or tokens[b,k-1]: the distribution dspark_draft_block drew token k
 *         from, recomputed bit-identically and normalised with its row_max /
 *         row_logZ outputs;
 *   p_k = softmax(target[b,k] / T) (target slots 0..gamma-1; the bonus slot
 *         is not read);
 *   greedy requests (T <= 0): tv = 0 if tokens[b,k] is the target row's
 *         lowest-index argmax, else 1.
 * Sums: per element fp32, per 64-entry tile fp32, across tiles fp64.
 * in : target [B,gamma+1,V], U [B,gamma,V], W1 [V,rank], W2 [rank,V] (dtype);
 *      anchor [B], tokens [B,gamma] int32; row_max, row_logZ [B,gamma] fp32
 *      (dspark_draft_block outputs); temperature [B]
 * out: tv [B,gamma] fp32; label [B,gamma] fp32 (or NULL)
 * workspace: dspark_tv_label_workspace(...) bytes (B*gamma*(3 + ceil(V/64))
 *      fp32 words, each part 256-byte aligned).
 * ---------------------------------------------------------------------- */
size_t dspark_tv_label_workspace(int B, int gamma, int V, int rank, int dtype);
int dspark_tv_label(int B, int gamma, int V, int rank, int dtype,
                    const void* target, const void* U, const void* W1, const void* W2,
                    const int32_t* anchor, const int32_t* tokens,
                    const float* row_max, const float* row_logZ,
                    const float* temperature, float* tv, float* label,
                    int32_t* status, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Optional per-kernel timing (not on the sampling path).
 * dspark_trace_enable(1) clears earlier records and brackets every later
 * kernel launch by a pair of hipEvents on its stream; (0) stops recording.
 * dspark_trace_summary() waits for the recorded events and writes one line
 * "<kernel> <launches> <total_ms>" per kernel into buf (NUL-terminated,
 * truncated to len); returns the full text length or a negative status.
 * Tracing adds event records between launches: time the step without it.
 * ---------------------------------------------------------------------- */
int dspark_trace_enable(int on);
int dspark_trace_summary(char* buf, size_t len);

/* ------------------------------------------------------------------------
 * Drafting implementation choice (process-wide; for tests and benchmarks).
 * The setting is one atomic word read by every later dspark_draft_block
 * call, from any host thread: the one exception to "keep no state".
 * 0 = automatic (default): for bf16 inputs, the pipelined single-launch
 *     kernel (request windows of 32 drafted while the previous windows'
 *     tokens are drawn by dedicated work-groups; one work-group per compute
 *     unit, launched on the stream's own queue, so its work-groups must find
 *     the compute units free: with other work running beside it on the
 *     device they start as units free up, and a wait that outlasts 0.2 s
 *     reports DSPARK_DEV_TIMEOUT), else the earlier single-launch kernel
 *     (cooperative launch), else one launch
 *     pair per position;
 * 1 = always one launch pair per position;
 * 2 = the earlier single-launch kernel only: dspark_draft_block returns
 *     DSPARK_EHIP where it cannot run;
 * 3, 4 = that kernel only, with 8 (one register-resident W2 tile each) or
 *     4 (two each) waves per work-group; 2 picks 8;
 * 5 = the pipelined kernel only (DSPARK_EHIP where it cannot run);
 * 6 = the pipelined kernel by a cooperative launch (every work-group
 *     resident whatever else the device runs; the launch goes through a
 *     queue of its own, about 20 us more per call).
 * Settings 1-4 return identical bits, and so do 5 and 6.  The pipelined kernel draws from the
 * same statistics with the group and tile masses summed in another order
 * (a token can differ only where the uniform lies within about 1e-6 of a
 * boundary of the inverse CDF; q and the row statistics differ in the last
 * bits).
 * Returns the previous setting, or DSPARK_EINVAL for another value.
 * ---------------------------------------------------------------------- */
int dspark_set_draft_path(int path);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
