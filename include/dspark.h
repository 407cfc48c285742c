/*
 * dspark.h -- C ABI of the MI355X (gfx950) library for one DSpark
 * draft-and-verify round over vocabulary-sized logits.
 *
 * Sources (page title -- section):
 *  [MG] "DSpark：DeepSeek 线上跑的投机解码，半自回归 + 置信度调度怎么做到的"
 *       (marsggbo.github.io): 3.2 Sequential Stage -- Markov head
 *       B_k = W2(W1[x_{k-1}]), the RNN head, and the left-to-right sampling
 *       loop;
 *       4.1 Confidence Head -- c_k from [h_k, W1[x_{k-1}]], acceptance
 *       probability 1 - TV; 4.2 -- survival products;
 *       4.3 Hardware-Aware Prefix Scheduler -- a_{r,j}, B, tau, Theta, greedy
 *       extension in descending a with early stop.
 *  [CE] "DeepSeek DSpark explained" (share.concentrate1.com): section 02 --
 *       the first rejection truncates the suffix, a bonus token follows when
 *       every draft passes; section 03 -- q_k = softmax(U_k + B_k); section
 *       04 -- a_j, tau, Theta = tau * SPS(B); section 05 -- accept with
 *       min(1, p/q), resample from max(p - q, 0) normalised.
 *
 * Conventions shared by every entry point:
 *  - Arrays are row-major and densely packed.  "device" pointers are HIP
 *    device memory (or memory the device can read at full speed); "host"
 *    pointers are ordinary CPU memory.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory: scratch space is the caller's `workspace`, sized by the
 *    matching *_workspace_size query.  Workspace contents need no
 *    initialisation and are not meaningful between calls, except that
 *    dspark_verify_check reads the status the last dspark_verify left there.
 *    The one exception is dspark_draft_sample_noalloc, which takes no
 *    workspace and uses a fixed array the library holds on each device.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device entry
 *    points only enqueue work on it and return; results are ready when the
 *    stream is.  Two calls that share a workspace must be ordered on one
 *    stream.  dspark_schedule is synchronous host code.
 *  - Every entry point returns a dspark_status.  Arguments are validated on
 *    the host before anything is enqueued; on an error nothing is enqueued
 *    and no output is written.
 *  - Random numbers come from Philox4x32-10 (Salmon et al., SC'11), keyed by
 *    `seed` and addressed by the counter (stream << 24 | position, i >> 2 or
 *    0, request index, low 32 bits of round_id), output word i & 3, where i
 *    is a vocabulary entry (streams 0 and 2) or a 32-entry vocabulary tile
 *    (streams 3 and 4).  Streams: 0 = draft entry noise, 1 = accept uniforms
 *    (word 0 of counter word1 = 0), 2 = resample / bonus entry noise, 3 =
 *    draft tile noise, 4 = resample / bonus tile noise.  Uniforms are
 *    ((w >> 8) + 0.5) * 2^-24, Gumbel noise -ln(-ln u).  Every sampled draw is
 *    a two-level Gumbel-max: tile t = v / 32 wins the race of
 *    logsumexp_{v in t} log-mass + tile noise, then entry v of that tile wins
 *    log-mass(v) + entry noise -- an exact draw from the normalised mass.
 *    Outputs are a pure function of the inputs, seed and round_id: two
 *    identical calls give identical bits.
 *  - Logits may be -inf (probability 0).  NaN inputs give undefined values
 *    but never out-of-bounds accesses or hangs.
 */
#ifndef DSPARK_H_
#define DSPARK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_ERR_ARG = -1,          /* null required pointer or size out of range */
    DSPARK_ERR_UNSUPPORTED = -2,  /* valid arguments this build has no kernel for */
    DSPARK_ERR_WORKSPACE = -3,    /* workspace missing or smaller than queried */
    DSPARK_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
    DSPARK_ERR_DEVICE_INPUT = -5, /* device-resident input failed its check */
    DSPARK_ERR_SCRATCH = -6       /* sizes need more than the allocation-free entry point's fixed scratch */
} dspark_status;

/* Element type of the Markov factors W1 and W2. */
typedef enum dspark_dtype {
    DSPARK_BF16 = 0, /* bfloat16 bit patterns (uint16_t) */
    DSPARK_F32 = 1   /* IEEE float32 */
} dspark_dtype;

/* Size limits checked by every entry point. */
#define DSPARK_MAX_GAMMA 32
#define DSPARK_MAX_BATCH 65536
#define DSPARK_MAX_VOCAB 16777215
#define DSPARK_MAX_HIDDEN 65536 /* d of the confidence head */
#define DSPARK_MAX_STS_SAMPLES (1 << 28) /* samples of one calibration fit */
#define DSPARK_MAX_STS_CELLS 4096        /* grid values x bins of one fit */
#define DSPARK_MAX_STS_GRID 1024         /* grid values of one fit */

/* Library version, major * 10000 + minor * 100 + patch. */
int dspark_version(void);

/* Static text for a dspark_status value (never NULL). */
const char *dspark_status_string(int status);

/* ------------------------------------------------------------------ */
/* Draft half ([MG] 3.2; [CE] 03)                                      */
/* ------------------------------------------------------------------ */

/* Bytes of device workspace dspark_draft_sample needs for these sizes;
 * 0 when the sizes are invalid. */
size_t dspark_draft_workspace_size(int B, int gamma, int V, int r);

/* Markov-head draft sampling for B requests over block positions k = 1..gamma.
 * For every request b and k, with x_0 = anchor[b]:
 *   z_k = (U[b, k-1, :] + W1[x_{k-1}, :] . W2^T) / T_b
 *   T_b > 0: x_k = the two-level Gumbel-max draw from q_k = softmax(z_k)
 *            (tile noise stream 3, entry noise stream 0, position k);
 *   T_b = 0: x_k = argmax_v z_k(v), lowest index first among equal values.
 * The [B, V] bias W1[x_{k-1}] W2^T is never written to memory.
 *
 *   U           device [B, gamma, V] float32   base logits U_k of the parallel stage
 *   W1, W2      device [V, r] of `wdtype`      Markov factors (W1: embedding rows,
 *                                              W2: output projection rows)
 *   anchor      device [B] int32 in [0, V)     x_0 of each request
 *   temperature device [B] float32 >= 0        T_b (0 = greedy)
 *   B in [1, DSPARK_MAX_BATCH], gamma in [1, DSPARK_MAX_GAMMA],
 *   V in [1, DSPARK_MAX_VOCAB], r in {16, 32, 64, 128, 256} (bf16) or
 *   {16, 32, 64, 128} (f32), otherwise DSPARK_ERR_UNSUPPORTED.
 *   seed, round_id                             Philox key and round counter
 *   x_out       device [B, gamma] int32        sampled drafts x_1..x_gamma
 *   lse_out     device [B, gamma] float32      logsumexp(z_k), so q_k = exp(z_k - lse);
 *                                              for T_b = 0 the largest logit
 *   qx_out      device [B, gamma] float32      q_k(x_k) (1 for T_b = 0)
 *   margin_out  device [B, gamma] float32 or NULL   the smaller of the draw's two
 *                                              top-two score gaps (tile race and
 *                                              entry race; logits for T_b = 0)
 *   workspace   device, >= dspark_draft_workspace_size bytes
 * Anchors outside [0, V) are clamped into range on the device. */
int dspark_draft_sample(const float *U, const void *W1, const void *W2, int wdtype,
                        const int32_t *anchor, const float *temperature,
                        int B, int gamma, int V, int r,
                        uint64_t seed, uint64_t round_id,
                        int32_t *x_out, float *lse_out, float *qx_out, float *margin_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the fixed device array dspark_draft_sample_noalloc draws its
 * scratch from (one array on each device the library runs on, held until the
 * process ends). */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* dspark_draft_sample for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: its scratch is a fixed array of
 * DSPARK_NOALLOC_SCRATCH_BYTES in the library, one per device, whose address
 * is resolved once per device on the first call made with that device
 * current.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine; with per-kernel profiling off, no host
 * allocation either).  Outputs are the bits dspark_draft_sample writes for the
 * same inputs.
 *
 *   every argument: as for dspark_draft_sample, without the workspace; the
 *   device current at the call must be the one that holds the buffers and
 *   owns `stream`.
 * Returns DSPARK_ERR_SCRATCH when dspark_draft_workspace_size(B, gamma, V, r)
 * exceeds DSPARK_NOALLOC_SCRATCH_BYTES (B above 13,696 at V = 129,280,
 * r = 256), DSPARK_ERR_HIP when the array's address cannot be resolved, and
 * otherwise the errors of dspark_draft_sample.
 * Every call on one device shares that device's array and leaves it in an
 * arbitrary state; nothing in it needs clearing before a call.  Calls that
 * overlap on one device (on different streams, or from threads that do not
 * order their streams) race on the array and give undefined outputs. */
int dspark_draft_sample_noalloc(const float *U, const void *W1, const void *W2, int wdtype,
                                const int32_t *anchor, const float *temperature, int B, int gamma, int V,
                                int r, uint64_t seed, uint64_t round_id, int32_t *x_out, float *lse_out,
                                float *qx_out, float *margin_out, void *stream);

/* dspark_draft_sample plus the confidence head of every position ([MG] 4.1
 * Confidence Head; [MG] 4.2 and [CE] 04 for the survival products): with
 * x_0 = anchor and the drafts this call samples,
 *   c_k = 1 / (1 + exp(-(w[0..d) . h_k + w[d..d+r) . W1[x_{k-1}]) / tau_k))
 * -- a bias-free linear layer over the concatenation [h_k, W1[x_{k-1}]] and
 * a sigmoid -- and a_k = c_1 * ... * c_k, the estimated probability that
 * drafts 1..k all survive verification.  The sampling outputs are the same
 * bits dspark_draft_sample writes for the same inputs.
 *
 *   hidden        device [B, gamma, d] float32: h_k of request b at row
 *                 b * gamma + k - 1 (may be NULL when d = 0)
 *   conf_w        device [d + r] float32: the head's weights, the h_k part
 *                 first
 *   d             0 .. DSPARK_MAX_HIDDEN
 *   conf_tau      device [gamma] float32 or NULL: the head's per-position
 *                 temperatures tau_k (those dspark_sts_fit chooses; NULL = 1)
 *   conf_out      device [B, gamma] float32: c_k
 *   survival_out  device [B, gamma] float32: a_k
 *   every other argument: as for dspark_draft_sample (same workspace size).
 * Rows of hidden and conf_w that are 16-byte aligned with d a multiple of 4
 * are read as float4. */
int dspark_draft_sample_confidence(const float *U, const void *W1, const void *W2, int wdtype,
                                   const int32_t *anchor, const float *temperature,
                                   int B, int gamma, int V, int r,
                                   uint64_t seed, uint64_t round_id,
                                   const float *hidden, const float *conf_w, int d, const float *conf_tau,
                                   int32_t *x_out, float *lse_out, float *qx_out, float *margin_out,
                                   float *conf_out, float *survival_out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace dspark_draft_sample_rnn needs; 0 for invalid
 * sizes.  Besides the draft step's partials and the two states it holds,
 * when d >= 4r and gamma >= 2, the h part of every position's gate product,
 * Wgco[:, 2r:] h_k, computed for the whole block before position 1 (float32
 * split-K partials, at most 512 MiB; otherwise the per-position product
 * covers h itself and the space is not taken). */
size_t dspark_draft_rnn_workspace_size(int B, int gamma, int V, int r, int d);

/* Draft sampling with the RNN head ([MG] 3.2, RNN Head) in place of the
 * Markov head: a recurrent state s_k over the block, s_0 = 0.  For every
 * request b and k = 1..gamma, with x_0 = anchor[b]:
 *   z   = [s_{k-1}, W1[x_{k-1}], h_k]                       (2r + d entries)
 *   g   = sigmoid(Wgco[0:r] z),  c = tanh(Wgco[r:2r] z),  o = Wgco[2r:3r] z
 *   s_k = g * s_{k-1} + (1 - g) * c,   e_k = tanh(o)
 *   z_k = (U[b, k-1, :] + e_k . W2^T) / T_b, and x_k drawn from it exactly as
 *   dspark_draft_sample draws (same streams, same outputs).
 * The head's products take bfloat16 operands: s_{k-1} and h_k are rounded to
 * bfloat16 (nearest, ties to even) where they enter the gate product, and e_k
 * is rounded to bfloat16 before the W2 product; s_k is kept in float32.
 *
 *   Wgco        device [3r, 2r + d] bfloat16 (nn.Linear weight layout: row j
 *               holds the weights of gate output j; rows 0..r-1 gate,
 *               r..2r-1 candidate, 2r..3r-1 output; columns in z's order)
 *   hidden      device [B, gamma, d] float32: h_k of request b at row
 *               b * gamma + k - 1 (may be NULL when d = 0); 16-byte aligned
 *   d           0 .. DSPARK_MAX_HIDDEN, a multiple of 32
 *   e_out       device [B, gamma, r] bfloat16, 16-byte aligned: the rows e_k
 *               the W2 product used -- what dspark_verify_rnn and
 *               dspark_acceptance_rnn need to rebuild q_k
 *   state_out   device [B, r] float32 or NULL: s_gamma
 *   workspace   device, >= dspark_draft_rnn_workspace_size bytes
 *   every other argument: as for dspark_draft_sample; wdtype must be
 *   DSPARK_BF16 (DSPARK_F32 returns DSPARK_ERR_UNSUPPORTED). */
int dspark_draft_sample_rnn(const float *U, const void *W1, const void *W2, const void *Wgco, int wdtype,
                            const int32_t *anchor, const float *temperature, const float *hidden, int d,
                            int B, int gamma, int V, int r, uint64_t seed, uint64_t round_id,
                            int32_t *x_out, float *lse_out, float *qx_out, float *margin_out,
                            void *e_out, float *state_out,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Sequential temperature scaling of the confidences ([MG] 4.2)        */
/* ------------------------------------------------------------------ */

/* Bytes of device workspace dspark_sts_fit needs; 0 for invalid sizes. */
size_t dspark_sts_workspace_size(int N, int gamma, int G, int n_bins);

/* Calibrates the confidence head from N observed rounds, left to right: for
 * k = 1..gamma, with the temperatures of positions < k fixed, tau_k is the
 * first grid value that minimises
 *   ECE_k(tau) = sum over n_bins equal-width bins of |sum y - sum a'| / N_k,
 *   a'_k = c'_1 ... c'_k,  c'_i = 1 / (1 + exp(-logit(c_i) / tau_i)),
 *   y_k = 1 if sample n accepted drafts 1..k (n_accept >= k), else 0,
 * over the N_k samples that verified position k (ell >= k); a' falls in bin
 * min(floor(a' n_bins), n_bins - 1).  Temperature scaling keeps the drafts'
 * order (tau > 0).  A position that no sample verified keeps tau_k = 1 and
 * gets ECE NaN; grid values <= 0 are never chosen.  The sums over samples
 * are exact integer sums (a' in 2^-32 fixed point), so results do not depend
 * on the order the GPU adds them in.
 *
 *   c            device [N, gamma] float32: the head's confidences (raw, tau = 1)
 *   n_accept     device [N] int32: accepted drafts of the sample's round
 *   ell          device [N] int32 or NULL (= gamma): verified positions
 *   grid         device [G] float32: candidate temperatures
 *   N            1 .. DSPARK_MAX_STS_SAMPLES
 *   G, n_bins    >= 1, G <= DSPARK_MAX_STS_GRID, G * n_bins <= DSPARK_MAX_STS_CELLS
 *   tau_out      device [gamma] float32 (feed it to the head's conf_tau)
 *   ece_out      device [gamma] float32: the ECE at the chosen tau_k
 *   ece_grid_out device [gamma, G] float32 or NULL: every grid value's ECE
 *                (+inf for grid values <= 0)
 *   workspace    device, >= dspark_sts_workspace_size bytes */
int dspark_sts_fit(const float *c, const int32_t *n_accept, const int32_t *ell, int N, int gamma,
                   const float *grid, int G, int n_bins, float *tau_out, float *ece_out,
                   float *ece_grid_out, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Verify half ([CE] 02, 05; [MG] 1, 4.1)                              */
/* ------------------------------------------------------------------ */

/* Bytes of device workspace dspark_verify needs; 0 for invalid sizes. */
size_t dspark_verify_workspace_size(int B, int gamma, int V, int r);

/* Exact rejection-sampling verification with per-request verify lengths.
 * Request b verifies its first ell[b] drafts against packed target rows
 * off_b .. off_b + ell[b] (row off_b + k - 1 = target logits for position
 * k; the last one feeds the bonus token).  With p_k = softmax(t_k / T_b)
 * and q_k the draft distribution recomputed from U, W1, W2 and lse_q:
 *   k = 1..ell[b]: accept x_k iff u_k * q_k(x_k) < p_k(x_k), u_k a Philox
 *                  uniform (T_b = 0: iff x_k = argmax t_k);
 *   first rejection j: y drawn from r = max(p_j - q_j, 0) / S, S = sum of
 *                  the residual (T_b = 0: y = argmax t_j); S = 0 falls back
 *                  to p_j;
 *   every draft accepted: y drawn from p_{ell+1} (the bonus token).
 * The draws are two-level Gumbel-max draws at position j (tile noise stream
 * 4, entry noise stream 2); entries of zero mass never win.
 * Request b emits n_b + 1 tokens: x_1..x_{n_b}, y.
 *
 *   target        device [n_target_rows, V] float32   packed target logits
 *   n_target_rows rows in `target`; a request whose rows fall outside it is
 *                 not verified (outputs -1, device status set)
 *   ell           device [B] int32 in [0, gamma]
 *   row_offsets   device [B + 1] int32 or NULL: off_b, the exclusive scan of
 *                 (1 + ell); NULL = computed on the device
 *   U, W1, W2, wdtype, temperature, B, gamma, V, r: as for dspark_draft_sample
 *   anchor, x     device [B] and [B, gamma] int32: x_0 and the drafts
 *   lse_q, qx     device [B, gamma] float32: lse_out and qx_out of the draft
 *   seed, round_id  same values as the draft call of this round
 *   n_accept_out  device [B] int32: n_b (-1 for a request that failed its check)
 *   tokens_out    device [B, gamma + 1] int32: x_1..x_n, y, then -1
 *   out_offsets   device [B + 1] int32 or NULL: exclusive scan of (n_b + 1)
 *   diag_out      device [B, gamma + 1, 2] float32 or NULL: for tested
 *                 positions (p_k(x_k), min(1, p_k(x_k) / q_k(x_k))), NaN elsewhere
 *   resid_out     device [B] float32 or NULL: residual mass S at a sampled
 *                 rejection, -1 otherwise
 *   workspace     device, >= dspark_verify_workspace_size bytes
 * Invalid ell / row_offsets values are device-resident, so they are found on
 * the device: the affected request outputs -1 and dspark_verify_check
 * reports DSPARK_ERR_DEVICE_INPUT. */
int dspark_verify(const float *target, int n_target_rows, const int32_t *ell,
                  const int32_t *row_offsets,
                  const float *U, const void *W1, const void *W2, int wdtype,
                  const int32_t *anchor, const int32_t *x, const float *lse_q, const float *qx,
                  const float *temperature, int B, int gamma, int V, int r,
                  uint64_t seed, uint64_t round_id,
                  int32_t *n_accept_out, int32_t *tokens_out, int32_t *out_offsets,
                  float *diag_out, float *resid_out,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Waits for `stream`, then returns DSPARK_OK or DSPARK_ERR_DEVICE_INPUT for
 * the device-side input checks of the last dspark_verify that used
 * `workspace` (DSPARK_ERR_HIP if the copy fails). */
int dspark_verify_check(const void *workspace, void *stream);

/* dspark_verify for drafts of the RNN head: q_k is rebuilt from the head's
 * rows e_k (head_rows, the e_out of dspark_draft_sample_rnn, [B, gamma, r]
 * of `wdtype`, 16-byte aligned) instead of W1[x_{k-1}].  Arguments, outputs,
 * workspace and device checks as for dspark_verify. */
int dspark_verify_rnn(const float *target, int n_target_rows, const int32_t *ell,
                      const int32_t *row_offsets,
                      const float *U, const void *head_rows, const void *W2, int wdtype,
                      const int32_t *anchor, const int32_t *x, const float *lse_q, const float *qx,
                      const float *temperature, int B, int gamma, int V, int r,
                      uint64_t seed, uint64_t round_id,
                      int32_t *n_accept_out, int32_t *tokens_out, int32_t *out_offsets,
                      float *diag_out, float *resid_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Per-position acceptance probability ([MG] 4.1; [CE] 05)             */
/* ------------------------------------------------------------------ */

/* Bytes of device workspace dspark_acceptance needs; 0 for invalid sizes. */
size_t dspark_acceptance_workspace_size(int B, int gamma, int V, int r);

/* The probability that draft k of request b passes the rejection test, taken
 * before x_k is drawn -- the confidence head's training label:
 *   alpha_k = sum_v min(p_k(v), q_k(v)) = 1 - TV(p_k, q_k),
 * with p_k = softmax(t_k / T_b) and q_k = softmax((U_k + W1[x_{k-1}] W2^T) / T_b)
 * recomputed from U, W1, W2 and lse_q on the drafted prefix (x_0 = anchor).
 * T_b = 0: alpha_k = 1 if x_k is the lowest-index argmax of t_k, else 0.
 * Every verified position k = 1..ell[b] is evaluated, also past the first
 * rejection (the target rows exist for the whole verified block).
 *
 *   target, n_target_rows, ell, row_offsets, U, W1, W2, wdtype, anchor, x,
 *   lse_q, temperature, B, gamma, V, r: as for dspark_verify (packed target
 *                 rows; row off_b + k - 1 holds position k)
 *   alpha_out     device [B, gamma] float32: alpha_k for k <= ell[b], NaN for
 *                 k > ell[b] and for every position of a request whose ell /
 *                 row_offsets fail the checks dspark_verify makes
 *   workspace     device, >= dspark_acceptance_workspace_size bytes
 * Cost: every verified row is read twice (its logsumexp, then the accepted
 * mass beside its U_k row and the W2 tiles), so this is a labelling pass, not
 * a step of the serving round. */
int dspark_acceptance(const float *target, int n_target_rows, const int32_t *ell,
                      const int32_t *row_offsets,
                      const float *U, const void *W1, const void *W2, int wdtype,
                      const int32_t *anchor, const int32_t *x, const float *lse_q,
                      const float *temperature, int B, int gamma, int V, int r,
                      float *alpha_out, void *workspace, size_t workspace_bytes, void *stream);

/* dspark_acceptance for drafts of the RNN head: q_k from head_rows as in
 * dspark_verify_rnn. */
int dspark_acceptance_rnn(const float *target, int n_target_rows, const int32_t *ell,
                          const int32_t *row_offsets,
                          const float *U, const void *head_rows, const void *W2, int wdtype,
                          const int32_t *anchor, const int32_t *x, const float *lse_q,
                          const float *temperature, int B, int gamma, int V, int r,
                          float *alpha_out, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Host scheduler ([MG] 4.3; [CE] 04)                                  */
/* ------------------------------------------------------------------ */

/* Confidence-scheduled prefix lengths.  Synchronous, host memory only.
 *   c         host [R, gamma] double in [0, 1]: calibrated confidences c_{r,j}
 *   sps       host [sps_len] double: SPS(B) for B = 0..sps_len-1; B beyond the
 *             table counts as 0.  sps_len must exceed R.
 *   ell_out   host [R] int32: chosen verify lengths
 *   theta_out, tau_out, B_out  (each may be NULL): Theta, tau and B of the choice
 * a_{r,j} = prod_{i<=j} c_{r,i}; starting from ell = 0 (B = tau = R), the
 * candidates with a > 0 are taken in descending a (ties: lower r, then lower
 * j); each extends its request by one (B += 1, tau += a) and is kept while
 * Theta = tau * SPS(B) strictly improves; the first step that does not
 * improve ends the search.  R = 0 is valid and returns Theta = 0. */
int dspark_schedule(const double *c, int R, int gamma, const double *sps, int sps_len,
                    int32_t *ell_out, double *theta_out, double *tau_out, int32_t *B_out);

/* Production-style scheduling ([CE] 04, the strict implementation: in an
 * asynchronous pipeline the step's capacity comes from the previous two
 * steps' predictions and the current candidates are only sorted into it).
 *
 * dspark_history_capacity: the capacity of the current step, R requests,
 *   round(R * mean_i B_hist[i] / R_hist[i]) over the first min(n_hist, 2)
 *   entries with R_hist[i] > 0 (the synchronous scheduler's B and R of the
 *   previous steps), rounding half up, clamped to [R, R (1 + gamma)];
 *   R (1 + gamma) (verify everything) when no entry is usable.  Host.
 * dspark_schedule_capacity: with c, R, gamma as for dspark_schedule, extends
 *   the requests in the same candidate order (-a, r, j) under the same
 *   prefix rule until B = capacity (or the candidates with a > 0 run out),
 *   without the early stop; ell_out [R], tau_out and B_out as for
 *   dspark_schedule.  With the capacity the synchronous scheduler chose it
 *   returns that scheduler's lengths; for any capacity its tau is the largest
 *   a prefix-valid choice of that B reaches.  Host, synchronous. */
int dspark_history_capacity(const int32_t *B_hist, const int32_t *R_hist, int n_hist, int R, int gamma,
                            int64_t *capacity_out);
int dspark_schedule_capacity(const double *c, int R, int gamma, int64_t capacity,
                             int32_t *ell_out, double *tau_out, int32_t *B_out);

/* ------------------------------------------------------------------ */
/* Diagnostics                                                         */
/* ------------------------------------------------------------------ */

/* Writes the library's 32-bit Philox words for indices v0 .. v0 + n - 1
 * (entries for streams 0 and 2, tiles for 3 and 4; ignored for stream 1) of
 * random stream `stream_id` in [0, 4] at position k of request `req` to
 * device [n] uint32 `out`. */
int dspark_debug_random_words(uint64_t seed, uint64_t round_id, int stream_id, int k, int req,
                              int v0, int n, uint32_t *out, void *stream);

/* Applies the library's device Gumbel transform to n device words:
 * out[i] = -log2(-log2(u_i)), u_i = ((w_i >> 8) + 0.5) * 2^-24. */
int dspark_debug_gumbel(const uint32_t *words, int n, float *out, void *stream);

/* The Markov-bias product alone, to measure the matrix-unit tiling of the
 * draft step ([MG] 3.2; [CE] 03: B_k = W1[x_{k-1}] W2^T) without the rest of
 * the step: rowmax_out[b] = max_v sum_i W1[idx[b]][i] * W2[v][i], computed
 * with the draft step's workgroups, LDS-staged W2 tiles and MFMA tiles, with
 * no U_k read and no sampling.
 *   W1, W2, wdtype, V, r  as for dspark_draft_sample
 *   idx         device [B] int32: the W1 rows (clamped into [0, V))
 *   rowmax_out  device [B] float32
 *   workspace   device, >= dspark_draft_workspace_size(B, 1, V, r) bytes
 * Same argument checks and error codes as dspark_draft_sample. */
int dspark_debug_bias_gemm(const void *W1, const void *W2, int wdtype, const int32_t *idx, int B, int V, int r,
                           float *rowmax_out, void *workspace, size_t workspace_bytes, void *stream);

/* Per-kernel timing with HIP events.  While enabled, every kernel the
 * library enqueues is launched with a start / stop event pair that the
 * dispatch itself stamps (hipExtLaunchKernel), so a duration is the kernel's
 * own execution time, without the launch gap; dspark_profile_collect waits
 * for the events and adds their durations to per-kernel totals.  Not for
 * concurrent use from several threads. */
int dspark_profile_enable(int enable);
int dspark_profile_collect(void);
/* Number of kernel names with totals, and the totals of entry i. */
int dspark_profile_count(void);
int dspark_profile_get(int i, const char **name, int64_t *launches, double *total_ms);
int dspark_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H_ */
