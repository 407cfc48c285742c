/*
 * oracle.c -- plain fp64 CPU oracle for one DSpark draft-and-verify round.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it: only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, constant table or helper with the HIP library; the two meet
 * only through the seeded synthetic inputs handed to both.
 *
 * Every quantity is computed in IEEE double precision, in the order the
 * pages describe, with no blocking, fusion or reordering.  Inputs arrive as
 * float32 arrays (bf16 weights are exactly representable in float32) and are
 * widened to double element by element.
 *
 * Sources (page title -- section):
 *  [MG] "DSpark：DeepSeek 线上跑的投机解码，半自回归 + 置信度调度怎么做到的"
 *       (marsggbo.github.io) -- 3.2 Sequential Stage (Markov head and the
 *       sequential sampling loop), 4.1 (acceptance = 1 - TV), 4.3 Hardware-Aware
 *       Prefix Scheduler (survival products, B, tau, Theta, greedy with early stop).
 *  [CE] "DeepSeek DSpark explained" interactive page (share.concentrate1.com)
 *       -- section 03 (q_k = softmax(U_k + B_k), B_k = W1[x_{k-1}] W2),
 *       section 02 (first rejection truncates the suffix, bonus token when all
 *       drafts pass), section 04 (a_j, B, tau, Theta, SPS), section 05
 *       (alpha = min(1, p/q), residual r(v) = max(p-q,0)/sum max(p-q,0)).
 *  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *       Easy as 1, 2, 3", SC'11 -- the 10-round Philox block function.
 *
 * Readings of points the pages leave open (each one is also listed in the
 * design notes of the repository):
 *  - The draft sampler is Gumbel-max on z = (U_k + B_k)/T with Philox
 *    uniforms; the pages sample with a multinomial draw, which has the same
 *    distribution.  Temperature 0 means greedy: lowest index wins ties.
 *  - Philox counter: word0 = (stream << 24) | k, word1 = v >> 2 for the
 *    per-vocabulary streams (0: draft noise, 2: resample noise; 0 for the
 *    accept stream 1), word2 = request index, word3 = low 32 bits of the
 *    round id; key = (seed low 32, seed high 32).  Per-vocabulary streams
 *    take output word (v & 3), the accept stream word 0.
 *    Uniform: u = ((w >> 8) + 0.5) * 2^-24, never 0 or 1.
 *  - Every sampled draw (x_k ~ q_k; y ~ r or p_{ell+1}) is a two-level
 *    Gumbel-max: a Gumbel race over the logsumexp of 32-entry vocabulary
 *    tiles, then one over the entries of the winning tile.  The pages fix the
 *    distributions (q_k = softmax(U_k + B_k); r(v) = max(p - q, 0) / sum;
 *    p for the bonus), not the sampler; this one is exact and its decisions
 *    are argmaxes with margins.  Noise: tiles from stream 3 (draft) / 4
 *    (resample), entries from stream 0 / 2.  Entries of zero mass never win.
 *  - Accept iff u * q(x) < p(x).  S = 0 on a rejection (only possible through
 *    rounding) falls back to p_j.
 *  - ell_r drafts are verified; ell_r = 0 still emits one token drawn from p_1.
 *  - Scheduler candidates are ordered by (-a, r, j); improvement must be
 *    strict; SPS beyond the table is 0; candidates with a = 0 are dropped.
 *  - The confidence head's weight vector is [d + r] long, its first d
 *    entries multiplying h_k and the last r the gathered W1 row, the order
 *    of the concatenation; there is no bias term.  alpha_k for T = 0 places
 *    q_k's mass on the greedy draft x_k.
 *
 * parity pins: the Philox block function is pinned to published known-answer
 * vectors and to rocRAND's implementation; the sampling, verification and
 * scheduling functions are pinned to the pages' worked examples, closed forms
 * and brute force (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11)                                */
/* ------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t mul_a = 0xD2511F53u, mul_b = 0xCD9E8D57u; /* round multipliers */
    const uint32_t weyl_a = 0x9E3779B9u, weyl_b = 0xBB67AE85u; /* key schedule increments */
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { /* the key is bumped before every round but the first */
            k0 += weyl_a;
            k1 += weyl_b;
        }
        uint64_t pa = (uint64_t)mul_a * (uint64_t)x0;
        uint64_t pb = (uint64_t)mul_b * (uint64_t)x2;
        uint32_t pa_hi = (uint32_t)(pa >> 32), pa_lo = (uint32_t)pa;
        uint32_t pb_hi = (uint32_t)(pb >> 32), pb_lo = (uint32_t)pb;
        uint32_t n0 = pb_hi ^ x1 ^ k0;
        uint32_t n1 = pb_lo;
        uint32_t n2 = pa_hi ^ x3 ^ k1;
        uint32_t n3 = pa_lo;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

double orc_u01(uint32_t w)
{
    return ((double)(w >> 8) + 0.5) * (1.0 / 16777216.0);
}

/* One 32-bit random word of the round's streams.  v indexes a vocabulary
 * entry (streams 0, 2) or a 32-entry tile (streams 3, 4).
 * stream 0: Gumbel noise of entry v at draft position k;
 * stream 1: accept uniform at position k (v ignored);
 * stream 2: Gumbel noise of entry v of the resample / bonus draw at position j;
 * stream 3: Gumbel noise of tile v at draft position k;
 * stream 4: Gumbel noise of tile v of the resample / bonus draw at position j. */
uint32_t orc_random_word(uint64_t seed, uint64_t round_id, int stream, int k, int req, int v)
{
    uint32_t ctr[4], key[2], out[4];
    int per_vocab = (stream != 1);
    ctr[0] = ((uint32_t)stream << 24) | (uint32_t)k;
    ctr[1] = per_vocab ? ((uint32_t)v >> 2) : 0u;
    ctr[2] = (uint32_t)req;
    ctr[3] = (uint32_t)round_id;
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
    return per_vocab ? out[v & 3] : out[0];
}

/* Gumbel noise -log(-log u) of stream word w. */
static double orc_gumbel(uint32_t w)
{
    return -log(-log(orc_u01(w)));
}

/* ------------------------------------------------------------------ */
/* Shared pieces of the draft and verify halves                        */
/* ------------------------------------------------------------------ */

/* z(v) = (U_k(v) + B_k(v)) / T with B_k(v) = sum_i e[i] * W2[v][i], e the
 * head's row for position k: W1[x_{k-1}] for the Markov head ([MG] 3.2;
 * [CE] 03), the RNN head's e_k otherwise.  T = 0 leaves the raw logit. */
static void orc_logits(const float *Uk, const float *e, const float *W2,
                       double T, int V, int r, double *z)
{
    for (int v = 0; v < V; ++v) {
        const float *w = W2 + (size_t)v * (size_t)r;
        double bias = 0.0;
        for (int i = 0; i < r; ++i)
            bias += (double)e[i] * (double)w[i];
        double logit = (double)Uk[v] + bias;
        z[v] = (T > 0.0) ? logit / T : logit;
    }
}

/* The head's row for request b at position k: E[b][k-1] when the caller
 * passes the rows the head produced ([B, gamma, r], the RNN head), else the
 * Markov head's W1[x_{k-1}] with x_0 = anchor. */
static const float *orc_head_row(const float *W1, const float *E, const int32_t *anchor, const int32_t *x,
                                 int b, int k, int gamma, int r)
{
    if (E) return E + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)r;
    int prev = (k == 1) ? anchor[b] : x[(size_t)b * (size_t)gamma + (size_t)(k - 2)];
    return W1 + (size_t)prev * (size_t)r;
}

/* log sum_v exp(z(v)); -inf when no entry is finite. */
static double orc_logsumexp(const double *z, int V)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (z[v] > m) m = z[v];
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int v = 0; v < V; ++v)
        s += exp(z[v] - m);
    return m + log(s);
}

/* Index of the largest entry (lowest index among equals) and the gap to the
 * runner-up (+inf when V == 1). */
static int orc_argmax(const double *z, int V, double *gap)
{
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (z[v] > z[best]) best = v;
    double second = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (v != best && z[v] > second) second = z[v];
    if (gap) *gap = z[best] - second;
    return best;
}

#define ORC_TILE 32 /* vocabulary entries per tile of the two-level draw */

/* Two-level Gumbel-max draw over log-masses s(v) (-inf: excluded):
 * level 1 picks the tile t = v / 32 maximising logsumexp_{v in t} s(v) + G_t
 * (noise from tile_stream at index t), level 2 the entry v of that tile
 * maximising s(v) + G_v (noise from entry_stream at index v); lowest index
 * wins ties.  P(v) = exp(s(v)) / sum exp(s): an exact draw.  *margin receives
 * the smaller of the two top-two score gaps (+inf where a level has one
 * candidate).  Returns 0 when no entry has finite log-mass. */
static int orc_two_level_draw(const double *s, int V, uint64_t seed, uint64_t round_id, int tile_stream,
                              int entry_stream, int k, int req, double *margin)
{
    int ntile = (V + ORC_TILE - 1) / ORC_TILE;
    int tbest = -1;
    double b1 = -INFINITY, s1 = -INFINITY;
    for (int t = 0; t < ntile; ++t) {
        int v0 = t * ORC_TILE, v1 = v0 + ORC_TILE < V ? v0 + ORC_TILE : V;
        double m = -INFINITY;
        for (int v = v0; v < v1; ++v)
            if (s[v] > m) m = s[v];
        if (m == -INFINITY) continue;
        double acc = 0.0;
        for (int v = v0; v < v1; ++v)
            acc += exp(s[v] - m);
        double score = m + log(acc) + orc_gumbel(orc_random_word(seed, round_id, tile_stream, k, req, t));
        if (tbest < 0 || score > b1) {
            s1 = b1;
            b1 = score;
            tbest = t;
        } else if (score > s1) {
            s1 = score;
        }
    }
    if (tbest < 0) {
        if (margin) *margin = 0.0;
        return 0;
    }
    int pick = -1;
    double b2 = -INFINITY, s2 = -INFINITY;
    int v0 = tbest * ORC_TILE, v1 = v0 + ORC_TILE < V ? v0 + ORC_TILE : V;
    for (int v = v0; v < v1; ++v) {
        if (s[v] == -INFINITY) continue;
        double score = s[v] + orc_gumbel(orc_random_word(seed, round_id, entry_stream, k, req, v));
        if (pick < 0 || score > b2) {
            s2 = b2;
            b2 = score;
            pick = v;
        } else if (score > s2) {
            s2 = score;
        }
    }
    if (margin) *margin = fmin(b1 - s1, b2 - s2);
    return pick;
}

/* ------------------------------------------------------------------ */
/* Draft half: the sequential Markov-head sampling loop                */
/* ------------------------------------------------------------------ */

/* For each request b and k = 1..gamma ([MG] 3.2, [CE] 03):
 *   z = (U_k + W1[x_{k-1}] W2^T) / T,  x_0 = anchor,
 *   lse = logsumexp(z),  q_k(v) = exp(z(v) - lse),
 *   T > 0: x_k = the two-level Gumbel-max draw from softmax(z) (tiles:
 *          stream 3, entries: stream 0), G = -log(-log u);
 *   T = 0: x_k = argmax_v z(v) (lowest index wins), q_k one-hot.
 * Outputs per (b, k): x, lse (the max logit for T = 0), q_k(x_k) (1 for
 * T = 0), and the smaller of the draw's two top-two score gaps (the top-two
 * logit gap for T = 0).
 * req_ids (nullable) gives the request index used in the Philox counter. */
int orc_draft(const float *U, const float *W1, const float *W2,
              const int32_t *anchor, const float *temperature, const int32_t *req_ids,
              int B, int gamma, int V, int r, uint64_t seed, uint64_t round_id,
              int32_t *x_out, double *lse_out, double *qx_out, double *margin_out)
{
    if (B < 0 || gamma < 1 || V < 1 || r < 1) return ORC_ERR_ARG;
    if (!U || !W1 || !W2 || !anchor || !temperature || !x_out) return ORC_ERR_ARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double *z = (double *)malloc((size_t)V * sizeof(double));
        if (!z) { status = ORC_ERR_ARG; continue; }
        int req = req_ids ? req_ids[b] : b;
        double T = (double)temperature[b];
        int prev = anchor[b];
        for (int k = 1; k <= gamma; ++k) {
            const float *Uk = U + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)V;
            orc_logits(Uk, W1 + (size_t)prev * (size_t)r, W2, T, V, r, z);
            int x;
            double lse, qx, margin;
            if (T > 0.0) {
                lse = orc_logsumexp(z, V);
                x = orc_two_level_draw(z, V, seed, round_id, 3, 0, k, req, &margin);
                qx = exp(z[x] - lse);
            } else {
                x = orc_argmax(z, V, &margin);
                lse = z[x];
                qx = 1.0;
            }
            size_t o = (size_t)b * (size_t)gamma + (size_t)(k - 1);
            x_out[o] = x;
            if (lse_out) lse_out[o] = lse;
            if (qx_out) qx_out[o] = qx;
            if (margin_out) margin_out[o] = margin;
            prev = x;
        }
        free(z);
    }
    return status;
}

/* ------------------------------------------------------------------ */
/* Draft half with the RNN head                                        */
/* ------------------------------------------------------------------ */

/* x rounded to the nearest bfloat16 value (8 significant bits), ties to
 * even, straight from double precision. */
double orc_bf16_round(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    const double tiny = ldexp(1.0, -126); /* below it bfloat16 steps by 2^-133 */
    if (fabs(x) < tiny) return ldexp(nearbyint(ldexp(x, 133)), -133);
    int e;
    double m = frexp(x, &e); /* |m| in [0.5, 1) */
    double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, r); /* past the largest bf16 */
    return r;
}

/* [MG] 3.2 RNN Head: a recurrent state s_k (s_0 = 0) carried across the
 * block positions.  For each request b and k = 1..gamma, with x_0 = anchor:
 *   z    = [s_{k-1}, W1[x_{k-1}], h_k]                     (2r + d entries)
 *   y    = Wgco z,  Wgco [3r, 2r + d] (nn.Linear weight layout),
 *          split as (gate, candidate, output), r entries each
 *   g    = sigmoid(y_gate),  s_k = g * s_{k-1} + (1 - g) * tanh(y_cand)
 *   e_k  = tanh(y_out),      B_k(v) = sum_i e_k[i] W2[v][i]
 *   z_k  = (U_k + B_k) / T,  x_k drawn exactly as orc_draft draws it.
 * Precision reading: the head's two products take bfloat16 operands, as
 * its weights are, so s_{k-1} and h_k enter the gate product rounded to
 * bfloat16 and e_k enters the W2 product rounded to bfloat16 (nearest, ties
 * to even); everything else is double.  Outputs as orc_draft's, plus the
 * final state s_gamma [B, r] and the rows e_k [B, gamma, r] the W2 product
 * used (both nullable; e_k is what verification needs to rebuild q_k). */
int orc_draft_rnn(const float *U, const float *W1, const float *W2, const float *Wgco, const float *h,
                  const int32_t *anchor, const float *temperature, const int32_t *req_ids,
                  int B, int gamma, int V, int r, int d, uint64_t seed, uint64_t round_id,
                  int32_t *x_out, double *lse_out, double *qx_out, double *margin_out, double *state_out,
                  double *e_out)
{
    if (B < 0 || gamma < 1 || V < 1 || r < 1 || d < 0) return ORC_ERR_ARG;
    if (!U || !W1 || !W2 || !Wgco || !anchor || !temperature || !x_out) return ORC_ERR_ARG;
    if (d > 0 && !h) return ORC_ERR_ARG;
    const int K = 2 * r + d;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double *z = (double *)malloc((size_t)V * sizeof(double));
        double *st = (double *)calloc((size_t)r, sizeof(double));
        double *in = (double *)malloc((size_t)K * sizeof(double));
        double *ek = (double *)malloc((size_t)r * sizeof(double));
        if (!z || !st || !in || !ek) { status = ORC_ERR_ARG; free(z); free(st); free(in); free(ek); continue; }
        int req = req_ids ? req_ids[b] : b;
        double T = (double)temperature[b];
        int prev = anchor[b];
        for (int k = 1; k <= gamma; ++k) {
            const float *hk = d > 0 ? h + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)d : NULL;
            for (int i = 0; i < r; ++i) in[i] = orc_bf16_round(st[i]);
            for (int i = 0; i < r; ++i) in[r + i] = (double)W1[(size_t)prev * (size_t)r + i];
            for (int i = 0; i < d; ++i) in[2 * r + i] = orc_bf16_round((double)hk[i]);
            for (int i = 0; i < r; ++i) {
                double yg = 0.0, yc = 0.0, yo = 0.0;
                const float *wg = Wgco + (size_t)i * (size_t)K;
                const float *wc = Wgco + (size_t)(r + i) * (size_t)K;
                const float *wo = Wgco + (size_t)(2 * r + i) * (size_t)K;
                for (int j = 0; j < K; ++j) {
                    yg += (double)wg[j] * in[j];
                    yc += (double)wc[j] * in[j];
                    yo += (double)wo[j] * in[j];
                }
                double g = 1.0 / (1.0 + exp(-yg));
                st[i] = g * st[i] + (1.0 - g) * tanh(yc);
                ek[i] = orc_bf16_round(tanh(yo));
            }
            if (e_out)
                for (int i = 0; i < r; ++i)
                    e_out[((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)r + i] = ek[i];
            const float *Uk = U + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)V;
            for (int v = 0; v < V; ++v) {
                const float *w = W2 + (size_t)v * (size_t)r;
                double bias = 0.0;
                for (int i = 0; i < r; ++i)
                    bias += ek[i] * (double)w[i];
                double logit = (double)Uk[v] + bias;
                z[v] = (T > 0.0) ? logit / T : logit;
            }
            int x;
            double lse, qx, margin;
            if (T > 0.0) {
                lse = orc_logsumexp(z, V);
                x = orc_two_level_draw(z, V, seed, round_id, 3, 0, k, req, &margin);
                qx = exp(z[x] - lse);
            } else {
                x = orc_argmax(z, V, &margin);
                lse = z[x];
                qx = 1.0;
            }
            size_t o = (size_t)b * (size_t)gamma + (size_t)(k - 1);
            x_out[o] = x;
            if (lse_out) lse_out[o] = lse;
            if (qx_out) qx_out[o] = qx;
            if (margin_out) margin_out[o] = margin;
            prev = x;
        }
        if (state_out)
            for (int i = 0; i < r; ++i) state_out[(size_t)b * (size_t)r + i] = st[i];
        free(z); free(st); free(in); free(ek);
    }
    return status;
}

/* ------------------------------------------------------------------ */
/* Verify half: exact rejection sampling with per-request lengths      */
/* ------------------------------------------------------------------ */

/* Target rows are packed: request b owns rows off_b .. off_b + ell_b, row
 * off_b + (k-1) holding the target logits for position k (k = ell_b + 1 is
 * the bonus row).  off (nullable) is the exclusive scan of (1 + ell).
 *
 * For each request ([CE] 02 and 05; [MG] 1 and 4.1):
 *   p_k = softmax(t_k / T) (T = 0: one-hot at the lowest-index argmax),
 *   q_k = softmax(z_k) recomputed from U_k, the head's row (W1[x_{k-1}], or
 *         E[b][k-1] when E is given) and W2 as in the draft;
 *   k = 1..ell: u from stream 1, accept iff u * q_k(x_k) < p_k(x_k)
 *               (T = 0: accept iff x_k = argmax t_k);
 *   first rejection j: y ~ max(p_j - q_j, 0) by the two-level Gumbel-max
 *               draw at position j (tiles: stream 4, entries: stream 2)
 *               (T = 0: y = argmax t_j);
 *   all accepted: y ~ p_{ell+1} the same way (the bonus token).
 * Outputs: n_accept[b], tokens[b][0..gamma] = x_1..x_n, y, then -1;
 * diag[b][k-1] = (p_k(x_k), min(1, p_k(x_k)/q_k(x_k))) for tested positions
 * (NaN elsewhere); resid_mass[b] = S at a sampled rejection (-1 otherwise);
 * accept_margin[b][k-1] = |u - p/q| (T > 0) or the top-two target gap
 * (T = 0) for tested positions (NaN elsewhere); pick_margin[b] = the
 * smaller top-two score gap of the two-level draw of y (T > 0) or the
 * top-two gap of t_j (T = 0). */
int orc_verify(const float *target, const int32_t *off, const int32_t *ell,
               const float *U, const float *W1, const float *W2, const float *E,
               const int32_t *anchor, const int32_t *x, const float *temperature,
               const int32_t *req_ids, int B, int gamma, int V, int r,
               uint64_t seed, uint64_t round_id,
               int32_t *n_accept, int32_t *tokens, double *diag, double *resid_mass,
               double *accept_margin, double *pick_margin)
{
    if (B < 0 || gamma < 1 || V < 1 || r < 1) return ORC_ERR_ARG;
    if (!target || !ell || !U || !W1 || !W2 || !anchor || !x || !temperature) return ORC_ERR_ARG;
    if (!n_accept || !tokens) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (ell[b] < 0 || ell[b] > gamma) return ORC_ERR_ARG;
    int64_t *row0 = (int64_t *)malloc((size_t)(B > 0 ? B : 1) * sizeof(int64_t));
    if (!row0) return ORC_ERR_ARG;
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        row0[b] = off ? (int64_t)off[b] : acc;
        acc += 1 + ell[b];
    }
    const double nan = NAN;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double *zq = (double *)malloc((size_t)V * sizeof(double));
        double *zt = (double *)malloc((size_t)V * sizeof(double));
        double *mass = (double *)malloc((size_t)V * sizeof(double));
        if (!zq || !zt || !mass) { status = ORC_ERR_ARG; free(zq); free(zt); free(mass); continue; }
        int req = req_ids ? req_ids[b] : b;
        double T = (double)temperature[b];
        int L = ell[b];
        const int32_t *xb = x + (size_t)b * (size_t)gamma;
        for (int k = 0; k < gamma; ++k) {
            if (diag) {
                diag[((size_t)b * (size_t)(gamma + 1) + k) * 2 + 0] = nan;
                diag[((size_t)b * (size_t)(gamma + 1) + k) * 2 + 1] = nan;
            }
            if (accept_margin) accept_margin[(size_t)b * (size_t)gamma + k] = nan;
        }
        if (diag) {
            diag[((size_t)b * (size_t)(gamma + 1) + gamma) * 2 + 0] = nan;
            diag[((size_t)b * (size_t)(gamma + 1) + gamma) * 2 + 1] = nan;
        }
        int n = 0;
        int rejected = 0;
        for (int k = 1; k <= L; ++k) {
            const float *tk = target + (size_t)(row0[b] + k - 1) * (size_t)V;
            int xk = xb[k - 1];
            int accept;
            double pk, ratio, margin;
            if (T > 0.0) {
                for (int v = 0; v < V; ++v) zt[v] = (double)tk[v] / T;
                double lse_t = orc_logsumexp(zt, V);
                pk = exp(zt[xk] - lse_t);
                const float *Uk = U + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)V;
                orc_logits(Uk, orc_head_row(W1, E, anchor, x, b, k, gamma, r), W2, T, V, r, zq);
                double lse_q = orc_logsumexp(zq, V);
                double qk = exp(zq[xk] - lse_q);
                double u = orc_u01(orc_random_word(seed, round_id, 1, k, req, 0));
                accept = (u * qk < pk);
                ratio = (qk > 0.0) ? fmin(1.0, pk / qk) : 1.0;
                margin = (qk > 0.0) ? fabs(u - pk / qk) : INFINITY;
            } else {
                for (int v = 0; v < V; ++v) zt[v] = (double)tk[v];
                int am = orc_argmax(zt, V, &margin);
                accept = (xk == am);
                pk = accept ? 1.0 : 0.0;
                ratio = pk;
            }
            if (diag) {
                diag[((size_t)b * (size_t)(gamma + 1) + (k - 1)) * 2 + 0] = pk;
                diag[((size_t)b * (size_t)(gamma + 1) + (k - 1)) * 2 + 1] = ratio;
            }
            if (accept_margin) accept_margin[(size_t)b * (size_t)gamma + (k - 1)] = margin;
            if (!accept) { rejected = 1; break; }
            n = k;
        }
        /* position of the emitted non-draft token */
        int j = n + 1;
        const float *tj = target + (size_t)(row0[b] + j - 1) * (size_t)V;
        int y;
        double pmargin = 0.0, S = -1.0;
        if (T > 0.0) {
            /* log-mass of the draw: log p_j, or log max(p_j - q_j, 0) after a rejection */
            for (int v = 0; v < V; ++v) zt[v] = (double)tj[v] / T;
            double lse_t = orc_logsumexp(zt, V);
            for (int v = 0; v < V; ++v) mass[v] = zt[v] - lse_t;
            if (rejected) {
                const float *Uj = U + ((size_t)b * (size_t)gamma + (size_t)(j - 1)) * (size_t)V;
                orc_logits(Uj, orc_head_row(W1, E, anchor, x, b, j, gamma, r), W2, T, V, r, zq);
                double lse_q = orc_logsumexp(zq, V);
                double tot = 0.0;
                for (int v = 0; v < V; ++v) {
                    double d = exp(zt[v] - lse_t) - exp(zq[v] - lse_q);
                    zq[v] = d > 0.0 ? log(d) : -INFINITY; /* residual log-mass, reusing the buffer */
                    tot += d > 0.0 ? d : 0.0;
                }
                S = tot;
                if (tot > 0.0)
                    memcpy(mass, zq, (size_t)V * sizeof(double));
                /* tot == 0: fall back to p_j, already in mass */
            }
            y = orc_two_level_draw(mass, V, seed, round_id, 4, 2, j, req, &pmargin);
        } else {
            for (int v = 0; v < V; ++v) zt[v] = (double)tj[v];
            y = orc_argmax(zt, V, &pmargin);
        }
        n_accept[b] = n;
        int32_t *tb = tokens + (size_t)b * (size_t)(gamma + 1);
        for (int i = 0; i <= gamma; ++i) tb[i] = -1;
        for (int i = 0; i < n; ++i) tb[i] = xb[i];
        tb[n] = y;
        if (resid_mass) resid_mass[b] = (T > 0.0 && rejected) ? S : -1.0;
        if (pick_margin) pick_margin[b] = pmargin;
        free(zq); free(zt); free(mass);
    }
    free(row0);
    return status;
}

/* ------------------------------------------------------------------ */
/* Confidence head and exact per-position acceptance                   */
/* ------------------------------------------------------------------ */

/* [MG] 4.1 (the confidence head): for each request b and position k, with
 * x_0 = anchor and the drafted prefix x,
 *   s_k = sum_{i<d} w[i] h[b][k][i] + sum_{i<r} w[d + i] W1[x_{k-1}][i]
 *         (a bias-free linear layer over the concatenation [h_k, W1[x_{k-1}]]),
 *   c_k = 1 / (1 + exp(-s_k)),
 * and ([MG] 4.2, [CE] 04) the prefix survival a_k = c_1 * ... * c_k.  With
 * tau (nullable, [gamma]) the head is the temperature-scaled one of [MG] 4.2:
 * c_k = 1 / (1 + exp(-s_k / tau_k)).
 * h is [B, gamma, d], w is [d + r]; outputs are [B, gamma]. */
int orc_confidence(const float *h, const float *w, const float *W1,
                   const int32_t *anchor, const int32_t *x, const float *tau,
                   int B, int gamma, int d, int r, double *c_out, double *a_out)
{
    if (B < 0 || gamma < 1 || d < 0 || r < 1) return ORC_ERR_ARG;
    if (!w || !W1 || !anchor || !x || !c_out) return ORC_ERR_ARG;
    if (d > 0 && !h) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        double a = 1.0;
        for (int k = 1; k <= gamma; ++k) {
            int prev = (k == 1) ? anchor[b] : x[(size_t)b * (size_t)gamma + (size_t)(k - 2)];
            const float *hk = h ? h + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)d : NULL;
            const float *e = W1 + (size_t)prev * (size_t)r;
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += (double)w[i] * (double)hk[i];
            for (int i = 0; i < r; ++i)
                s += (double)w[d + i] * (double)e[i];
            if (tau) s /= (double)tau[k - 1]; /* [MG] 4.2: the calibrated head */
            double c = 1.0 / (1.0 + exp(-s));
            a *= c;
            size_t o = (size_t)b * (size_t)gamma + (size_t)(k - 1);
            c_out[o] = c;
            if (a_out) a_out[o] = a;
        }
    }
    return ORC_OK;
}

/* [MG] 4.1 and [CE] 05: the probability that the draft at position k passes
 * the rejection test, before x_k is drawn, is
 *   alpha_k = sum_v min(p_k(v), q_k(v)) = 1 - TV(p_k, q_k),
 * with p_k = softmax(t_k / T) and q_k = softmax((U_k + W1[x_{k-1}] W2^T) / T)
 * on the drafted prefix (x_0 = anchor).  T = 0: both are one-hot, q_k at the
 * greedy draft x_k and p_k at the lowest-index argmax of t_k, so alpha_k is
 * 1 when they agree and 0 otherwise.  Computed for k = 1..ell_b (the rows
 * the target produced, packed as in orc_verify); NaN for k > ell_b. */
int orc_acceptance(const float *target, const int32_t *off, const int32_t *ell,
                   const float *U, const float *W1, const float *W2, const float *E,
                   const int32_t *anchor, const int32_t *x, const float *temperature,
                   int B, int gamma, int V, int r, double *alpha_out)
{
    if (B < 0 || gamma < 1 || V < 1 || r < 1) return ORC_ERR_ARG;
    if (!target || !ell || !U || !W1 || !W2 || !anchor || !x || !temperature || !alpha_out)
        return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (ell[b] < 0 || ell[b] > gamma) return ORC_ERR_ARG;
    int64_t *row0 = (int64_t *)malloc((size_t)(B > 0 ? B : 1) * sizeof(int64_t));
    if (!row0) return ORC_ERR_ARG;
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        row0[b] = off ? (int64_t)off[b] : acc;
        acc += 1 + ell[b];
    }
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double *zq = (double *)malloc((size_t)V * sizeof(double));
        double *zt = (double *)malloc((size_t)V * sizeof(double));
        if (!zq || !zt) { status = ORC_ERR_ARG; free(zq); free(zt); continue; }
        double T = (double)temperature[b];
        const int32_t *xb = x + (size_t)b * (size_t)gamma;
        for (int k = 1; k <= gamma; ++k) {
            double alpha = NAN;
            if (k <= ell[b]) {
                const float *tk = target + (size_t)(row0[b] + k - 1) * (size_t)V;
                if (T > 0.0) {
                    for (int v = 0; v < V; ++v) zt[v] = (double)tk[v] / T;
                    double lse_t = orc_logsumexp(zt, V);
                    const float *Uk = U + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)V;
                    orc_logits(Uk, orc_head_row(W1, E, anchor, x, b, k, gamma, r), W2, T, V, r, zq);
                    double lse_q = orc_logsumexp(zq, V);
                    alpha = 0.0;
                    for (int v = 0; v < V; ++v)
                        alpha += fmin(exp(zt[v] - lse_t), exp(zq[v] - lse_q));
                } else {
                    for (int v = 0; v < V; ++v) zt[v] = (double)tk[v];
                    alpha = (orc_argmax(zt, V, NULL) == xb[k - 1]) ? 1.0 : 0.0;
                }
            }
            alpha_out[(size_t)b * (size_t)gamma + (size_t)(k - 1)] = alpha;
        }
        free(zq); free(zt);
    }
    free(row0);
    return status;
}

/* ------------------------------------------------------------------ */
/* Sequential temperature scaling of the confidences                   */
/* ------------------------------------------------------------------ */

/* [MG] 4.2: calibrate the head's confidences position by position, left to
 * right, each with a one-dimensional grid search for the temperature that
 * minimises the expected calibration error of the prefix survival product,
 * the earlier positions' temperatures held fixed.  Readings:
 *  - temperature scaling acts on the logit: c' = sigmoid(logit(c) / tau), an
 *    order-preserving map for tau > 0;
 *  - the calibrated quantity at position k is a'_k = c'_1 ... c'_k and its
 *    outcome is y_k = [n >= k] (drafts 1..k all accepted), over the samples
 *    that verified position k (ell >= k);
 *  - ECE = sum over M equal-width bins of |sum_bin y - sum_bin a'| / N_k
 *    (the usual weighted gap between accuracy and confidence), a' in bin
 *    min(floor(a' M), M - 1);
 *  - the smallest-index grid value wins ties; grid values <= 0 never win;
 *    a position no sample verified keeps tau = 1 and ECE = NaN.
 * c [N, gamma], n [N], ell [N] (nullable: every sample verified gamma
 * positions).  Outputs tau [gamma], ece [gamma], ece_grid [gamma, G]
 * (nullable; +inf for grid values <= 0). */
int orc_sts_fit(const float *c, const int32_t *n, const int32_t *ell, int N, int gamma,
                const float *grid, int G, int M, double *tau_out, double *ece_out, double *ece_grid)
{
    if (N < 0 || gamma < 1 || G < 1 || M < 1 || !c || !n || !grid || !tau_out || !ece_out) return ORC_ERR_ARG;
    double *a = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    double *sp = (double *)malloc((size_t)M * sizeof(double));
    double *sy = (double *)malloc((size_t)M * sizeof(double));
    if (!a || !sp || !sy) { free(a); free(sp); free(sy); return ORC_ERR_ARG; }
    for (int i = 0; i < N; ++i) a[i] = 1.0;
    for (int k = 1; k <= gamma; ++k) {
        int Nk = 0;
        for (int i = 0; i < N; ++i) {
            int L = ell ? ell[i] : gamma;
            if (L >= k && L <= gamma) ++Nk;
        }
        double best = INFINITY, tau = 1.0;
        for (int g = 0; g < G; ++g) {
            double t = (double)grid[g];
            double e = INFINITY;
            if (t > 0.0 && Nk > 0) {
                for (int m = 0; m < M; ++m) sp[m] = sy[m] = 0.0;
                for (int i = 0; i < N; ++i) {
                    int L = ell ? ell[i] : gamma;
                    if (L < k || L > gamma) continue;
                    double ci = (double)c[(size_t)i * (size_t)gamma + (size_t)(k - 1)];
                    double lg = log(ci) - log1p(-ci);
                    double p = a[i] / (1.0 + exp(-lg / t));
                    int m = (int)floor(p * M);
                    if (m > M - 1) m = M - 1;
                    if (m < 0) m = 0;
                    sp[m] += p;
                    sy[m] += (n[i] >= k) ? 1.0 : 0.0;
                }
                e = 0.0;
                for (int m = 0; m < M; ++m) e += fabs(sy[m] - sp[m]);
                e /= (double)Nk;
            }
            if (ece_grid) ece_grid[(size_t)(k - 1) * (size_t)G + g] = e;
            if (e < best) {
                best = e;
                tau = t;
            }
        }
        if (Nk == 0 || best == INFINITY) {
            tau = 1.0;
            best = NAN;
        }
        tau_out[k - 1] = tau;
        ece_out[k - 1] = best;
        for (int i = 0; i < N; ++i) {
            double ci = (double)c[(size_t)i * (size_t)gamma + (size_t)(k - 1)];
            double lg = log(ci) - log1p(-ci);
            a[i] = a[i] / (1.0 + exp(-lg / tau));
        }
    }
    free(a); free(sp); free(sy);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Host scheduler: confidence-scheduled prefix lengths                 */
/* ------------------------------------------------------------------ */

typedef struct { double a; int r; int j; } orc_cand;

static int orc_cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *x = (const orc_cand *)pa, *y = (const orc_cand *)pb;
    if (x->a > y->a) return -1;
    if (x->a < y->a) return 1;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->j != y->j) return x->j < y->j ? -1 : 1;
    return 0;
}

static double orc_sps(const double *sps, int sps_len, int64_t B)
{
    return (B >= 0 && B < sps_len) ? sps[B] : 0.0;
}

/* [MG] 4.3 and [CE] 04: a_{r,j} = prod_{i<=j} c_{r,i}; start from ell = 0,
 * B = tau = R, best Theta = R * SPS(R); walk all (r, j) with a > 0 in
 * descending a (ties: lower r, then lower j), extend only when j equals the
 * current length of request r, B += 1, tau += a, Theta = tau * SPS(B); keep
 * the lengths while Theta strictly improves, stop at the first step that
 * does not improve.  j here is 0-based (position j+1). */
int orc_schedule(const double *c, int R, int gamma, const double *sps, int sps_len,
                 int32_t *ell_out, double *theta_out, double *tau_out, int32_t *B_out)
{
    if (R < 0 || gamma < 1 || !c || !sps || !ell_out) return ORC_ERR_ARG;
    if (sps_len <= R) return ORC_ERR_ARG;
    size_t ncand_max = (size_t)R * (size_t)gamma;
    orc_cand *cand = (orc_cand *)malloc((ncand_max ? ncand_max : 1) * sizeof(orc_cand));
    int32_t *len = (int32_t *)calloc((size_t)(R ? R : 1), sizeof(int32_t));
    if (!cand || !len) { free(cand); free(len); return ORC_ERR_ARG; }
    size_t n = 0;
    for (int r = 0; r < R; ++r) {
        double a = 1.0;
        for (int j = 0; j < gamma; ++j) {
            a *= c[(size_t)r * (size_t)gamma + j];
            if (a > 0.0) {
                cand[n].a = a; cand[n].r = r; cand[n].j = j;
                ++n;
            }
        }
    }
    qsort(cand, n, sizeof(orc_cand), orc_cand_cmp);
    int64_t B = R;
    double tau = (double)R;
    double best_theta = tau * orc_sps(sps, sps_len, B);
    double best_tau = tau;
    int64_t best_B = B;
    size_t taken = 0; /* candidates consumed at the best point */
    size_t walked = 0;
    for (size_t i = 0; i < n; ++i) {
        const orc_cand *cd = &cand[i];
        if (cd->j != len[cd->r]) continue;
        len[cd->r] += 1;
        B += 1;
        tau += cd->a;
        ++walked;
        double theta = tau * orc_sps(sps, sps_len, B);
        if (theta > best_theta) {
            best_theta = theta;
            best_tau = tau;
            best_B = B;
            taken = walked;
        } else {
            break;
        }
    }
    /* the best lengths are those after the first `taken` extensions */
    memset(len, 0, (size_t)(R ? R : 1) * sizeof(int32_t));
    size_t used = 0;
    for (size_t i = 0; i < n && used < taken; ++i) {
        const orc_cand *cd = &cand[i];
        if (cd->j != len[cd->r]) continue;
        len[cd->r] += 1;
        ++used;
    }
    for (int r = 0; r < R; ++r) ell_out[r] = len[r];
    if (theta_out) *theta_out = best_theta;
    if (tau_out) *tau_out = best_tau;
    if (B_out) *B_out = (int32_t)best_B;
    free(cand);
    free(len);
    return ORC_OK;
}

/* [CE] 04 (the paragraph on the strict implementation): the synchronous
 * scheduler above stops early on the current step's own Theta; the
 * production scheme fixes the step's capacity from the previous two steps'
 * predictions and only sorts the current candidates, which suits an
 * asynchronous pipeline and a cost curve that is not smooth.  Readings:
 *  - capacity_t = round(R_t * mean over the previous two steps of B / R),
 *    B the synchronous scheduler's choice for that step (its predictions),
 *    steps with R = 0 skipped, rounding half up, clamped to [R_t,
 *    R_t (1 + gamma)]; with no history, R_t (1 + gamma) (verify everything);
 *  - the current candidates, in the synchronous order (-a, r, j), each extend
 *    their request when they are its next position, until B = capacity; no
 *    early stop; candidates with a = 0 are dropped.
 * orc_history_capacity returns the capacity; orc_schedule_capacity the
 * lengths, tau and B for a given capacity. */
int64_t orc_history_capacity(const int32_t *B_hist, const int32_t *R_hist, int n_hist, int R, int gamma)
{
    double sum = 0.0;
    int used = 0;
    for (int i = 0; i < n_hist && i < 2; ++i) {
        if (R_hist[i] <= 0) continue;
        sum += (double)B_hist[i] / (double)R_hist[i];
        ++used;
    }
    int64_t hi = (int64_t)R * (int64_t)(1 + gamma);
    if (used == 0) return hi;
    int64_t cap = (int64_t)floor((double)R * (sum / used) + 0.5);
    if (cap < R) cap = R;
    if (cap > hi) cap = hi;
    return cap;
}

int orc_schedule_capacity(const double *c, int R, int gamma, int64_t capacity,
                          int32_t *ell_out, double *tau_out, int32_t *B_out)
{
    if (R < 0 || gamma < 1 || (R > 0 && (!c || !ell_out))) return ORC_ERR_ARG;
    size_t ncand_max = (size_t)R * (size_t)gamma;
    orc_cand *cand = (orc_cand *)malloc((ncand_max ? ncand_max : 1) * sizeof(orc_cand));
    int32_t *len = (int32_t *)calloc((size_t)(R ? R : 1), sizeof(int32_t));
    if (!cand || !len) { free(cand); free(len); return ORC_ERR_ARG; }
    size_t n = 0;
    for (int r = 0; r < R; ++r) {
        double a = 1.0;
        for (int j = 0; j < gamma; ++j) {
            a *= c[(size_t)r * (size_t)gamma + j];
            if (a > 0.0) {
                cand[n].a = a; cand[n].r = r; cand[n].j = j;
                ++n;
            }
        }
    }
    qsort(cand, n, sizeof(orc_cand), orc_cand_cmp);
    int64_t B = R;
    double tau = (double)R;
    for (size_t i = 0; i < n && B < capacity; ++i) {
        const orc_cand *cd = &cand[i];
        if (cd->j != len[cd->r]) continue;
        len[cd->r] += 1;
        B += 1;
        tau += cd->a;
    }
    for (int r = 0; r < R; ++r) ell_out[r] = len[r];
    if (tau_out) *tau_out = tau;
    if (B_out) *B_out = (int32_t)B;
    free(cand);
    free(len);
    return ORC_OK;
}
