/*
 * oracle.c -- plain, slow, fp64 CPU reference for DSpark draft sampling and
 * lossless rejection-sampling verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under draft_sampling_lossless_head_amd/) shares no code with it:
 * no headers, helpers, tables or constant generators.
 *
 * Every step follows the pages' definitions in their own order, in double
 * precision, one request at a time, with plain loops (no blocking, no fusion,
 * no SIMD intrinsics; build without -ffast-math):
 *
 *   [P1] DSpark review (kimjy99.github.io, "[논문리뷰] DSpark ..."),
 *        §1.2 "Sequential stage": block factorisation and per-position softmax
 *        equation; Markov-head equation B(x_{k-1},.) = W1[x_{k-1}] W2;
 *        RNN-head equation (gated state update and W2^T tanh(W_o z_k)).
 *   [P2] VESSL AI blog "Speculative Decoding Part 1", section "알고리즘"
 *        (one speculative cycle: draft loop, ratio tests, first rejection,
 *        corrected or bonus token); section "수락 규칙" (acceptance rule,
 *        residual distribution, lossless theorem, closed form of alpha).
 *   [P1] also §2.1 "Confidence Head" (c_k = sigma(w^T [h_k; W1[x_{k-1}]]))
 *        and §2.2 "Hardware-Aware Prefix Scheduler" (survival products,
 *        B and tau, Theta = tau * SPS(B), global greedy order, early stop).
 *   [P2] also section "γ 재배분: 체인 대신 트리" (tree drafts: the top-n nodes by
 *        survival probability, ties to the shallower node).
 *   [PX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *        1, 2, 3", SC'11 -- Philox4x32 with 10 rounds.
 *
 * Readings where the pages leave a step open (all stated in the design notes):
 *   - sample(): inverse CDF over ascending token id with ONE uniform u in
 *     [0,1): the smallest v with u*Z < S_v (S_v = running sum of weights).
 *   - greedy (T == 0): argmax, lowest token id on ties.
 *   - ratio test: accept iff u * q(x) < p(x)  (the page's rejection test is
 *     u > p/q; the two differ only on a measure-zero set).
 *   - residual with zero mass after rounding: sample p_n instead (flagged).
 *   - position 1 conditions on the anchor x_0; the RNN concat order is
 *     [s_{k-1}; W1[x_{k-1}]; h_k]; the bias uses W_o z_k; s_0 = 0.
 *   - uniforms: Philox4x32-10, key = (seed lo, seed hi), counter =
 *     (request b, position k, stream, call offset); u = (word0 >> 8) * 2^-24.
 *     stream 0 = draft sample, 1 = ratio test, 2 = final (corrected/bonus),
 *     3 = tree verification (index v < M: node v's ratio test; index M: the
 *     final draw).
 *   - scheduler: survival a_{r,j} is the float32 product of c_{r,0..j} taken
 *     left to right; candidates are ordered by a descending, then request,
 *     then position; tau sums each a cut to a multiple of 2^-48 in exact
 *     integers; B = R + admitted; SPS(B) = 0 past the end of its table; the
 *     search stops at the first admission that lowers tau * SPS(B) (ties
 *     continue), and that admission is not made.
 *   - tree verification: siblings are tested in increasing index against a
 *     running residual r (p, then normalize(max(0, r - q)) after each
 *     failure); the first passing child is descended into; no pass: final
 *     token from r; a leaf: bonus from its p (see orc_verify_tree).
 *   - tree selection: nodes come parents first (parent[v] < v, -1 = a child
 *     of the root, the last accepted token); a_v = c_v * a_parent in float32
 *     (root 1); order a descending, then depth ascending, then node id; the
 *     score sums the chosen a cut to multiples of 2^-48, as the scheduler.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* [PX] Philox4x32-10.                                                       */
/* ------------------------------------------------------------------------ */

/* One Philox4x32 round: two 32x32->64 multiplies, the high halves xored
 * with the other two counter words and the round key, then a permutation. */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t out0 = hi1 ^ c[1] ^ k[0];
    uint32_t out1 = lo1;
    uint32_t out2 = hi0 ^ c[3] ^ k[1];
    uint32_t out3 = lo0;
    c[0] = out0; c[1] = out1; c[2] = out2; c[3] = out3;
}

/* Ten rounds; the key is bumped by the Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4], k[2];
    int i;
    for (i = 0; i < 4; i++) c[i] = ctr[i];
    k[0] = key[0];
    k[1] = key[1];
    for (i = 0; i < 10; i++) {
        philox_round(c, k);
        k[0] += 0x9E3779B9u;
        k[1] += 0xBB67AE85u;
    }
    for (i = 0; i < 4; i++) out[i] = c[i];
}

/* Uniform in [0,1) with 24 significant bits (exact in fp32). */
double orc_uniform(uint64_t seed, uint32_t offset, uint32_t b, uint32_t k, uint32_t stream)
{
    uint32_t ctr[4], key[2], out[4];
    ctr[0] = b;
    ctr[1] = k;
    ctr[2] = stream;
    ctr[3] = offset;
    key[0] = (uint32_t)(seed & 0xFFFFFFFFu);
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------ */
/* Softmax weights, inverse CDF, greedy choice.                              */
/* ------------------------------------------------------------------------ */

/* [P1] per-position softmax at temperature T > 0: w[v] = exp(l[v]/T - M)
 * with M = max_v l[v]/T; *Z = sum_v w[v] in ascending v.  Returns
 * log of the normaliser of exp(l/T), i.e. M + ln Z (or -inf if every logit
 * is -inf, in which case every weight is 0). */
double orc_softmax_weights(const double *l, int V, double T, double *w, double *Z)
{
    double M = -INFINITY, sum = 0.0;
    int v;
    for (v = 0; v < V; v++) {
        double t = l[v] / T;
        if (t > M) M = t;
    }
    if (M == -INFINITY) {
        for (v = 0; v < V; v++) w[v] = 0.0;
        *Z = 0.0;
        return -INFINITY;
    }
    for (v = 0; v < V; v++) {
        w[v] = exp(l[v] / T - M);
        sum += w[v];
    }
    *Z = sum;
    return M + log(sum);
}

/* Inverse CDF: thr = u * Z; returns the smallest v with thr < S_v where
 * S_v = w[0] + ... + w[v].  *thr_norm = thr / Z and *margin = distance of
 * thr to the nearer end of the chosen interval, divided by Z.  If rounding
 * leaves thr >= S_{V-1}, the last token with positive weight is returned
 * (margin 0).  Returns -1 when Z <= 0. */
int orc_inverse_cdf(const double *w, int V, double Z, double u, double *thr_norm, double *margin)
{
    double thr = u * Z, S = 0.0, prev;
    int v, last = -1;
    if (!(Z > 0.0)) {
        *thr_norm = 0.0;
        *margin = 0.0;
        return -1;
    }
    *thr_norm = u;
    for (v = 0; v < V; v++) {
        prev = S;
        S += w[v];
        if (w[v] > 0.0) last = v;
        if (thr < S) {
            double a = thr - prev, b = S - thr;
            *margin = (a < b ? a : b) / Z;
            return v;
        }
    }
    *margin = 0.0;
    return last;
}

/* Normalised CDF interval [lo, hi) of token y for weights w: lo = S_{y-1}/Z,
 * hi = S_y/Z, with S summed in ascending v as in orc_inverse_cdf.  Used by
 * the parity tests to decide whether a differing draw lies in the band
 * around a CDF boundary. */
void orc_cdf_interval(const double *w, int V, int y, double *lo, double *hi)
{
    double S = 0.0, Z = 0.0, below = 0.0;
    int v;
    for (v = 0; v < V; v++) {
        if (v == y) below = S;
        S += w[v];
    }
    Z = S;
    if (!(Z > 0.0) || y < 0 || y >= V) {
        *lo = NAN;
        *hi = NAN;
        return;
    }
    *lo = below / Z;
    *hi = (below + w[y]) / Z;
}

/* Greedy (T == 0): argmax with the lowest index on ties.  *gap = l[x] minus
 * the largest logit of any other token (0 on an exact tie). */
int orc_argmax(const double *l, int V, double *gap)
{
    int v, best = 0;
    double second = -INFINITY;
    for (v = 1; v < V; v++)
        if (l[v] > l[best]) best = v;
    for (v = 0; v < V; v++)
        if (v != best && l[v] > second) second = l[v];
    *gap = (V > 1) ? (l[best] - second) : INFINITY;
    return best;
}

/* One draw from softmax(l/T) (T > 0) or the greedy choice (T == 0).
 * Outputs: token, logZ (of l/T; max logit when T == 0), probability of the
 * token (1 when T == 0), normalised threshold and margin (top-2 gap when
 * T == 0).  w is scratch of length V. */
static int draw_from_logits(const double *l, int V, double T, double u, double *w,
                            double *logZ, double *tok_prob, double *thr_norm, double *margin)
{
    int tok;
    if (T == 0.0) {
        double gap;
        tok = orc_argmax(l, V, &gap);
        *logZ = l[tok];
        *tok_prob = 1.0;
        *thr_norm = 0.0;
        *margin = gap;
        return tok;
    } else {
        double Z;
        *logZ = orc_softmax_weights(l, V, T, w, &Z);
        tok = orc_inverse_cdf(w, V, Z, u, thr_norm, margin);
        *tok_prob = (tok >= 0) ? w[tok] / Z : 0.0;
        return tok;
    }
}

/* ------------------------------------------------------------------------ */
/* [P1] Sequential stage, Markov head.                                       */
/* ------------------------------------------------------------------------ */

/* One request.  U: [gamma, V] base logits; W1: [V, r]; W2: [r, V];
 * x0: anchor; u: [gamma] uniforms (unused when T == 0).  forced: NULL, or
 * [gamma] tokens that replace the oracle's own draw as the conditioning
 * token of the next position (replay of another sampler's prefix).
 * Outputs (each [gamma], q_logits [gamma, V] and may be NULL): tokens,
 * draft logits l = U + bias (before temperature), logZ, q(x_k),
 * normalised threshold and margin.  Returns 0, or -1 on a bad token id or
 * an all -inf row. */
int orc_draft_markov(int V, int gamma, int r,
                     const double *U, const double *W1, const double *W2,
                     int x0, double T, const double *u, const int *forced,
                     int *tokens, double *q_logits, double *logZ, double *q_tok,
                     double *thr_norm, double *margin)
{
    double *l = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *bias = (double *)malloc(sizeof(double) * (size_t)V);
    int k, j, v, status = 0;
    if (!l || !w || !bias) { free(l); free(w); free(bias); return -2; }
    for (k = 0; k < gamma; k++) {
        int prev;
        if (k == 0) prev = x0;
        else prev = forced ? forced[k - 1] : tokens[k - 1];
        if (prev < 0 || prev >= V) { status = -1; break; }
        /* bias(prev, v) = sum_j W1[prev, j] * W2[j, v], j ascending */
        for (v = 0; v < V; v++) bias[v] = 0.0;
        for (j = 0; j < r; j++) {
            double e = W1[(size_t)prev * r + j];
            const double *row = W2 + (size_t)j * V;
            for (v = 0; v < V; v++) bias[v] += e * row[v];
        }
        for (v = 0; v < V; v++) l[v] = U[(size_t)k * V + v] + bias[v];
        if (q_logits) memcpy(q_logits + (size_t)k * V, l, sizeof(double) * (size_t)V);
        tokens[k] = draw_from_logits(l, V, T, T == 0.0 ? 0.0 : u[k], w,
                                     &logZ[k], &q_tok[k], &thr_norm[k], &margin[k]);
        if (tokens[k] < 0) { status = -1; break; }
    }
    free(l); free(w); free(bias);
    return status;
}

/* ------------------------------------------------------------------------ */
/* [P1] Sequential stage, RNN head.                                          */
/* ------------------------------------------------------------------------ */

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* One request.  Adds h: [gamma, d] backbone hidden states and the gate
 * matrices Wg, Wc, Wo, each [r, 2r+d] row-major; everything else as in
 * orc_draft_markov.  Per position k (1-based on the page):
 *   z_k = [s_{k-1}; W1[x_{k-1}]; h_k]
 *   g = sigmoid(Wg z_k), c = tanh(Wc z_k), o = tanh(Wo z_k)
 *   s_k = g * s_{k-1} + (1 - g) * c
 *   bias_k = W2^T o      (bias_k[v] = sum_j W2[j, v] o[j])
 * with s_0 = 0 and no bias vectors in the projections. */
int orc_draft_rnn(int V, int gamma, int r, int d,
                  const double *U, const double *h, const double *W1, const double *W2,
                  const double *Wg, const double *Wc, const double *Wo,
                  int x0, double T, const double *u, const int *forced,
                  int *tokens, double *q_logits, double *logZ, double *q_tok,
                  double *thr_norm, double *margin)
{
    int n = 2 * r + d;
    double *l = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *bias = (double *)malloc(sizeof(double) * (size_t)V);
    double *s = (double *)calloc((size_t)r, sizeof(double));
    double *s_next = (double *)malloc(sizeof(double) * (size_t)r);
    double *o = (double *)malloc(sizeof(double) * (size_t)r);
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    int k, i, t, j, v, status = 0;
    if (!l || !w || !bias || !s || !s_next || !o || !z) {
        free(l); free(w); free(bias); free(s); free(s_next); free(o); free(z);
        return -2;
    }
    for (k = 0; k < gamma; k++) {
        int prev;
        if (k == 0) prev = x0;
        else prev = forced ? forced[k - 1] : tokens[k - 1];
        if (prev < 0 || prev >= V) { status = -1; break; }
        /* z_k = [s_{k-1}; W1[x_{k-1}]; h_k] */
        for (i = 0; i < r; i++) z[i] = s[i];
        for (i = 0; i < r; i++) z[r + i] = W1[(size_t)prev * r + i];
        for (i = 0; i < d; i++) z[2 * r + i] = h[(size_t)k * d + i];
        for (i = 0; i < r; i++) {
            double ag = 0.0, ac = 0.0, ao = 0.0, g, c;
            for (t = 0; t < n; t++) {
                ag += Wg[(size_t)i * n + t] * z[t];
                ac += Wc[(size_t)i * n + t] * z[t];
                ao += Wo[(size_t)i * n + t] * z[t];
            }
            g = sigmoid(ag);
            c = tanh(ac);
            o[i] = tanh(ao);
            s_next[i] = g * s[i] + (1.0 - g) * c;
        }
        for (i = 0; i < r; i++) s[i] = s_next[i];
        for (v = 0; v < V; v++) bias[v] = 0.0;
        for (j = 0; j < r; j++) {
            const double *row = W2 + (size_t)j * V;
            for (v = 0; v < V; v++) bias[v] += o[j] * row[v];
        }
        for (v = 0; v < V; v++) l[v] = U[(size_t)k * V + v] + bias[v];
        if (q_logits) memcpy(q_logits + (size_t)k * V, l, sizeof(double) * (size_t)V);
        tokens[k] = draw_from_logits(l, V, T, T == 0.0 ? 0.0 : u[k], w,
                                     &logZ[k], &q_tok[k], &thr_norm[k], &margin[k]);
        if (tokens[k] < 0) { status = -1; break; }
    }
    free(l); free(w); free(bias); free(s); free(s_next); free(o); free(z);
    return status;
}

/* ------------------------------------------------------------------------ */
/* [P2] Lossless verification.                                               */
/* ------------------------------------------------------------------------ */

/* Residual weights max(0, p - q) of two logit rows at temperature T > 0,
 * with p = exp(lp/T - logZp), q = exp(lq/T - logZq).  Returns their sum. */
double orc_residual_weights(const double *lp, const double *lq, int V, double T,
                            double logZp, double logZq, double *w)
{
    double R = 0.0;
    int v;
    for (v = 0; v < V; v++) {
        double pv = exp(lp[v] / T - logZp);
        double qv = exp(lq[v] / T - logZq);
        double d = pv - qv;
        w[v] = d > 0.0 ? d : 0.0;
        R += w[v];
    }
    return R;
}

/* One request with L drafted positions (0 <= L).  P: [L+1, V] target
 * logits, Q: [L, V] draft logits (before temperature), draft: [L] tokens,
 * u_test: [L] ratio-test uniforms, u_final: uniform of the final draw.
 * Outputs: *n_acc = number of accepted draft tokens n (first rejection, or
 * L); out: [L+1] emitted tokens (draft[0..n-1], then the corrected or
 * bonus token, then -1); logZp [L+1]; logZq [L]; accept_prob [L] =
 * min(1, p/q) at the draft token; test_margin [L] = |u - min(1, p/q)|
 * (T == 0: top-2 gap of the target row); *final_thr = u_final;
 * *final_margin = margin of the final draw; *fallback = 1 when the residual
 * had zero mass and p_n was sampled instead.  Returns 0, or -1 on bad
 * input (token out of range, all -inf row). */
int orc_verify(int V, int L, double T,
               const double *P, const double *Q, const int *draft,
               const double *u_test, double u_final,
               int *n_acc, int *out, double *logZp, double *logZq,
               double *accept_prob, double *test_margin,
               double *final_thr, double *final_margin, int *fallback)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    double Z, R;
    int k, n, tok, status = 0;
    if (!w) return -2;
    *fallback = 0;
    *final_thr = 0.0;
    *final_margin = 0.0;
    for (k = 0; k <= L; k++) out[k] = -1;
    for (k = 0; k < L; k++)
        if (draft[k] < 0 || draft[k] >= V) { free(w); return -1; }

    if (T == 0.0) {
        /* Greedy: the target's top-1 must equal the draft token. */
        for (k = 0; k <= L; k++) {
            double gap;
            int a = orc_argmax(P + (size_t)k * V, V, &gap);
            logZp[k] = P[(size_t)k * V + a];
            if (k < L) {
                double g2;
                int aq = orc_argmax(Q + (size_t)k * V, V, &g2);
                logZq[k] = Q[(size_t)k * V + aq];
                accept_prob[k] = (a == draft[k]) ? 1.0 : 0.0;
                test_margin[k] = gap;
            }
        }
        n = L;
        for (k = 0; k < L; k++)
            if (accept_prob[k] == 0.0) { n = k; break; }
        {
            double gap;
            tok = orc_argmax(P + (size_t)n * V, V, &gap);
            *final_margin = gap;
        }
    } else {
        /* Normalisers of every target row and every draft row. */
        for (k = 0; k <= L; k++) logZp[k] = orc_softmax_weights(P + (size_t)k * V, V, T, w, &Z);
        for (k = 0; k < L; k++) logZq[k] = orc_softmax_weights(Q + (size_t)k * V, V, T, w, &Z);
        for (k = 0; k <= L; k++) if (logZp[k] == -INFINITY) status = -1;
        for (k = 0; k < L; k++) if (logZq[k] == -INFINITY) status = -1;
        if (status) { free(w); return status; }
        /* Ratio test at every drafted position. */
        for (k = 0; k < L; k++) {
            int x = draft[k];
            double px = exp(P[(size_t)k * V + x] / T - logZp[k]);
            double qx = exp(Q[(size_t)k * V + x] / T - logZq[k]);
            double a = (qx > 0.0) ? (px / qx < 1.0 ? px / qx : 1.0) : (px > 0.0 ? 1.0 : 0.0);
            accept_prob[k] = a;
            test_margin[k] = fabs(u_test[k] - a);
        }
        /* First rejection: accept iff u * q(x) < p(x). */
        n = L;
        for (k = 0; k < L; k++) {
            int x = draft[k];
            double px = exp(P[(size_t)k * V + x] / T - logZp[k]);
            double qx = exp(Q[(size_t)k * V + x] / T - logZq[k]);
            if (!(u_test[k] * qx < px)) { n = k; break; }
        }
        if (n < L) {
            /* Corrected token from normalize(max(0, p_n - q_n)). */
            R = orc_residual_weights(P + (size_t)n * V, Q + (size_t)n * V, V, T,
                                     logZp[n], logZq[n], w);
            if (R > 0.0) {
                tok = orc_inverse_cdf(w, V, R, u_final, final_thr, final_margin);
            } else {
                *fallback = 1;
                orc_softmax_weights(P + (size_t)n * V, V, T, w, &Z);
                tok = orc_inverse_cdf(w, V, Z, u_final, final_thr, final_margin);
            }
        } else {
            /* Every draft token accepted: bonus token from p at slot L. */
            orc_softmax_weights(P + (size_t)L * V, V, T, w, &Z);
            tok = orc_inverse_cdf(w, V, Z, u_final, final_thr, final_margin);
        }
    }
    for (k = 0; k < n; k++) out[k] = draft[k];
    out[n] = tok;
    *n_acc = n;
    free(w);
    return status;
}

/* ------------------------------------------------------------------------ */
/* [P2] "γ 재배분: 체인 대신 트리": verification of a tree of draft             */
/* continuations in one target pass, under the acceptance rule of "수락 규칙". */
/* ------------------------------------------------------------------------ */

/* Nodes 0..M-1 come parents first (parent[v] < v; -1 = a child of the root,
 * the last accepted token).  Row 0 of P and Q belongs to the root and row
 * 1 + v to node v: the P row holds the target's next-token logits after the
 * path to that node; the Q row holds the draft logits its children were drawn
 * from (one independent draw per child).  tok[v] is node v's draft token.
 *
 * Reading (recursive rejection over siblings): the walk starts at the root
 * with target law r = p (softmax of the node's P row at T).  The node's
 * children are tested in increasing index; child c with token x passes iff
 * u_node[c] * q(x) < r(x) (q = softmax of the node's Q row).  A pass emits x
 * and moves the walk to c, with r = p of c.  A failure replaces r by
 * normalize(max(0, r - q)) and tests the next child.  When every child has
 * failed the final token is drawn from r by the inverse CDF with u_final; at
 * a node without children it is drawn from that node's p (bonus token).  If a
 * residual has no mass after rounding, the walk stops there and the final
 * token is drawn from that node's p (*fallback = 1).
 * T == 0: a child passes iff its token is the argmax of the node's P row
 * (lowest id on ties); the final token is that argmax.
 *
 * Outputs: *n_acc = number of accepted nodes; path[0..n-1] their ids (-1
 * after); out[0..n-1] their tokens, out[n] the final token (-1 after;
 * out has M + 1 entries); test_ratio[c] = r(x)/q(x) (capped at 1) of every
 * tested child c, NaN for children never tested; *final_thr, *final_margin
 * as orc_inverse_cdf (T == 0: the argmax's logit gap); final_w (V entries,
 * or NULL) receives the weights the final token was drawn from (T > 0).
 * Returns 0; -1 for an invalid tree (parent out of range), a token outside
 * [0, V) or a tested row without a finite logit (then n_acc = -1 and every
 * output -1). */
int orc_verify_tree(int V, int M, double T, const int *parent, const int *tok,
                    const double *P, const double *Q, const double *u_node, double u_final,
                    int *n_acc, int *path, int *out, double *test_ratio,
                    double *final_thr, double *final_margin, int *fallback, double *final_w)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    double *q = (double *)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    int v, c, node = -1, n = 0, final_tok = -1, bad = 0;
    if (!r || !q || !w) { free(r); free(q); free(w); return -2; }
    *fallback = 0;
    *final_thr = 0.0;
    *final_margin = 0.0;
    *n_acc = -1;
    for (v = 0; v <= M; v++) out[v] = -1;
    for (v = 0; v < M; v++) { path[v] = -1; test_ratio[v] = NAN; }
    for (v = 0; v < M; v++) {
        if (parent[v] < -1 || parent[v] >= v) bad = 1;
        if (tok[v] < 0 || tok[v] >= V) bad = 1;
    }
    if (bad) { free(r); free(q); free(w); return -1; }

    for (;;) {
        const double *pl = P + (size_t)(node + 1) * V;   /* the node's target row */
        const double *ql = Q + (size_t)(node + 1) * V;   /* its children's draft row */
        int accepted = -1, stop_fallback = 0;
        if (T == 0.0) {
            double gap;
            int a = orc_argmax(pl, V, &gap);
            if (pl[a] == -INFINITY) { bad = 1; break; }
            for (c = node + 1; c < M; c++) {
                if (parent[c] != node) continue;
                test_ratio[c] = (tok[c] == a) ? 1.0 : 0.0;
                if (tok[c] == a) { accepted = c; break; }
            }
            if (accepted < 0) { final_tok = a; *final_margin = gap; break; }
        } else {
            double Zp, Zq, Zr, lzp, lzq;
            int has_child = 0;
            lzp = orc_softmax_weights(pl, V, T, r, &Zp);
            if (lzp == -INFINITY) { bad = 1; break; }
            for (v = 0; v < V; v++) r[v] /= Zp;               /* r = p */
            for (c = node + 1; c < M; c++) if (parent[c] == node) has_child = 1;
            if (has_child) {
                lzq = orc_softmax_weights(ql, V, T, q, &Zq);
                if (lzq == -INFINITY) { bad = 1; break; }
                for (v = 0; v < V; v++) q[v] /= Zq;           /* q of the children */
            }
            for (c = node + 1; c < M && has_child; c++) {
                int x;
                double rx, qx;
                if (parent[c] != node) continue;
                x = tok[c];
                rx = r[x];
                qx = q[x];
                test_ratio[c] = qx > 0.0 ? (rx / qx < 1.0 ? rx / qx : 1.0) : (rx > 0.0 ? 1.0 : 0.0);
                if (u_node[c] * qx < rx) { accepted = c; break; }
                /* failure: r <- normalize(max(0, r - q)) */
                Zr = 0.0;
                for (v = 0; v < V; v++) {
                    double d = r[v] - q[v];
                    r[v] = d > 0.0 ? d : 0.0;
                    Zr += r[v];
                }
                if (!(Zr > 0.0)) { stop_fallback = 1; break; }
                for (v = 0; v < V; v++) r[v] /= Zr;
            }
            if (accepted < 0) {
                double Z;
                if (stop_fallback) {
                    *fallback = 1;
                    orc_softmax_weights(pl, V, T, w, &Z);
                    final_tok = orc_inverse_cdf(w, V, Z, u_final, final_thr, final_margin);
                } else {
                    Z = 0.0;
                    for (v = 0; v < V; v++) { w[v] = r[v]; Z += w[v]; }
                    final_tok = orc_inverse_cdf(w, V, Z, u_final, final_thr, final_margin);
                }
                if (final_w)
                    for (v = 0; v < V; v++) final_w[v] = w[v];
                break;
            }
        }
        path[n] = accepted;
        out[n] = tok[accepted];
        n++;
        node = accepted;
    }
    if (bad) {
        for (v = 0; v <= M; v++) out[v] = -1;
        for (v = 0; v < M; v++) path[v] = -1;
        free(r); free(q); free(w);
        return -1;
    }
    out[n] = final_tok;
    *n_acc = n;
    free(r); free(q); free(w);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [P1]/[P2] Diagnostics: acceptance rate and total variation.               */
/* ------------------------------------------------------------------------ */

/* alpha = sum_v min(p(v), q(v)) and D_TV = 1/2 sum_v |p(v) - q(v)| of one
 * target row and one draft row at temperature T > 0. */
void orc_alpha_tv(const double *lp, const double *lq, int V, double T, double *alpha, double *tv)
{
    double *wp = (double *)malloc(sizeof(double) * (size_t)V);
    double *wq = (double *)malloc(sizeof(double) * (size_t)V);
    double Zp, Zq, a = 0.0, t = 0.0;
    int v;
    if (!wp || !wq) { free(wp); free(wq); *alpha = NAN; *tv = NAN; return; }
    orc_softmax_weights(lp, V, T, wp, &Zp);
    orc_softmax_weights(lq, V, T, wq, &Zq);
    for (v = 0; v < V; v++) {
        double pv = wp[v] / Zp, qv = wq[v] / Zq;
        a += pv < qv ? pv : qv;
        t += fabs(pv - qv);
    }
    *alpha = a;
    *tv = 0.5 * t;
    free(wp);
    free(wq);
}

/* ------------------------------------------------------------------------ */
/* [P1] §2.1 Confidence head and §2.2 hardware-aware prefix scheduler.        */
/* ------------------------------------------------------------------------ */

/* c = sigma(w^T [h; e]) with h the backbone hidden state (d values) and e the
 * Markov embedding W1[x_{k-1}] (r values); w has d + r weights. */
double orc_confidence(const double *h, int d, const double *e, int r, const double *w)
{
    double z = 0.0;
    int i;
    for (i = 0; i < d; i++) z += w[i] * h[i];
    for (i = 0; i < r; i++) z += w[d + i] * e[i];
    return 1.0 / (1.0 + exp(-z));
}

/* One candidate prefix extension: request r, position j (0-based), survival
 * probability a_{r,j}. */
typedef struct { float a; int r, j; } orc_cand;

static int orc_cand_cmp(const void *x, const void *y)
{
    const orc_cand *p = (const orc_cand *)x, *q = (const orc_cand *)y;
    if (p->a != q->a) return p->a > q->a ? -1 : 1;   /* higher survival first */
    if (p->r != q->r) return p->r < q->r ? -1 : 1;
    return p->j < q->j ? -1 : (p->j > q->j);
}

/* Acceptance lengths l_r in {0..gamma} for R requests from their per-position
 * confidences c [R][gamma] (each in [0, 1]) and the engine's steps-per-second
 * table sps[B], B = 0 .. nsps - 1 (0 beyond it):
 *   a_{r,j} = prod_{i <= j} c_{r,i}                (fp32, left to right)
 *   candidates sorted by a descending (then request, then position), admitted
 *   one by one; after t admissions B_t = R + t and
 *   tau_t = R + sum of the admitted a (each a cut to a multiple of 2^-48 and
 *   summed exactly in integers), Theta_t = tau_t * SPS(B_t) in double;
 *   the search stops at the first t with Theta_t < Theta_{t-1} (that
 *   candidate is not admitted).
 * Fixing the precision of a (fp32 products) and of tau (exact integer sums)
 * makes the decisions independent of summation order.  Outputs l [R], the
 * chosen B and tau.  Returns 0, or -1 when memory runs out. */
int orc_prefix_schedule(const float *c, int R, int gamma, const double *sps, int nsps,
                        int *lens, double *B_out, double *tau_out)
{
    const int N = R * gamma;
    orc_cand *cand = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(N > 0 ? N : 1));
    const double scale = 281474976710656.0;   /* 2^48 */
    int64_t sum_q = 0;
    int r, j, t, admitted = 0;
    double theta_prev, tau;
    if (!cand) return -1;
    for (r = 0; r < R; r++) {
        float a = 1.0f;
        for (j = 0; j < gamma; j++) {
            a = a * c[(size_t)r * gamma + j];
            cand[r * gamma + j].a = a;
            cand[r * gamma + j].r = r;
            cand[r * gamma + j].j = j;
        }
    }
    qsort(cand, (size_t)N, sizeof(orc_cand), orc_cand_cmp);
    tau = (double)((int64_t)R * (int64_t)scale) / scale;
    theta_prev = tau * (R < nsps ? sps[R] : 0.0);
    for (t = 1; t <= N; t++) {
        const int64_t q = (int64_t)((double)cand[t - 1].a * scale);   /* exact, truncated */
        const int Bt = R + t;
        double tau_t, theta;
        sum_q += q;
        tau_t = (double)((int64_t)R * (int64_t)scale + sum_q) / scale;
        theta = tau_t * (Bt < nsps ? sps[Bt] : 0.0);
        if (theta < theta_prev) break;   /* throughput fell: stop before it */
        theta_prev = theta;
        tau = tau_t;
        admitted = t;
    }
    for (r = 0; r < R; r++) lens[r] = 0;
    for (t = 0; t < admitted; t++) lens[cand[t].r]++;
    *B_out = (double)(R + admitted);
    *tau_out = tau;
    free(cand);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* [P2] Tree drafts: top-n nodes by survival probability.                    */
/* ------------------------------------------------------------------------ */

typedef struct { float a; int depth, v; } orc_node;

static int orc_node_cmp(const void *x, const void *y)
{
    const orc_node *p = (const orc_node *)x, *q = (const orc_node *)y;
    if (p->a != q->a) return p->a > q->a ? -1 : 1;            /* higher survival first */
    if (p->depth != q->depth) return p->depth < q->depth ? -1 : 1;   /* then shallower */
    return p->v < q->v ? -1 : (p->v > q->v);
}

/* One tree of M candidate nodes: parent[v] in [-1, v) (-1: child of the
 * root), c[v] = chance that v is accepted once its parent is.  Survival
 * a_v = c_v * a_parent (root 1) in float32.  Writes the n nodes of highest
 * survival (ties: shallower, then lower id) to sel[0 .. n-1] in that order,
 * -1 past M, and their summed survival (each cut to a multiple of 2^-48,
 * summed exactly) to *score.  Returns 0; -1 for a parent outside [-1, v)
 * (sel all -1, score NaN) or when memory runs out. */
int orc_tree_select(const int *parent, const float *c, int M, int n, int *sel, double *score)
{
    orc_node *nd = (orc_node *)malloc(sizeof(orc_node) * (size_t)(M > 0 ? M : 1));
    float *a = (float *)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int *depth = (int *)malloc(sizeof(int) * (size_t)(M > 0 ? M : 1));
    const double scale = 281474976710656.0;   /* 2^48 */
    int64_t sum_q = 0;
    int v, i;
    if (!nd || !a || !depth) { free(nd); free(a); free(depth); return -1; }
    for (i = 0; i < n; i++) sel[i] = -1;
    for (v = 0; v < M; v++) {
        const int p = parent[v];
        if (p < -1 || p >= v) {
            *score = NAN;
            free(nd); free(a); free(depth);
            return -1;
        }
        a[v] = (p < 0 ? 1.0f : a[p]) * c[v];
        depth[v] = p < 0 ? 1 : depth[p] + 1;
        nd[v].a = a[v];
        nd[v].depth = depth[v];
        nd[v].v = v;
    }
    qsort(nd, (size_t)M, sizeof(orc_node), orc_node_cmp);
    for (i = 0; i < n && i < M; i++) {
        sel[i] = nd[i].v;
        sum_q += (int64_t)((double)nd[i].a * scale);
    }
    *score = (double)sum_q / scale;
    free(nd); free(a); free(depth);
    return 0;
}
