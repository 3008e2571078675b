/*
 * specdec.h -- C ABI of the MI355X (gfx950) speculative-decoding sampling
 * library: DSpark's sequential draft stage (Markov or RNN head) and lossless
 * rejection-sampling verification.
 *
 * Sources of the operations (page title, then section / equation):
 *   [DSpark]  "[논문리뷰] DSpark: Confidence-Scheduled Speculative Decoding
 *             with Semi-Autoregressive Generation" (kimjy99.github.io),
 *             §1.2 Sequential stage: block factorisation, per-position softmax,
 *             Markov-head equation, RNN-head equation; §2.2 scheduled
 *             acceptance lengths l_r in {0..gamma}.
 *   [VESSL]   "Speculative Decoding Part 1" (vessl.ai blog), section
 *             "알고리즘" (one speculative cycle) and section "수락 규칙"
 *             (acceptance rule, residual distribution, lossless theorem).
 *   [H-Spec]  "H-Spec: Parallel Speculative Decoding Without a Drafter-Side KV
 *             Cache" (jaehun.me), Appx. B.1 settings: Markov rank 256,
 *             vocabulary pruned to 32000, fixed-length verification.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *   row-major buffers on the current HIP device.  The library never
 *   allocates or frees caller memory; the only scratch is the caller's
 *   workspace (size from the *_workspace_size query, alignment 256 bytes).
 *   Concurrent calls need distinct workspaces.  A call keeps nothing after it
 *   returns except in its workspace and in these process-wide settings, each
 *   atomic and read once per call when the call launches its kernels:
 *     spec_draft_set_persistent  engine of the q-free Markov draft (default 1);
 *     spec_draft_set_poll_limit  wait limit of the persistent draft and of
 *                                the split tree walk;
 *     spec_profile_enable        kernel timing (off by default; a mutex);
 *   plus per-device caches of device attributes (CU count, cooperative
 *   launch support) and each kernel's LDS limit, set once per process, and
 *   two areas of static device memory per device: the exchange words of the
 *   split tree walk (spec_verify_tree, 64 KB, with its count of finished
 *   workgroups; each call leaves both zeroed) and the scratch of
 *   spec_verify_noalloc.
 * - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   All work is enqueued asynchronously on it; outputs are valid once the
 *   stream has been synchronised.  No entry point reads results back to the
 *   host or records a memset, and every word a call reads from its workspace
 *   or the static areas is written or reset by that call, so a sequence of
 *   calls can be captured in a HIP graph and replayed (the process-wide
 *   settings are then those at capture time); the GPU tests replay the
 *   q-free Markov cycle and the split tree walk this way.
 * - Argument validation is synchronous and happens before any launch; a
 *   non-SPEC_OK status means nothing was enqueued.  Checks that need device
 *   data (token ids, lengths) are done by the kernels: an offending request
 *   gets token -1 / accepted -1 in its outputs and the others are unaffected.
 *   Device faults surface at the caller's next synchronisation.
 * - spec_last_error() returns a thread-local description of the last failure.
 * - Logit dtypes: SPEC_F32 or SPEC_BF16.  Temperature T > 0 samples from
 *   softmax(logits / T); T == 0 is greedy (argmax, lowest token id on ties)
 *   and consumes no uniforms.  The library multiplies logits by the fp32
 *   value 1/T.
 * - Uniforms: if `uniforms` is non-NULL it is a device float array in
 *   [0, 1) laid out as documented per call; otherwise uniforms come from the
 *   counter-based Philox4x32-10 generator (Salmon et al., SC'11) with key
 *   (seed low 32 bits, seed high 32 bits) and counter
 *   (request b, position k, stream, offset); u = (word0 >> 8) * 2^-24.
 *   Streams: 0 = draft sample at position k, 1 = ratio test at position k,
 *   2 = the final (corrected or bonus) draw, position 0.  A draft call and a
 *   verify call of one cycle may therefore share (seed, offset).
 * - Sampling is by inverse CDF over ascending token id: the token is the
 *   smallest v with u * Z < S_v, S_v the running sum of the unnormalised
 *   weights and Z their total.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_ERR_INVALID = 1,      /* bad argument (null pointer, size, T < 0) */
    SPEC_ERR_UNSUPPORTED = 2,  /* dtype combination or size not supported */
    SPEC_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
    SPEC_ERR_HIP = 4           /* a HIP call or kernel launch failed */
} spec_status_t;

typedef enum {
    SPEC_F32 = 0,
    SPEC_BF16 = 1
} spec_dtype_t;

/* Library version (major * 10000 + minor * 100 + patch). */
int spec_version(void);

/* Thread-local text of the last error ("" if none). */
const char *spec_last_error(void);

/*
 * Counter-based uniforms, as used by every entry point: out[b * K + k] =
 * u(seed, offset, request b, position k, stream) for b < B, k < K.
 * out: device float [B, K].  Exposed so callers can reproduce or log the
 * draws of a cycle.
 */
spec_status_t spec_philox_uniforms(uint64_t seed, uint32_t offset, uint32_t stream,
                                   int B, int K, float *out, void *stream_handle);

/*
 * ---------------------------------------------------------------------------
 * Draft, Markov head  [DSpark §1.2, block factorisation and Markov-head eq.]
 * ---------------------------------------------------------------------------
 * For every request b and position k = 0..gamma-1, left to right:
 *     prev    = (k == 0) ? x0[b] : tokens[b, k-1]
 *     l[v]    = U[b, k, v] + sum_j W1[prev, j] * W2[j, v]
 *     tokens[b, k] ~ softmax(l / T)      (greedy if T == 0)
 *
 * U        [B, gamma, V]  base logits, dtype U_dtype (F32 or BF16)
 * x0       [B]            int32 anchor tokens (the previous cycle's last)
 * W1       [V, r]         embedding table,  dtype w_dtype
 * W2       [r, V]         logit projection, dtype w_dtype
 *                         (BF16 runs on MFMA with fp32 accumulation; F32 runs
 *                         on the vector ALUs)
 * W2T                     optional: W2 already packed by spec_pack_w2 (bf16
 *                         only).  NULL: W2 is packed into the workspace on
 *                         every call.  W2 may be NULL when W2T is given.
 * uniforms [B, gamma]     optional caller uniforms (stream 0 otherwise)
 * tokens   [B, gamma]     out: int32 draft tokens
 * q_logits [B, gamma, V]  out: fp32 draft logits l BEFORE temperature; pass
 *                         them unchanged (with the same T) to spec_verify.
 *                         NULL selects the q-free draft (bf16 weights): no
 *                         logits are written, q_logZ and q_tok_prob become
 *                         required, and spec_verify_markov verifies the block.
 * q_logZ   [B, gamma]     out: ln sum_v exp(l[v] / T) (T == 0: max l)
 * q_tok_prob [B, gamma]   out: q(tokens[b, k]) (T == 0: 1)
 *                         (both optional when q_logits is given)
 * Errors: SPEC_ERR_INVALID for null required pointers, B < 0, gamma < 0,
 * V <= 0, r <= 0, T < 0 or NaN; SPEC_ERR_UNSUPPORTED for other dtypes;
 * SPEC_ERR_WORKSPACE if ws_bytes < spec_draft_markov_workspace_size(...).
 * A request whose anchor is outside [0, V) gets tokens -1 from there on.
 * The draft entry points support V <= 262144 (SPEC_ERR_UNSUPPORTED above).
 */
size_t spec_draft_markov_workspace_size(int B, int gamma, int V, int r);

spec_status_t spec_draft_sample_markov(
    const void *U, int U_dtype, const int32_t *x0,
    const void *W1, const void *W2, const void *W2T, int w_dtype, int r,
    int B, int gamma, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *tokens, float *q_logits, float *q_logZ, float *q_tok_prob,
    void *ws, size_t ws_bytes, void *stream);

/*
 * W2 [r, V] bf16 -> W2T, the packed image the bias contraction copies into
 * LDS one 128-token tile at a time.  Weights are static, so callers pack once
 * and pass W2T to the draft and verify calls.
 * Layout (bf16 elements; a stable part of this interface): tile t holds tokens
 * 128t .. 128t + 127 as 128 rows of r elements (rows past V are zero); row v's
 * 16-byte chunk kc (elements 8kc .. 8kc + 7) is stored in chunk slot
 * kc ^ s(v mod 128), where s(u) = (u & 3) | ((((u >> 4) ^ (u >> 2)) & 3) << 2)
 * masked to F - 1, F = the largest power of two <= 16 that divides r / 8.
 * So W2[j][v] sits at element v * r + 8 * ((j / 8) ^ s) + j % 8.
 * W2T: caller-owned device buffer of spec_pack_w2_bytes(r, V) bytes,
 * 16-byte aligned.  Needs r % 16 == 0 and r <= 256 (SPEC_ERR_UNSUPPORTED).
 */
size_t spec_pack_w2_bytes(int r, int V);

spec_status_t spec_pack_w2(const void *W2, void *W2T, int r, int V, void *stream);

/*
 * Engine of the q-free Markov draft (bf16 weights, q_logits == NULL; U bf16
 * or fp32).
 *
 * 1 (the default) and 2: where the shape allows it (V % 8 == 0, r in {64,
 * 128, 256}, the device's share of packed W2 fitting in registers: V <= 153600
 * at r = 256 on 256 CUs, twice that per halving of r), every position runs in
 * one launch of one workgroup per CU that keeps W2 on chip: most workgroups
 * compute the bias and softmax summaries of 64-row blocks, a few draw the
 * tokens, and they synchronise through tagged summary and token words, so
 * every workgroup must be resident at once.
 *   1: plain launch.  Residency holds when no other kernel keeps CUs busy
 *      during the draft (e.g. the draft and the target model on one
 *      stream).  If it does not hold, the draft's bounded waits give up
 *      after about a second and the rows not drawn keep token -1: the call
 *      has still returned SPEC_OK (it only enqueues).  spec_draft_status
 *      reports that case after the fact, and the verification marks the
 *      requests holding a -1 token invalid (accepted -1).
 *   2: cooperative launch: the runtime guarantees residency by running the
 *      launch alone on the device, at the cost of ~20 us of idle device per
 *      call.  For callers that run other kernels concurrently.  One
 *      rocprofv3 counter run of a benchmark in this mode ended with a
 *      segmentation fault in the process's exit handlers after every result
 *      was written; its cause is not known (the library registers no exit
 *      work of its own), so this mode is not the default.
 * 0: two launches per position (a tile + finalize; the streaming tile when U
 *    is bf16 and B > 64).
 *
 * All modes give the same draws up to the rounding of the sums (1 and 2 are
 * the same kernel and give identical results).  Process-wide and atomic
 * (read once per draft call); returns the previous mode, or -1 (nothing
 * changed) for a mode outside 0..2.
 */
int spec_draft_set_persistent(int mode);

/*
 * Completion of the last Markov or RNN draft call made with the workspace
 * `ws` (same B, gamma, V, r as that call).  Enqueues on `stream` a copy of
 * the call's completion word into status[0] (device int32): 0 when every
 * draw of the call happened; 1 when the persistent engine's bounded waits
 * gave up (mode 1 without residency, or the poll limit reached), in which
 * case the rows not drawn hold token -1 from their first undrawn position
 * on.  Engines without waits always leave 0.  Stream-ordered after the draft
 * when enqueued on the draft's stream; read status after synchronising.
 * Errors: SPEC_ERR_INVALID for a null status or bad sizes,
 * SPEC_ERR_WORKSPACE for a workspace smaller than the draft's.
 */
spec_status_t spec_draft_status(const void *ws, size_t ws_bytes, int B, int gamma, int V, int r,
                                int32_t *status, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Draft, RNN head  [DSpark §1.2, RNN-head equation]
 * ---------------------------------------------------------------------------
 * As the Markov head, with the bias of position k given by
 *     z_k  = [s_{k-1}; W1[prev]; h[b, k]]            (length 2r + d)
 *     g    = sigmoid(Wg z_k),  c = tanh(Wc z_k),  o = tanh(Wo z_k)
 *     s_k  = g * s_{k-1} + (1 - g) * c,    s_0 = 0
 *     l[v] = U[b, k, v] + sum_j W2[j, v] * o[j]
 * h  [B, gamma, d]  backbone hidden states, dtype h_dtype (BF16)
 * Wg, Wc, Wo [r, 2r + d]  gate matrices, dtype w_dtype (BF16), no bias terms
 * The state s and o are kept in fp32; o enters the W2 contraction as an
 * exact three-term bf16 split so the bf16 MFMA path keeps fp32 accuracy.
 * Other arguments, outputs and errors as spec_draft_sample_markov.  With
 * q_logits == NULL the draft is q-free, as the Markov head's per-position
 * engine: only tokens, q_logZ and q_tok_prob are written; the group of the
 * draw is rebuilt from U, W2 and the three bf16 terms of o_k.  After either
 * mode the workspace holds the conditioning rows of every position: the
 * three bf16 terms of o_k, [B, gamma, 3, r], at byte offset
 * spec_draft_rnn_cond_offset(B, gamma, V, r, d).  spec_verify_rnn reads them
 * from there, so a q-free RNN cycle keeps the draft's workspace (unchanged)
 * until its verification has run.
 */
size_t spec_draft_rnn_workspace_size(int B, int gamma, int V, int r, int d);
size_t spec_draft_rnn_cond_offset(int B, int gamma, int V, int r, int d);

spec_status_t spec_draft_sample_rnn(
    const void *U, int U_dtype, const int32_t *x0,
    const void *h, int h_dtype, int d,
    const void *W1, const void *W2, const void *W2T,
    const void *Wg, const void *Wc, const void *Wo, int w_dtype, int r,
    int B, int gamma, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *tokens, float *q_logits, float *q_logZ, float *q_tok_prob,
    void *ws, size_t ws_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Lossless verification  [VESSL "알고리즘" and "수락 규칙"]
 * ---------------------------------------------------------------------------
 * For every request b with L = lens ? lens[b] : gamma_max drafted positions:
 *     p_k = softmax(P_k / T) for k = 0..L,  q_k = softmax(Q_k / T) for k < L
 *     accept position k iff u_k * q_k(x_k) < p_k(x_k)   (x_k = draft[b, k])
 *     n = first rejected position, or L
 *     n < L: final ~ max(0, p_n - q_n) / sum(max(0, p_n - q_n))
 *     n = L: final ~ p_L (bonus token)
 *     out[b] = x_0..x_{n-1}, final, then -1;   accepted[b] = n  (tau = n + 1)
 * T == 0: accept iff argmax p_k == x_k; final = argmax p_n.
 * If the residual has zero mass after rounding, p_n is sampled instead.
 *
 * P         target logits, dtype p_dtype.  Dense: [B, gamma_max + 1, V].
 *           Packed (p_row_off != NULL): request b owns rows
 *           p_row_off[b] .. p_row_off[b] + L (L + 1 rows of V).
 * Q         draft logits before temperature, dtype q_dtype.  Dense:
 *           [B, gamma_max, V]; packed (q_row_off != NULL): rows
 *           q_row_off[b] .. q_row_off[b] + L - 1.
 * draft     [B, gamma_max] int32 draft tokens (first L used)
 * lens      [B] int32 in [0, gamma_max], or NULL for fixed length gamma_max
 * p_row_off, q_row_off  [B] int64 row offsets, or NULL for dense
 * uniforms  [B, gamma_max + 1] optional caller uniforms: column k < gamma_max
 *           is the ratio test of position k, column gamma_max the final draw
 * accepted  [B] out int32 n (-1 for a request with invalid tokens/length)
 * out_tokens [B, gamma_max + 1] out int32
 * p_logZ    [B, gamma_max + 1] optional out: ln sum exp(P_k / T) (T == 0:
 *           max logit); q_logZ [B, gamma_max] likewise for Q;
 * accept_prob [B, gamma_max] optional out: min(1, p_k(x_k) / q_k(x_k))
 *           (T == 0: 1 or 0).  Entries for k beyond L are 0.
 * Errors: SPEC_ERR_INVALID for null required pointers, B < 0,
 * gamma_max < 0, V <= 0, T < 0 or NaN; SPEC_ERR_UNSUPPORTED for other
 * dtypes; SPEC_ERR_WORKSPACE for a short workspace.
 */
size_t spec_verify_workspace_size(int B, int gamma_max, int V);

spec_status_t spec_verify(
    const void *P, int p_dtype, const void *Q, int q_dtype,
    const int32_t *draft, const int32_t *lens,
    const int64_t *p_row_off, const int64_t *q_row_off,
    int B, int gamma_max, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *accepted, int32_t *out_tokens,
    float *p_logZ, float *q_logZ, float *accept_prob,
    void *ws, size_t ws_bytes, void *stream);

/*
 * spec_verify without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs, kernels and results as
 * spec_verify; the scratch is a fixed array of spec_verify_noalloc_max_bytes()
 * (16 MiB) in the library's device image, one per GPU, held until the process
 * ends; its address on the current device is looked up on the first call
 * there.  The call allocates nothing (no hipMalloc or hipFree); calls whose
 * spec_verify_workspace_size(B, gamma_max, V) exceeds the limit return
 * SPEC_ERR_WORKSPACE before any launch.  Every call on one GPU uses the same
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race and give wrong results: serialise them.  Nothing in the array must
 * start at zero; each call writes every word it reads.
 */
size_t spec_verify_noalloc_max_bytes(void);

spec_status_t spec_verify_noalloc(
    const void *P, int p_dtype, const void *Q, int q_dtype,
    const int32_t *draft, const int32_t *lens,
    const int64_t *p_row_off, const int64_t *q_row_off,
    int B, int gamma_max, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *accepted, int32_t *out_tokens,
    float *p_logZ, float *q_logZ, float *accept_prob, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Lossless verification of a q-free Markov draft
 * [VESSL "알고리즘", "수락 규칙"; DSpark §1.2 Markov-head eq.]
 * ---------------------------------------------------------------------------
 * The same acceptance rule as spec_verify, for a block drafted with
 * q_logits == NULL.  q_k(x_k) and the normaliser of q_k come from the draft
 * (q_tok_prob, q_logZ); the draft row that feeds a correction is rebuilt as
 * l_n = U[b, n] + W1[x_{n-1}] W2 in fp32 by other kernels than the draft's:
 * with bf16 P and U, T > 0 and gamma_max > 0 by a streaming kernel that keeps
 * the rebuilt row in registers and sums the residual weights per 8-token group
 * (verify_resid_stream, then verify_resid_finalize descends to the token);
 * otherwise the rebuilt rows are written to the workspace and drawn from.  The
 * rebuild sums the contraction in another order than the draft engine, so it
 * matches the logits the draft sampled from to fp32 rounding (about 1e-6
 * relative), not bit for bit; draws differ only inside the 1e-6 boundary band
 * of a CDF interval.  Only target rows are streamed in full.
 * U, x0, W1, W2/W2T, w_dtype, r  as passed to spec_draft_sample_markov
 * (U dense [B, gamma_max, V]); draft [B, gamma_max] = the draft's tokens;
 * q_logZ, q_tok_prob [B, gamma_max] = the draft's outputs (same T).
 * P, lens, p_row_off, uniforms, accepted, out_tokens, p_logZ, accept_prob:
 * as spec_verify.  Needs bf16 weights and V <= 262144.
 */
size_t spec_verify_markov_workspace_size(int B, int gamma_max, int V, int r);

spec_status_t spec_verify_markov(
    const void *P, int p_dtype, const void *U, int U_dtype, const int32_t *x0,
    const void *W1, const void *W2, const void *W2T, int w_dtype, int r,
    const int32_t *draft, const float *q_logZ, const float *q_tok_prob,
    const int32_t *lens, const int64_t *p_row_off,
    int B, int gamma_max, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *accepted, int32_t *out_tokens, float *p_logZ, float *accept_prob,
    void *ws, size_t ws_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Lossless verification of a q-free RNN draft
 * [VESSL "알고리즘", "수락 규칙"; DSpark §1.2 RNN-head eq.]
 * ---------------------------------------------------------------------------
 * spec_verify_markov's rule and outputs for a block drafted by
 * spec_draft_sample_rnn with q_logits == NULL.  q_k(x_k) and the normaliser
 * of q_k come from the draft (q_tok_prob, q_logZ); the draft row of a
 * rejected position n is rebuilt as l_n = U[b, n] + W2^T o_n from the draft's
 * conditioning rows cond = (char *)draft_ws + spec_draft_rnn_cond_offset(...)
 * ([B, gamma, 3, r] bf16, the three bf16 terms of o_n), written to this
 * call's workspace and drawn from (fp32, same summation as the draft's tile:
 * the rebuilt logits match the draft's to fp32 rounding).
 * P, U, W2 / W2T (bf16, r % 16 == 0, r <= 256), draft, q_logZ, q_tok_prob,
 * lens, p_row_off, uniforms, outputs and errors as spec_verify_markov.
 */
size_t spec_verify_rnn_workspace_size(int B, int gamma_max, int V, int r);

spec_status_t spec_verify_rnn(
    const void *P, int p_dtype, const void *U, int U_dtype, const void *cond,
    const void *W2, const void *W2T, int r,
    const int32_t *draft, const float *q_logZ, const float *q_tok_prob,
    const int32_t *lens, const int64_t *p_row_off,
    int B, int gamma_max, int V, float T,
    const float *uniforms, uint64_t seed, uint32_t offset,
    int32_t *accepted, int32_t *out_tokens, float *p_logZ, float *accept_prob,
    void *ws, size_t ws_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Verification of a tree draft  [VESSL "Speculative Decoding Part 1",
 * section "γ 재배분: 체인 대신 트리" (a tree of continuations verified in one
 * target pass), with the acceptance rule of section "수락 규칙"]
 * ---------------------------------------------------------------------------
 * Request b holds a tree of n = n_nodes ? n_nodes[b] : M draft nodes, listed
 * parents first: parent[b, v] in [-1, v) (-1: a child of the root, the last
 * accepted token), tokens[b, v] its draft token in [0, V).  Row 0 of P and Q
 * belongs to the root and row 1 + v to node v (rows of unused nodes are not
 * read): the P row is the target's next-token logits after the path to that
 * node, the Q row the draft logits its children were drawn from (one
 * independent draw per child).  With p = softmax(P row / T) and q =
 * softmax(Q row / T) of the current node, starting at the root with r = p:
 *     test the node's children in increasing index; child c (token x) passes
 *     iff u_c * q(x) < r(x): emit x, move to c, r = p of c, repeat;
 *     on a failure r <- normalize(max(0, r - q)) and test the next child;
 *     no child passes: final ~ r (inverse CDF with u_final); a node without
 *     children: final ~ p of that node (bonus token).
 * T == 0: the first child whose token is the argmax of p passes (lowest id
 * on ties); the final token is that argmax.  If a residual has no mass after
 * rounding the final token is drawn from the node's p.  Every emitted token
 * follows the target's law given the tokens before it; a chain-shaped tree
 * (parent[v] = v - 1) is spec_verify's rule.
 *
 * P, Q       [B, M + 1, V] dtype p_dtype / q_dtype (f32 or bf16), 16-byte
 *            aligned.  Q may be NULL when M == 0.
 * parent, tokens  [B, M] int32 (NULL allowed when M == 0)
 * n_nodes    [B] int32 in [0, M], or NULL for M
 * uniforms   [B, M + 1] optional: column v < M is node v's ratio test,
 *            column M the final draw; NULL: Philox stream 3 (index v, and M
 *            for the final draw)
 * accepted   [B] out int32: number of accepted nodes (-1 for a request with
 *            a parent out of range, a token outside [0, V), n_nodes outside
 *            [0, M] or a row on the walk without a finite logit)
 * out_tokens [B, M + 1] out int32: the accepted nodes' tokens, the final
 *            token, then -1 (all -1 for an invalid request)
 * path       [B, M] optional out int32: the accepted node ids, then -1
 * W workgroups per request, W = min(8, CUs / B, ceil(V / 512)) (one when the
 * batch fills the device): each covers a range of the vocabulary, every
 * tested sibling after the first costs one pass over the node's two rows,
 * and the workgroups of a request exchange each pass's partial sums through
 * the library's static exchange area (device memory; the last workgroup of
 * each call zeroes what the call used, so the call can also be captured in a
 * graph and replayed).  No workspace.  With W > 1 all of a call's
 * workgroups must be resident at once, which an otherwise idle device gives;
 * calls that overlap on one device (other streams) are not supported then.  Every wait of the walk is bounded
 * (spec_draft_set_poll_limit): when one gives up, the requests not finished
 * report accepted -1 with all-(-1) out_tokens and path.
 * Errors: SPEC_ERR_INVALID (null required pointers, B or M < 0, V outside
 * [1, 2^20], T < 0 or NaN), SPEC_ERR_UNSUPPORTED (dtype, M > 1024,
 * misaligned P or Q), SPEC_ERR_HIP (launch).
 */
spec_status_t spec_verify_tree(const void *P, int p_dtype, const void *Q, int q_dtype,
                               const int32_t *parent, const int32_t *tokens,
                               const int32_t *n_nodes, int B, int M, int V, float T,
                               const float *uniforms, uint64_t seed, uint32_t offset,
                               int32_t *accepted, int32_t *out_tokens, int32_t *path,
                               void *stream);

/*
 * ---------------------------------------------------------------------------
 * Acceptance rate per drafted position  [VESSL "Speculative Decoding Part 1",
 * section "수락 규칙": a token drawn from q passes the ratio test with
 * probability alpha = sum_v min(p(v), q(v)) = 1 - D_TV(p, q)]
 * ---------------------------------------------------------------------------
 * For every request b and position k < L_b (L_b = lens[b], or gamma_max when
 * lens is NULL): p_k = softmax(P row / T), q_k = softmax(Q row / T),
 *   alpha[b, k] = sum_v min(p_k(v), q_k(v)),
 *   tv[b, k]    = 1/2 sum_v |p_k(v) - q_k(v)|   (optional; returned as
 *                 1 - alpha, which it equals).
 * T = 0: both are one-hot at their argmax (lowest id on ties), so alpha is 1
 * when the argmaxes agree and 0 otherwise.  The row layout is spec_verify's:
 * P dense [B, gamma_max + 1, V] or packed rows from p_row_off[b] on (position
 * k at row p_row_off[b] + k); Q dense [B, gamma_max, V] or packed from
 * q_row_off[b] on.  The bonus row of P is not read.  Positions k >= L_b, a
 * length outside [0, gamma_max] and rows without a finite logit give NaN.
 *
 * P, Q, alpha, tv: caller-owned device buffers (f32 or bf16 logits; alpha and
 * tv fp32 [B, gamma_max]).  No workspace.  Errors: SPEC_ERR_INVALID (null P,
 * Q or alpha, B or gamma_max < 0, V out of range, T < 0 or not finite),
 * SPEC_ERR_UNSUPPORTED (dtype), SPEC_ERR_HIP (launch).  One pass for the
 * normalisers and one for the sums: reads every used P and Q row twice.
 */
spec_status_t spec_acceptance_rate(const void *P, int p_dtype, const void *Q, int q_dtype,
                                   const int32_t *lens, const int64_t *p_row_off,
                                   const int64_t *q_row_off, int B, int gamma_max, int V,
                                   float T, float *alpha, float *tv, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Confidence head  [DSpark §2.1 "Confidence Head", head equation]
 * ---------------------------------------------------------------------------
 * For every request b < R and drafted position k < gamma:
 *     prev    = (k == 0) ? x0[b] : draft[b, k-1]
 *     c[b, k] = sigmoid( sum_i w[i] h[b, k, i] + sum_j w[d + j] W1[prev, j] )
 * an estimate of the chance that the draft token at position k is accepted.
 *
 * h     [R, gamma, d]  backbone hidden state at each drafted position, h_dtype
 * x0    [R]            int32 anchor tokens; draft [R, gamma] int32 draft tokens
 *                      (draft[b, gamma-1] is not read)
 * W1    [V, r]         the Markov head's embedding table, w_dtype
 * w     [d + r]        fp32 head weights (hidden block first)
 * c     [R, gamma]     out: fp32 confidences; 0 where prev is outside [0, V)
 *                      (e.g. after an undrawn token -1)
 * Dot products in fp32 (per-lane sums, then a wave tree), sigmoid in fp32.
 * All pointers are device memory, stream-ordered; nothing is kept.
 * Errors: SPEC_ERR_INVALID for null pointers, R, gamma < 0, d, r, V <= 0;
 * SPEC_ERR_UNSUPPORTED for other dtypes; R * gamma == 0 does nothing.
 */
spec_status_t spec_confidence_head(const void *h, int h_dtype, int d, const int32_t *x0,
                                   const int32_t *draft, const void *W1, int w_dtype, int r,
                                   const float *w, int R, int gamma, int V, float *c,
                                   void *stream);

/*
 * ---------------------------------------------------------------------------
 * Hardware-aware prefix scheduler  [DSpark §2.2, survival products,
 * B and tau, Theta = tau * SPS(B), global greedy admission, early stop]
 * ---------------------------------------------------------------------------
 * Chooses how many drafted tokens l_r in [0, gamma] each request sends to
 * verification:
 *     a[r, j]  = c[r, 0] * ... * c[r, j]   (fp32, left to right)
 *     candidates (r, j) in order of a descending (ties: lower r, then lower j)
 *     are admitted one at a time; after t admissions B_t = R + t and
 *     tau_t = R + sum of the admitted a, each a cut to a multiple of 2^-48
 *     and summed exactly in integers; Theta_t = tau_t * sps[B_t] in double
 *     (0 for B_t >= nsps).  The search stops at the first t with
 *     Theta_t < Theta_{t-1}; that candidate is not admitted.
 * Because a is non-increasing along a request, the admitted set is a prefix
 * of every request.
 *
 * c       [R, gamma]  fp32 confidences, each in [0, 1] (other values are
 *                     clamped into [0, 1], NaN to 0)
 * sps     [nsps]      double steps per second of the engine at batch size B
 *                     (index B); may be NULL when nsps == 0
 * lens    [R]         out: int32 l_r
 * B_out   [1]         out (optional): int32 chosen batch size R + sum l_r
 * tau_out [1]         out (optional): double tau at that size
 * ws      [ws_bytes]  caller workspace, 16-byte aligned, at least
 *                     spec_prefix_schedule_workspace_size(R, gamma) bytes (the
 *                     candidates in sorted order); unused when R * gamma == 0
 * Two launches: workgroups that rank slices of the candidates, then one
 * workgroup that scans them.  All pointers device memory, stream-ordered.
 * Errors: SPEC_ERR_INVALID for null c or lens (R > 0), R, gamma, nsps < 0,
 * null sps with nsps > 0; SPEC_ERR_UNSUPPORTED for R > 8192 or
 * R * gamma > 8192; SPEC_ERR_WORKSPACE for a missing, unaligned or short
 * workspace.
 */
size_t spec_prefix_schedule_workspace_size(int R, int gamma);
spec_status_t spec_prefix_schedule(const float *c, int R, int gamma, const double *sps,
                                   int nsps, int32_t *lens, int32_t *B_out, double *tau_out,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Tree drafts: top-n nodes by survival probability  [VESSL "Speculative
 * Decoding Part 1", section "γ 재배분: 체인 대신 트리"]
 * ---------------------------------------------------------------------------
 * For each of R candidate trees of M nodes listed parents first:
 *     a_v = c_v * a_parent(v)   (fp32; a child of the root has a = c_v)
 *     sel[t, 0 .. n-1] = the n nodes of highest a_v, ties to the shallower
 *     node, then the lower id; -1 past M.  Because a never grows down a
 *     branch, the chosen set contains the parent of every chosen node.
 *     score[t] = the sum of the chosen a_v, each cut to a multiple of
 *     2^-48 and summed exactly (the expected number of accepted nodes).
 *
 * parent [R, M]  int32 parent ids, parent[t, v] in [-1, v) (-1: a child of
 *                the root, the last accepted token)
 * c      [R, M]  fp32 chance that node v is accepted once its parent is, in
 *                [0, 1] (other values are clamped into [0, 1], NaN to 0)
 * sel    [R, n]  out: int32 node ids in selection order
 * score  [R]     out (optional): fp64
 * A tree with a parent id outside [-1, v) gets sel -1 and score NaN.
 * One workgroup per tree; all pointers device memory, stream-ordered.
 * Errors: SPEC_ERR_INVALID for R, M, n < 0 or null parent, c (M > 0) or sel
 * (n > 0); SPEC_ERR_UNSUPPORTED for M > 4096.
 */
spec_status_t spec_tree_select(const int32_t *parent, const float *c, int R, int M, int n,
                               int32_t *sel, double *score, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Kernel timing (benchmarking aid; not needed for correct use)
 * ---------------------------------------------------------------------------
 * spec_profile_enable(name) starts a fresh record: from then on every launch
 * of the kernel `name` ("draft_tile", "draft_tile_qfree", "draft_finalize",
 * "draft_persist", "rnn_hidden_proj",
 * "rnn_gates", "w2_transpose", "verify_rows_p", "verify_rows_q",
 * "verify_decide", "verify_residual_rows", "verify_final_partials",
 * "verify_final_draw", "verify_resid", "acceptance_rate", "confidence_head",
 * "prefix_schedule", "tree_select", or "*" for all) is bracketed
 * by two hipEvents recorded on its launch stream.  NULL or "" stops timing.
 * spec_profile_read waits for the recorded events and returns the number of
 * timed launches and their summed duration in milliseconds.  Process-wide
 * state, guarded by a mutex; events are created on first use and reused.
 */
spec_status_t spec_profile_enable(const char *kernel);
spec_status_t spec_profile_read(int *launches, double *total_ms);

/*
 * Wait limit of the persistent draft (testing aid; not needed for correct
 * use).  Every wait of the persistent draft (a unit workgroup for the token
 * words of its rows, a finalize wave for the share summaries of its row) is a
 * poll that gives up after `polls` polls (about 1 us each on an idle device):
 * it sets the launch's abort word, every workgroup leaves at its next poll,
 * and the rows not drawn keep token -1 (spec_draft_status reports 1).  The
 * exchange waits of the split tree walk (spec_verify_tree with more than one
 * workgroup per request) use the same limit.  0 restores the default (2^20
 * polls).  Lets a test force that path from the host.  Process-wide and
 * atomic; applies to later launches; returns the previous limit.
 */
unsigned spec_draft_set_poll_limit(unsigned polls);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
