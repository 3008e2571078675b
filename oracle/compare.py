"""Element-by-element comparison of a GPU result with the oracle's.

TEST INFRASTRUCTURE ONLY.  The oracle runs on the same seeded inputs as the
GPU and never receives anything the GPU produced.  The bar:

* token ids and accepted counts match exactly, except a draw whose uniform
  lies within BAND (1e-6) of the oracle's CDF boundary between the oracle's
  choice and the GPU's, or, at T = 0, a draft argmax whose two logits differ
  by no more than the error bounds of their fp32 computation (Markov head:
  gamma_{r+1} (|U| + |W1[x]| . |W2|) per logit; the RNN head, whose o carries
  the gates' own rounding, keeps the fixed band 1e-5 * max(1, |l|)).
  Verification's greedy choices take the argmax of given rows and are exact.  Such draws are counted and reported.  After
  a boundary draw in a draft chain the rest of that request conditions on a
  different prefix and is not compared.
* normalisers (log Z): |delta| <= 1e-5; probabilities q(x), min(1, p/q):
  relative 1e-5; draft logits: within the same per-logit bound (Markov
  head) or 1e-5 * max(1, |l|) (RNN head).
"""
import numpy as np

from . import binding as orc

BAND = 1e-6
TOL_LOGZ = 1e-5
TOL_REL = 1e-5
U32 = 2.0 ** -24     # unit roundoff of fp32


def _gamma(n):
    """gamma_n = n u / (1 - n u) (Higham, Accuracy and Stability of Numerical
    Algorithms, §3.1): |fl(x^T y) - x^T y| <= gamma_n |x|^T |y| for a dot
    product of n terms summed in any order with each operation rounded."""
    return n * U32 / (1.0 - n * U32)


def markov_logit_bound(U_k, W1, W2, prev):
    """Bound on |fl(l) - l| for the fp32 kernels' Markov-head logits
    l = U_k + W1[prev] . W2 (r products and one add, every input exact in fp32:
    bf16 or fp32 values): gamma_{r+1} (|U_k| + |W1[prev]| . |W2|)."""
    r = W1.shape[1]
    if prev < 0 or prev >= W1.shape[0]:
        return np.full(U_k.shape, np.inf)
    return _gamma(r + 1) * (np.abs(U_k) + np.abs(W1[prev]) @ np.abs(W2))


class Tally:
    def __init__(self):
        self.draws = 0
        self.boundary = 0
        self.compared_positions = 0
        self.requests = 0
        self.skipped_after_boundary = 0
        self.fallbacks = 0

    def as_dict(self):
        return dict(draws=self.draws, boundary=self.boundary,
                    compared_positions=self.compared_positions, requests=self.requests,
                    skipped_after_boundary=self.skipped_after_boundary, fallbacks=self.fallbacks)


def _interval_distance(w, y, u):
    lo, hi = orc.cdf_interval(w, y)
    if not np.isfinite(lo):
        return np.inf
    if lo <= u < hi:
        return 0.0
    return max(lo - u, u - hi)


def _check_draw(w, orc_tok, gpu_tok, u, what):
    """Token equality or a draw inside the boundary band.  Returns True when
    it was a boundary draw."""
    if gpu_tok == orc_tok:
        return False
    if gpu_tok < 0 or gpu_tok >= len(w):
        raise AssertionError(f"{what}: GPU token {gpu_tok} out of range (oracle {orc_tok})")
    dist = _interval_distance(w, gpu_tok, u)
    if dist > BAND:
        raise AssertionError(f"{what}: GPU token {gpu_tok} != oracle {orc_tok}, uniform {u} is "
                             f"{dist:.3e} from the GPU token's CDF interval (band {BAND})")
    return True


def _check_greedy(l, orc_tok, gpu_tok, what, err=None):
    """A greedy mismatch is a tie within the GPU's arithmetic: the two exact
    logits differ by at most the sum of their computed values' error bounds
    (err, per token; without it the fixed band TOL_REL * max(1, |l|))."""
    if gpu_tok == orc_tok:
        return False
    if gpu_tok < 0 or gpu_tok >= len(l):
        raise AssertionError(f"{what}: greedy GPU token {gpu_tok} out of range")
    gap = l[orc_tok] - l[gpu_tok]
    tol = (err[orc_tok] + err[gpu_tok]) if err is not None else TOL_REL * max(1.0, abs(l[orc_tok]))
    if not (0 <= gap <= tol):
        raise AssertionError(f"{what}: greedy GPU token {gpu_tok} != oracle {orc_tok}, "
                             f"logit gap {gap:.3e} > {tol:.1e}")
    return True


def _close(a, b, atol, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bad = ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    if np.any(bad):
        i = int(np.flatnonzero(bad.ravel())[0])
        raise AssertionError(f"{what}: GPU {a.ravel()[i]!r} vs oracle {b.ravel()[i]!r} at flat "
                             f"index {i} ({int(bad.sum())} mismatches)")


def compare_draft_request(orc_out, U, gpu, T, u, what, tally, check_logits=True):
    """Compare one request's draft.  orc_out: oracle draft dict; U: base
    logits [gamma, V] (float64); gpu: dict of numpy arrays for this request
    (tokens [gamma], q_logits [gamma, V], q_logZ, q_tok_prob); u: uniforms."""
    gamma = len(orc_out["tokens"])
    tally.requests += 1
    mk = orc_out.get("markov")   # Markov head: the derived per-logit error bound
    for k in range(gamma):
        l = orc_out["q_logits"][k]
        gt, ot = int(gpu["tokens"][k]), int(orc_out["tokens"][k])
        err = markov_logit_bound(U[k], mk["W1"], mk["W2"], int(mk["prev"][k])) if mk else None
        if check_logits:
            tol = err + 1e-12 * np.abs(l) if err is not None else TOL_REL * np.maximum(1.0, np.abs(l))
            _close(gpu["q_logits"][k], l, tol, 0.0, f"{what} q_logits[k={k}]")
        if T > 0:
            _close(gpu["q_logZ"][k], orc_out["logZ"][k], TOL_LOGZ, 0.0, f"{what} q_logZ[k={k}]")
        tally.draws += 1
        tally.compared_positions += 1
        if T == 0:
            boundary = _check_greedy(l, ot, gt, f"{what} k={k}", err)
        else:
            w, Z, _ = orc.softmax_weights(l, T)
            boundary = _check_draw(w, ot, gt, u[k], f"{what} k={k}")
            if not boundary:
                _close(gpu["q_tok_prob"][k], orc_out["q_tok"][k], 1e-30, TOL_REL,
                       f"{what} q_tok_prob[k={k}]")
        if boundary:
            tally.boundary += 1
            tally.skipped_after_boundary += gamma - k - 1
            return False
    return True


def compare_verify_request(P, Q, draft, T, u_test, u_final, gpu, what, tally):
    """Compare one request's verification.  P [L+1, V], Q [L, V] float64
    (the exact values both sides received); gpu: dict with accepted (int),
    out_tokens [gamma_max+1], optional p_logZ, q_logZ, accept_prob rows."""
    L = len(draft)
    o = orc.verify(P, Q, draft, T, u_test, u_final)
    tally.requests += 1
    tally.fallbacks += o["fallback"]
    n_g, n_o = int(gpu["accepted"]), o["n"]
    if "p_logZ" in gpu:
        _close(gpu["p_logZ"][:L + 1], o["logZp"], TOL_LOGZ, 0.0, f"{what} p_logZ")
        if L:
            _close(gpu["q_logZ"][:L], o["logZq"], TOL_LOGZ, 0.0, f"{what} q_logZ")
            _close(gpu["accept_prob"][:L], o["accept_prob"], 1e-7, TOL_REL, f"{what} accept_prob")
    out_g = np.asarray(gpu["out_tokens"])
    if n_g != n_o:
        k = min(n_g, n_o)
        tally.draws += 1
        if T == 0 or not (o["test_margin"][k] <= BAND):
            raise AssertionError(f"{what}: accepted {n_g} != oracle {n_o}; ratio-test margin at "
                                 f"position {k} is {o['test_margin'][k]:.3e}")
        tally.boundary += 1
        return False
    if not np.array_equal(out_g[:n_o], np.asarray(draft[:n_o])):
        raise AssertionError(f"{what}: emitted draft tokens differ")
    if np.any(out_g[n_o + 1:] != -1):
        raise AssertionError(f"{what}: slots after the final token must be -1")
    tally.draws += 1
    final_g, final_o = int(out_g[n_o]), int(o["out"][n_o])
    if final_g == final_o:
        return True
    if T == 0:
        raise AssertionError(f"{what}: greedy final token {final_g} != oracle {final_o}")
    logZp = o["logZp"][n_o]
    if n_o < L and not o["fallback"]:
        w, _ = orc.residual_weights(P[n_o], Q[n_o], T, logZp, o["logZq"][n_o])
    else:
        w, _, _ = orc.softmax_weights(P[n_o], T)
    _check_draw(w, final_o, final_g, u_final, f"{what} final draw (n={n_o})")
    tally.boundary += 1
    return False


def compare_tree_request(P, Q, parent, tok, T, u_node, u_final, gpu, what, tally):
    """Compare one request's tree verification.  P, Q [M + 1, V] float64 (the
    exact values both sides received), parent / tok the nodes in use; gpu:
    dict with accepted (int), out_tokens [M + 1], path [M].

    The walks must agree node by node.  Where they part, the first sibling
    decided differently must have been a boundary test: its uniform within
    BAND of the oracle's ratio r(x)/q(x) (T = 0: the node's top-2 logit gap
    within the fp32 tolerance).  On the same walk the final token must match,
    or lie within BAND of the oracle's CDF boundary."""
    M = len(parent)
    o = orc.verify_tree(P, Q, parent, tok, T, u_node, u_final, want_weights=True)
    tally.requests += 1
    out_g = np.asarray(gpu["out_tokens"])
    n_g = int(gpu["accepted"])
    if o is None:
        if n_g != -1 or np.any(out_g != -1):
            raise AssertionError(f"{what}: invalid tree, GPU accepted {n_g} (expected -1, all -1)")
        return True
    tally.fallbacks += o["fallback"]
    n_o = o["n"]
    path_g = np.asarray(gpu["path"])[: max(n_g, 0)] if n_g >= 0 else np.zeros(0, np.int64)
    path_o = o["path"][:n_o]
    tally.draws += 1
    if n_g < 0:
        raise AssertionError(f"{what}: GPU marked a valid tree invalid")
    k = 0
    while k < min(n_g, n_o) and path_g[k] == path_o[k]:
        k += 1
    if k < n_g or k < n_o:
        # the walks part after k common nodes: the first sibling decided
        # differently is the smaller of the two next nodes (or the one side's)
        nxt = [int(x) for x in (path_g[k] if k < n_g else M, path_o[k] if k < n_o else M)]
        c = min(nxt)
        node = int(path_o[k - 1]) if k > 0 else -1
        if T == 0:
            l = P[node + 1]
            top = np.sort(l)[::-1]
            if not (top[0] - top[1] <= TOL_REL * max(1.0, abs(top[0]))):
                raise AssertionError(f"{what}: greedy walks part after {k} nodes, logit gap "
                                     f"{top[0] - top[1]:.3e}")
        else:
            ratio = o["test_ratio"][c] if c < M else np.nan
            if not np.isfinite(ratio) or abs(u_node[c] - ratio) > BAND:
                raise AssertionError(f"{what}: walks part after {k} nodes at node {c}: uniform "
                                     f"{u_node[c] if c < M else u_final} vs oracle ratio {ratio}")
        tally.boundary += 1
        return False
    if not np.array_equal(out_g[:n_o], np.asarray(tok)[path_o]):
        raise AssertionError(f"{what}: emitted tokens are not the accepted nodes' tokens")
    if np.any(out_g[n_o + 1:] != -1) or np.any(np.asarray(gpu["path"])[n_o:M] != -1):
        raise AssertionError(f"{what}: slots after the final token / path must be -1")
    final_g, final_o = int(out_g[n_o]), int(o["out"][n_o])
    if final_g == final_o:
        return True
    last = int(path_o[n_o - 1]) if n_o > 0 else -1
    if T == 0:
        _check_greedy(P[last + 1], final_o, final_g, f"{what} greedy final")
    else:
        _check_draw(o["final_w"], final_o, final_g, u_final, f"{what} final draw (n={n_o})")
    tally.boundary += 1
    return False
