"""ctypes binding of oracle.c (plain C, fp64).

TEST INFRASTRUCTURE ONLY.  Inputs are numpy float64 arrays for one request at
a time; callers decode bf16 inputs exactly (bits << 16) before passing them.
Nothing here does the method's arithmetic: every step runs in oracle.c.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# What pins each oracle function to something other than itself (tests in
# tests/test_oracle_*.py).  None of them is "parity unpinned".
PINS = {
    "philox4x32_10": "raw words equal ATen's header-only Philox engine on random counters/keys",
    "uniform": "mean/variance and 256-bin chi-square; exactly 24-bit grid",
    "softmax_weights": "logZ equals scipy.special.logsumexp; all-equal row gives Z=V",
    "inverse_cdf": "equals numpy.searchsorted(cumsum, u*Z, 'right'); chi-square of draws",
    "argmax": "lowest index on ties vs numpy.argmax; top-2 gap brute force",
    "draft_markov": "bias equals W1[x]@W2 (numpy); W2=0 reduces to i.i.d. softmax(U) draws",
    "draft_rnn": "gate limits (sigmoid->1 keeps s=0; ->0 gives s=tanh(Wc z)); Wo=0 gives no bias; hand-derived r=1 case",
    "verify": "exact output law by brute-force enumeration equals softmax(P/T) at T in "
              "{0.5, 0.7, 1, 1.3, 2} (lossless theorem); normalisers equal scipy logsumexp(row/T); "
              "min(1, p/q) equals numpy's ratio at T; acceptance frequency equals sum min(p,q); "
              "E[tau] closed form; T=0 top-1 match",
    "residual_weights": "equal numpy max(0, softmax(lp/T) - softmax(lq/T)) at T != 1; mass = D_TV",
    "alpha_tv": "sum min(p,q) == 1 - D_TV identity; equals numpy's sums at T != 1; MC acceptance "
                "frequency",
    "confidence": "w=0 gives 1/2; one-hot weights on either block give scipy expit of that "
                  "input; c(-w) = 1 - c(w); logits add over disjoint weight supports",
    "prefix_schedule": "brute force over every length assignment on tiny cases with unimodal "
                       "throughput; admitted set is the global top-t; constant SPS admits all; "
                       "SPS that vanishes past R admits none; hand-worked example; early stop at "
                       "the first fall even when a later size would be higher",
    "verify_tree": "exact output law (draft tokens enumerated with their draft probabilities, "
                   "uniforms integrated by bisecting the oracle's monotone decisions) equals the "
                   "target's autoregressive law at every emitted position, on five tree shapes at "
                   "T = 1 and 0.7; a chain-shaped tree equals orc_verify exactly (T = 1, 0.7, 0); "
                   "T = 0 emits the target's greedy sequence; q = p passes the lowest-index child",
    "tree_select": "brute force over every prefix-closed node set of the budget on tiny trees "
                   "(the chosen set is one of them and reaches the best summed survival); chain "
                   "gives its first n nodes; star gives numpy's stable top-n of c; all-ones gives "
                   "breadth-first order; a forest of chains matches the prefix scheduler's order",
}


def build(force=False):
    """Compile liboracle.so with gcc (no fast-math, no SIMD intrinsics)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        d = ctypes.POINTER(ctypes.c_double)
        i = ctypes.POINTER(ctypes.c_int)
        u32 = ctypes.POINTER(ctypes.c_uint32)
        lib.orc_philox4x32_10.argtypes = [u32, u32, u32]
        lib.orc_philox4x32_10.restype = None
        lib.orc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_uint32, ctypes.c_uint32]
        lib.orc_uniform.restype = ctypes.c_double
        lib.orc_softmax_weights.argtypes = [d, ctypes.c_int, ctypes.c_double, d, d]
        lib.orc_softmax_weights.restype = ctypes.c_double
        lib.orc_inverse_cdf.argtypes = [d, ctypes.c_int, ctypes.c_double, ctypes.c_double, d, d]
        lib.orc_inverse_cdf.restype = ctypes.c_int
        lib.orc_cdf_interval.argtypes = [d, ctypes.c_int, ctypes.c_int, d, d]
        lib.orc_cdf_interval.restype = None
        lib.orc_argmax.argtypes = [d, ctypes.c_int, d]
        lib.orc_argmax.restype = ctypes.c_int
        lib.orc_residual_weights.argtypes = [d, d, ctypes.c_int, ctypes.c_double,
                                             ctypes.c_double, ctypes.c_double, d]
        lib.orc_residual_weights.restype = ctypes.c_double
        lib.orc_alpha_tv.argtypes = [d, d, ctypes.c_int, ctypes.c_double, d, d]
        lib.orc_alpha_tv.restype = None
        lib.orc_draft_markov.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         d, d, d, ctypes.c_int, ctypes.c_double, d, i,
                                         i, d, d, d, d, d]
        lib.orc_draft_markov.restype = ctypes.c_int
        lib.orc_draft_rnn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      d, d, d, d, d, d, d, ctypes.c_int, ctypes.c_double, d, i,
                                      i, d, d, d, d, d]
        lib.orc_draft_rnn.restype = ctypes.c_int
        lib.orc_verify.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   d, d, i, d, ctypes.c_double,
                                   i, i, d, d, d, d, d, d, i]
        lib.orc_verify.restype = ctypes.c_int
        lib.orc_verify_tree.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, i, i,
                                        d, d, d, ctypes.c_double, i, i, i, d, d, d, i, d]
        lib.orc_verify_tree.restype = ctypes.c_int
        lib.orc_confidence.argtypes = [d, ctypes.c_int, d, ctypes.c_int, d]
        lib.orc_confidence.restype = ctypes.c_double
        f = ctypes.POINTER(ctypes.c_float)
        lib.orc_prefix_schedule.argtypes = [f, ctypes.c_int, ctypes.c_int, d, ctypes.c_int, i,
                                            d, d]
        lib.orc_prefix_schedule.restype = ctypes.c_int
        lib.orc_tree_select.argtypes = [i, f, ctypes.c_int, ctypes.c_int, i, d]
        lib.orc_tree_select.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------
# Uniform stream
# --------------------------------------------------------------------------

def philox4x32_10(ctr, key):
    """Raw Philox4x32-10 block: 4 counter words, 2 key words -> 4 words."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    u32 = ctypes.POINTER(ctypes.c_uint32)
    _L().orc_philox4x32_10(c.ctypes.data_as(u32), k.ctypes.data_as(u32), out.ctypes.data_as(u32))
    return out


def uniform(seed, offset, b, k, stream):
    return _L().orc_uniform(int(seed), int(offset), int(b), int(k), int(stream))


def draft_uniforms(seed, offset, B, gamma):
    """[B, gamma] uniforms of the draft samples (stream 0)."""
    L = _L()
    out = np.empty((B, gamma), dtype=np.float64)
    for b in range(B):
        for k in range(gamma):
            out[b, k] = L.orc_uniform(seed, offset, b, k, 0)
    return out


def verify_uniforms(seed, offset, B, gamma_max):
    """[B, gamma_max + 1]: ratio-test uniforms (stream 1) at k < gamma_max
    and the final-draw uniform (stream 2, position 0) in slot gamma_max."""
    L = _L()
    out = np.empty((B, gamma_max + 1), dtype=np.float64)
    for b in range(B):
        for k in range(gamma_max):
            out[b, k] = L.orc_uniform(seed, offset, b, k, 1)
        out[b, gamma_max] = L.orc_uniform(seed, offset, b, 0, 2)
    return out


# --------------------------------------------------------------------------
# Row primitives
# --------------------------------------------------------------------------

def softmax_weights(l, T):
    """(w, Z, logZ) with w = exp(l/T - max) summed in ascending order."""
    l = _f64(l)
    w = np.empty_like(l)
    Z = ctypes.c_double()
    logZ = _L().orc_softmax_weights(_dp(l), l.size, float(T), _dp(w), ctypes.byref(Z))
    return w, Z.value, logZ


def residual_weights(lp, lq, T, logZp, logZq):
    lp, lq = _f64(lp), _f64(lq)
    w = np.empty_like(lp)
    R = _L().orc_residual_weights(_dp(lp), _dp(lq), lp.size, float(T), float(logZp),
                                  float(logZq), _dp(w))
    return w, R


def inverse_cdf(w, Z, u):
    w = _f64(w)
    thr, margin = ctypes.c_double(), ctypes.c_double()
    tok = _L().orc_inverse_cdf(_dp(w), w.size, float(Z), float(u), ctypes.byref(thr),
                               ctypes.byref(margin))
    return tok, thr.value, margin.value


def cdf_interval(w, y):
    w = _f64(w)
    lo, hi = ctypes.c_double(), ctypes.c_double()
    _L().orc_cdf_interval(_dp(w), w.size, int(y), ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def argmax(l):
    l = _f64(l)
    gap = ctypes.c_double()
    tok = _L().orc_argmax(_dp(l), l.size, ctypes.byref(gap))
    return tok, gap.value


def alpha_tv(lp, lq, T=1.0):
    lp, lq = _f64(lp), _f64(lq)
    a, t = ctypes.c_double(), ctypes.c_double()
    _L().orc_alpha_tv(_dp(lp), _dp(lq), lp.size, float(T), ctypes.byref(a), ctypes.byref(t))
    return a.value, t.value


# --------------------------------------------------------------------------
# Draft (one request) and verify (one request)
# --------------------------------------------------------------------------

def _draft_outputs(gamma, V, want_logits):
    return dict(
        tokens=np.zeros(gamma, dtype=np.int32),
        q_logits=np.zeros((gamma, V), dtype=np.float64) if want_logits else None,
        logZ=np.zeros(gamma), q_tok=np.zeros(gamma), thr=np.zeros(gamma),
        margin=np.zeros(gamma))


def draft_markov(U, W1, W2, x0, T, u, forced=None, want_logits=True):
    """One request: U [gamma, V], W1 [V, r], W2 [r, V] (float64), anchor x0,
    uniforms u [gamma].  forced: tokens that condition the next position in
    place of the oracle's own draws (replay)."""
    U, W1, W2 = _f64(U), _f64(W1), _f64(W2)
    gamma, V = U.shape
    r = W1.shape[1]
    assert W1.shape == (V, r) and W2.shape == (r, V)
    u = _f64(np.zeros(gamma) if u is None else u)
    f = None if forced is None else _i32(forced)
    o = _draft_outputs(gamma, V, want_logits)
    st = _L().orc_draft_markov(V, gamma, r, _dp(U), _dp(W1), _dp(W2), int(x0), float(T), _dp(u),
                               _ip(f) if f is not None else None, _ip(o["tokens"]),
                               _dp(o["q_logits"]) if want_logits else None,
                               _dp(o["logZ"]), _dp(o["q_tok"]), _dp(o["thr"]), _dp(o["margin"]))
    if st != 0:
        raise ValueError(f"oracle draft_markov failed with status {st}")
    # the inputs of each position's logits, for the comparison's error bound:
    # W1, W2 and the token each position conditioned on
    prev = np.concatenate([[int(x0)], (o["tokens"] if f is None else f)[: gamma - 1]])
    o["markov"] = dict(W1=W1, W2=W2, prev=prev.astype(np.int64))
    return o


def draft_rnn(U, h, W1, W2, Wg, Wc, Wo, x0, T, u, forced=None, want_logits=True):
    """One request of the RNN head: h [gamma, d]; Wg, Wc, Wo [r, 2r+d]."""
    U, h, W1, W2 = _f64(U), _f64(h), _f64(W1), _f64(W2)
    Wg, Wc, Wo = _f64(Wg), _f64(Wc), _f64(Wo)
    gamma, V = U.shape
    r = W1.shape[1]
    d = h.shape[1]
    assert Wg.shape == (r, 2 * r + d) and Wc.shape == Wg.shape and Wo.shape == Wg.shape
    u = _f64(np.zeros(gamma) if u is None else u)
    f = None if forced is None else _i32(forced)
    o = _draft_outputs(gamma, V, want_logits)
    st = _L().orc_draft_rnn(V, gamma, r, d, _dp(U), _dp(h), _dp(W1), _dp(W2), _dp(Wg), _dp(Wc),
                            _dp(Wo), int(x0), float(T), _dp(u),
                            _ip(f) if f is not None else None, _ip(o["tokens"]),
                            _dp(o["q_logits"]) if want_logits else None,
                            _dp(o["logZ"]), _dp(o["q_tok"]), _dp(o["thr"]), _dp(o["margin"]))
    if st != 0:
        raise ValueError(f"oracle draft_rnn failed with status {st}")
    return o


def verify(P, Q, draft, T, u_test, u_final):
    """One request with L = len(draft): P [L+1, V], Q [L, V] logits."""
    P = _f64(P)
    L = len(draft)
    V = P.shape[1]
    Q = _f64(Q) if L > 0 else np.zeros((1, V))
    assert P.shape == (L + 1, V)
    dr = _i32(draft) if L > 0 else np.zeros(1, dtype=np.int32)
    ut = _f64(u_test) if L > 0 else np.zeros(1)
    n = ctypes.c_int()
    out = np.zeros(L + 1, dtype=np.int32)
    logZp = np.zeros(L + 1)
    logZq = np.zeros(max(L, 1))
    ap = np.zeros(max(L, 1))
    tm = np.zeros(max(L, 1))
    fthr, fmar = ctypes.c_double(), ctypes.c_double()
    fb = ctypes.c_int()
    st = _L().orc_verify(V, L, float(T), _dp(P), _dp(Q), _ip(dr), _dp(ut), float(u_final),
                         ctypes.byref(n), _ip(out), _dp(logZp), _dp(logZq), _dp(ap), _dp(tm),
                         ctypes.byref(fthr), ctypes.byref(fmar), ctypes.byref(fb))
    if st != 0:
        raise ValueError(f"oracle verify failed with status {st}")
    return dict(n=n.value, out=out, logZp=logZp, logZq=logZq[:L], accept_prob=ap[:L],
                test_margin=tm[:L], final_thr=fthr.value, final_margin=fmar.value,
                fallback=fb.value)


def tree_uniforms(seed, offset, B, M):
    """[B, M + 1]: the ratio-test uniform of node v (stream 3, index v) at
    v < M and the final-draw uniform (stream 3, index M) in slot M."""
    L = _L()
    out = np.empty((B, M + 1), dtype=np.float64)
    for b in range(B):
        for v in range(M + 1):
            out[b, v] = L.orc_uniform(seed, offset, b, v, 3)
    return out


def verify_tree(P, Q, parent, tok, T, u_node, u_final, want_weights=False):
    """One request's tree: P, Q [M + 1, V] logits (row 0 the root, row 1 + v
    node v), parent [M] (parents first, -1 = child of the root), tok [M]
    draft tokens, u_node [M] ratio-test uniforms, u_final.  Returns None for
    an invalid tree or token."""
    P, Q = _f64(P), _f64(Q)
    par, tk = _i32(parent), _i32(tok)
    M = len(par)
    V = P.shape[1]
    assert P.shape == (M + 1, V) and Q.shape == (M + 1, V) and len(tk) == M
    un = _f64(u_node) if M > 0 else np.zeros(1)
    n = ctypes.c_int()
    path = np.zeros(max(M, 1), dtype=np.int32)
    out = np.zeros(M + 1, dtype=np.int32)
    ratio = np.zeros(max(M, 1))
    fthr, fmar = ctypes.c_double(), ctypes.c_double()
    fb = ctypes.c_int()
    fw = np.zeros(V) if want_weights else None
    st = _L().orc_verify_tree(V, M, float(T), _ip(par if M else np.zeros(1, np.int32)),
                              _ip(tk if M else np.zeros(1, np.int32)), _dp(P), _dp(Q), _dp(un),
                              float(u_final), ctypes.byref(n), _ip(path), _ip(out), _dp(ratio),
                              ctypes.byref(fthr), ctypes.byref(fmar), ctypes.byref(fb),
                              _dp(fw) if want_weights else None)
    if st == -1:
        return None
    if st != 0:
        raise ValueError(f"oracle verify_tree failed with status {st}")
    return dict(n=n.value, path=path[:M], out=out, test_ratio=ratio[:M], final_thr=fthr.value,
                final_margin=fmar.value, fallback=fb.value, final_w=fw)


# --------------------------------------------------------------------------
# Confidence head and hardware-aware prefix scheduler (DSpark §2.1-2.2)
# --------------------------------------------------------------------------

def confidence(h, e, w):
    """c = sigmoid(w . [h; e]) for one drafted position (fp64)."""
    h, e, w = _f64(h), _f64(e), _f64(w)
    if w.size != h.size + e.size:
        raise ValueError("w must have len(h) + len(e) weights")
    return _L().orc_confidence(_dp(h), h.size, _dp(e), e.size, _dp(w))


def prefix_schedule(c, sps):
    """Acceptance lengths l [R] (int32), the chosen batch size B and expected
    accepted count tau from confidences c [R, gamma] (float32) and the
    steps-per-second table sps[B]."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    R, gamma = c.shape
    sps = _f64(sps)
    lens = np.zeros(R, dtype=np.int32)
    B, tau = ctypes.c_double(), ctypes.c_double()
    st = _L().orc_prefix_schedule(c.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), R, gamma,
                                  _dp(sps), sps.size, _ip(lens), ctypes.byref(B),
                                  ctypes.byref(tau))
    if st != 0:
        raise MemoryError("orc_prefix_schedule")
    return lens, int(B.value), tau.value


def tree_select(parent, c, n):
    """Top-n nodes of one draft tree by survival probability: (sel int32 [n],
    score).  parent int32 [M] with parent[v] in [-1, v); c float32 [M]."""
    parent = _i32(parent)
    c = np.ascontiguousarray(c, dtype=np.float32)
    M = parent.size
    sel = np.full(max(n, 0), -1, dtype=np.int32)
    score = ctypes.c_double()
    st = _L().orc_tree_select(_ip(parent), c.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), M,
                              n, _ip(sel), ctypes.byref(score))
    if st != 0:
        return sel, float("nan")
    return sel, score.value
