"""Seeded synthetic workloads for draft sampling and verification.

Recipe (stated here once; used identically by tests and benchmark):

* numpy PCG64 streams keyed by ``SeedSequence([data_seed, stream_id, b])``
  so any single request can be regenerated on its own.
* base logits ``G[b, k, v] = scale * N(0, 1) - s * ln(v + 1)`` (a Zipf(s)
  rank bias over token ids, rank = id + 1), ``k = 0..gamma`` (gamma + 1 rows).
* draft base logits ``U[b, k] = G[b, k]`` for ``k < gamma``.
* target logits ``P[b, k] = G[b, k] + sigma_b * N(0, 1)`` for ``k <= gamma``
  (the bonus row is ``G[b, gamma]`` plus noise).
* weights ``W ~ N(0, w_std**2)``; anchors ``x0 ~ U{0..V-1}``.
* ragged lengths ``L_b ~ U{1..gamma}`` and ``sigma_b ~ U(sigma_lo, sigma_hi)``.
* values are drawn in fp32 and rounded to bf16 (round to nearest even) where
  a workload says bf16; bf16 tensors are carried as uint16 bit patterns.

No public benchmark, dataset or trained weight is used: these synthetic
logits stand in for the evaluation suites the pages measure on.
"""
import numpy as np

# Named workloads.  Sizes follow the pages' settings: gamma (block size k),
# Markov rank r = 256, a vocabulary pruned to 32000 (H-Spec review, Appx. B.1
# settings) and a 151936-token vocabulary at concurrency up to 128.
CONFIGS = {
    "markov-tiny": dict(head="markov", B=1, gamma=4, V=1000, r=16, logit_dtype="f32",
                        w_dtype="f32", scale=3.0, zipf=1.1, sigma=0.5, w_std=0.02, T=1.0,
                        data_seed=1001),
    "markov-32k-b32": dict(head="markov", B=32, gamma=7, V=32000, r=256, logit_dtype="f32",
                           w_dtype="bf16", scale=4.0, zipf=1.1, sigma=0.85, w_std=0.02,
                           T=1.0, data_seed=1002),
    "markov-152k-b128": dict(head="markov", B=128, gamma=16, V=151936, r=256,
                             logit_dtype="bf16", w_dtype="bf16", scale=4.0, zipf=1.1,
                             sigma=1.0, w_std=0.02, T=1.0, data_seed=1003),
    "rnn-32k-b64": dict(head="rnn", B=64, gamma=8, V=32000, r=256, d=4096, logit_dtype="f32",
                        w_dtype="bf16", h_dtype="bf16", scale=3.0, zipf=1.1, sigma=0.5,
                        w_std=0.02, T=1.0, data_seed=1004),
    "ragged-128k-b256": dict(head="markov", B=256, gamma=16, V=128256, r=256,
                             logit_dtype="bf16", w_dtype="bf16", scale=4.0, zipf=1.1,
                             sigma=None, sigma_range=(0.2, 1.5), ragged=True, w_std=0.02,
                             T=1.0, data_seed=1005),
}

# Stream ids of the seed sequences.
_S_WEIGHTS, _S_LOGITS, _S_GLOBAL, _S_HIDDEN = 0, 1, 2, 3


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact decode of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(arr, dtype):
    """Exact float64 view of an input carried as fp32 or as bf16 bits."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x32, dtype):
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _rng(data_seed, stream, idx=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([data_seed, stream, idx])))


def _zipf_bias(V, s):
    return (-s * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)


def packed_offsets(lens):
    """Row offsets of a packed layout with lens[b] rows for request b."""
    lens = np.asarray(lens, dtype=np.int64)
    off = np.zeros(len(lens), dtype=np.int64)
    if len(lens) > 1:
        off[1:] = np.cumsum(lens)[:-1]
    return off


def _globals(cfg, B, V):
    g = _rng(cfg["data_seed"], _S_GLOBAL)
    x0 = g.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    gamma = cfg["gamma"]
    if cfg.get("ragged"):
        lens = g.integers(1, gamma + 1, size=B, dtype=np.int64).astype(np.int32)
        lo, hi = cfg["sigma_range"]
        sig = g.uniform(lo, hi, size=B)
    else:
        lens = None
        sig = np.full(B, cfg["sigma"], dtype=np.float64)
    return x0, lens, sig


def _logits(cfg, B, V, gamma, sig, lens, requests):
    """U [B, gamma, V] and P (dense [B, gamma+1, V] or packed) in storage form."""
    zb = _zipf_bias(V, cfg["zipf"])
    dt = cfg["logit_dtype"]
    nb = len(requests)
    store_dtype = np.uint16 if dt == "bf16" else np.float32
    U = np.empty((nb, gamma, V), dtype=store_dtype)
    if lens is None:
        P = np.empty((nb, gamma + 1, V), dtype=store_dtype)
    else:
        rows = int(sum(int(lens[b]) + 1 for b in requests))
        P = np.empty((rows, V), dtype=store_dtype)
    prow = 0
    for i, b in enumerate(requests):
        g = _rng(cfg["data_seed"], _S_LOGITS, b)
        G = g.standard_normal((gamma + 1, V), dtype=np.float32)
        G *= np.float32(cfg["scale"])
        G += zb
        noise = g.standard_normal((gamma + 1, V), dtype=np.float32)
        U[i] = _store(G[:gamma], dt)
        Pb = G + np.float32(sig[b]) * noise
        if lens is None:
            P[i] = _store(Pb, dt)
        else:
            n = int(lens[b]) + 1
            P[prow:prow + n] = _store(Pb[:n], dt)
            prow += n
    return U, P


def make_markov(cfg, B=None, V=None, gamma=None, r=None, requests=None, T=None):
    """Markov-head draft + verify workload.  Overrides shrink a named config
    for small parity cases; ``requests`` regenerates a subset of requests
    (their logits are identical to those of the full workload)."""
    cfg = dict(cfg)
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    gamma = cfg["gamma"] if gamma is None else gamma
    r = cfg["r"] if r is None else r
    cfg["gamma"] = gamma
    requests = list(range(B)) if requests is None else list(requests)
    x0, lens, sig = _globals(cfg, B, V)
    gw = _rng(cfg["data_seed"], _S_WEIGHTS)
    ws = np.float32(cfg["w_std"])
    W1 = _store(gw.standard_normal((V, r), dtype=np.float32) * ws, cfg["w_dtype"])
    W2 = _store(gw.standard_normal((r, V), dtype=np.float32) * ws, cfg["w_dtype"])
    U, P = _logits(cfg, B, V, gamma, sig, lens, requests)
    sel = np.asarray(requests, dtype=np.int64)
    return dict(head="markov", B=len(requests), gamma=gamma, V=V, r=r,
                logit_dtype=cfg["logit_dtype"], w_dtype=cfg["w_dtype"],
                T=cfg["T"] if T is None else T, U=U, P=P, W1=W1, W2=W2,
                x0=x0[sel], lens=None if lens is None else lens[sel], sigma=sig[sel],
                requests=requests)


def make_rnn(cfg, B=None, V=None, gamma=None, r=None, d=None, requests=None, T=None):
    """RNN-head draft + verify workload (adds h and the gate matrices)."""
    cfg = dict(cfg)
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    gamma = cfg["gamma"] if gamma is None else gamma
    r = cfg["r"] if r is None else r
    d = cfg["d"] if d is None else d
    cfg["gamma"] = gamma
    requests = list(range(B)) if requests is None else list(requests)
    x0, lens, sig = _globals(cfg, B, V)
    gw = _rng(cfg["data_seed"], _S_WEIGHTS)
    ws = np.float32(cfg["w_std"])
    wd = cfg["w_dtype"]
    W1 = _store(gw.standard_normal((V, r), dtype=np.float32) * ws, wd)
    W2 = _store(gw.standard_normal((r, V), dtype=np.float32) * ws, wd)
    Wg = _store(gw.standard_normal((r, 2 * r + d), dtype=np.float32) * ws, wd)
    Wc = _store(gw.standard_normal((r, 2 * r + d), dtype=np.float32) * ws, wd)
    Wo = _store(gw.standard_normal((r, 2 * r + d), dtype=np.float32) * ws, wd)
    hd = cfg.get("h_dtype", "bf16")
    H = np.empty((len(requests), gamma, d), dtype=np.uint16 if hd == "bf16" else np.float32)
    for i, b in enumerate(requests):
        gh = _rng(cfg["data_seed"], _S_HIDDEN, b)
        H[i] = _store(gh.standard_normal((gamma, d), dtype=np.float32), hd)
    U, P = _logits(cfg, B, V, gamma, sig, lens, requests)
    sel = np.asarray(requests, dtype=np.int64)
    return dict(head="rnn", B=len(requests), gamma=gamma, V=V, r=r, d=d,
                logit_dtype=cfg["logit_dtype"], w_dtype=wd, h_dtype=hd,
                T=cfg["T"] if T is None else T, U=U, P=P, W1=W1, W2=W2, Wg=Wg, Wc=Wc, Wo=Wo,
                H=H, x0=x0[sel], lens=None if lens is None else lens[sel], sigma=sig[sel],
                requests=requests)


def make_verify_only(B, gamma, V, seed, dtype="f32", scale=4.0, zipf=1.1, sigma=1.0,
                     lens=None):
    """Target and draft logits plus draft tokens drawn uniformly at random,
    for verification tests that do not run a draft."""
    cfg = dict(data_seed=seed, scale=scale, zipf=zipf, logit_dtype=dtype, gamma=gamma)
    sig = np.full(B, sigma)
    U, P = _logits(cfg, B, V, gamma, sig, lens, list(range(B)))
    g = _rng(seed, _S_GLOBAL, 7)
    draft = g.integers(0, V, size=(B, gamma), dtype=np.int64).astype(np.int32)
    return dict(B=B, gamma=gamma, V=V, logit_dtype=dtype, Q=U, P=P, draft=draft, lens=lens)


# Stream ids of the confidence-head and scheduler inputs.
_S_CONF, _S_SCHED, _S_TREE = 4, 5, 6


def make_confidence(R, gamma, V, r, d, seed, h_dtype="bf16", w_dtype="bf16", w_std=0.02,
                    z_std=1.5):
    """Confidence-head inputs: hidden states h ~ N(0, 1) [R, gamma, d], an
    embedding table W1 ~ N(0, w_std^2) [V, r], anchors and draft tokens
    uniform on [0, V), and fp32 head weights w [d + r] scaled so that each
    block's dot product has standard deviation about z_std / sqrt(2)."""
    g = _rng(seed, _S_CONF)
    h = _store(g.standard_normal((R, gamma, d), dtype=np.float32), h_dtype)
    W1 = _store(g.standard_normal((V, r), dtype=np.float32) * np.float32(w_std), w_dtype)
    x0 = g.integers(0, V, size=R, dtype=np.int64).astype(np.int32)
    draft = g.integers(0, V, size=(R, gamma), dtype=np.int64).astype(np.int32)
    s = z_std / np.sqrt(2.0)
    w = np.concatenate([g.standard_normal(d) * (s / np.sqrt(d)),
                        g.standard_normal(r) * (s / (np.sqrt(r) * w_std))]).astype(np.float32)
    return dict(R=R, gamma=gamma, V=V, r=r, d=d, h_dtype=h_dtype, w_dtype=w_dtype, h=h, W1=W1,
                x0=x0, draft=draft, w=w)


def make_schedule(R, gamma, seed, knee=None, beta=(4.0, 1.2)):
    """Scheduler inputs: confidences c ~ Beta(beta) in fp32 [R, gamma] (mean
    about 0.77), and a steps-per-second table over batch sizes
    B = 0 .. R (gamma + 1) of an engine whose step time is flat up to `knee`
    tokens (memory-bound) and grows linearly beyond it (compute-bound):
    sps(B) = 1 / (1 + max(0, B - knee) / knee)."""
    g = _rng(seed, _S_SCHED)
    c = g.beta(beta[0], beta[1], size=(R, gamma)).astype(np.float32)
    knee = 4 * R if knee is None else knee
    B = np.arange(R * (gamma + 1) + 1, dtype=np.float64)
    sps = 1.0 / (1.0 + np.maximum(0.0, B - knee) / knee)
    return dict(R=R, gamma=gamma, c=c, sps=sps, knee=knee)


def make_trees(R, M, seed, levels=16, beta=(4.0, 1.2)):
    """Candidate draft trees in breadth-first order (parents first): M nodes
    spread evenly over `levels` depths (a block of gamma positions, each a few
    dozen candidates wide); a node's parent is uniform over the nodes one
    level up (the root for the first level); acceptance chances
    c ~ Beta(beta) in fp32."""
    g = _rng(seed, _S_TREE)
    bounds = [(M * d) // levels for d in range(levels + 1)]
    parent = np.empty((R, M), dtype=np.int32)
    for d in range(levels):
        lo, hi = bounds[d], bounds[d + 1]
        if d == 0:
            parent[:, lo:hi] = -1
        else:
            plo, phi = bounds[d - 1], bounds[d]
            parent[:, lo:hi] = g.integers(plo, max(phi, plo + 1), size=(R, hi - lo)) if phi > plo else -1
    c = g.beta(beta[0], beta[1], size=(R, M)).astype(np.float32)
    return dict(R=R, M=M, parent=parent, c=c)


# Stream id of the repeated-request workload.
_S_REPEAT = 7


def make_repeated_markov(B, gamma, V, r, seed, scale=2.0, sigma=1.0, w_std=0.3, w1_zero=False,
                         dtype="bf16"):
    """One request's logits repeated over a batch of B requests, for statistical
    checks that use the batch as the trial axis: draft base logits
    U[k] = scale * N(0, 1) (k < gamma), target logits P[k] = U[k] + sigma *
    N(0, 1) (k < gamma) and P[gamma] = scale * N(0, 1), identical in every row;
    W1 [V, r] and W2 [r, V] ~ N(0, w_std**2) (W1 all zero with w1_zero, so the
    draft rows do not depend on the previous token); anchors x0 ~ U{0..V-1}
    per row.  Logits and weights are rounded to bf16 (dtype "bf16")."""
    g = _rng(seed, _S_REPEAT)
    U1 = (scale * g.standard_normal((gamma, V))).astype(np.float32)
    P1 = np.empty((gamma + 1, V), dtype=np.float32)
    P1[:gamma] = U1 + (sigma * g.standard_normal((gamma, V))).astype(np.float32)
    P1[gamma] = (scale * g.standard_normal(V)).astype(np.float32)
    W1 = (w_std * g.standard_normal((V, r))).astype(np.float32)
    if w1_zero:
        W1[:] = 0.0
    W2 = (w_std * g.standard_normal((r, V))).astype(np.float32)
    x0 = g.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    U = np.broadcast_to(U1, (B, gamma, V))
    P = np.broadcast_to(P1, (B, gamma + 1, V))
    return dict(B=B, gamma=gamma, V=V, r=r, logit_dtype=dtype, w_dtype=dtype,
                U=_store(np.ascontiguousarray(U), dtype), P=_store(np.ascontiguousarray(P), dtype),
                W1=_store(W1, dtype), W2=_store(W2, dtype), x0=x0,
                U1=_store(U1, dtype), P1=_store(P1, dtype))


# Stream id of the tree-verification workload.
_S_TREEV = 8


def make_tree_verify(B, M, V, seed, dtype="bf16", scale=4.0, zipf=1.1, sigma=1.0, levels=4,
                     n_nodes=False):
    """Tree drafts with their logit rows: per request, M nodes parents first
    over `levels` depths (a node's parent uniform over the level above, the
    root for the first level), one Zipf+Gaussian draft row Q per node (row 0
    the root, row 1 + v node v; the recipe of the chain workloads) and a target
    row P = Q + sigma * N(0, 1); random draft tokens (tests replace them with
    draws from the parent's draft row); with n_nodes, a count of nodes in use
    uniform on 0..M."""
    g = _rng(seed, _S_TREEV)
    zb = _zipf_bias(V, zipf)
    bounds = [(M * d) // levels for d in range(levels + 1)]
    parent = np.empty((B, M), dtype=np.int32)
    for d in range(levels):
        lo, hi = bounds[d], bounds[d + 1]
        if d == 0 or bounds[d - 1] == bounds[d]:
            parent[:, lo:hi] = -1
        else:
            parent[:, lo:hi] = g.integers(bounds[d - 1], bounds[d], size=(B, hi - lo))
    Q = np.empty((B, M + 1, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    P = np.empty_like(Q)
    for b in range(B):
        gb = _rng(seed, _S_TREEV, b + 1)
        G = gb.standard_normal((M + 1, V), dtype=np.float32) * np.float32(scale) + zb
        Q[b] = _store(G, dtype)
        P[b] = _store(G + np.float32(sigma) * gb.standard_normal((M + 1, V), dtype=np.float32), dtype)
    tok = g.integers(0, V, size=(B, M), dtype=np.int64).astype(np.int32)
    nn = g.integers(0, M + 1, size=B, dtype=np.int64).astype(np.int32) if n_nodes else None
    return dict(B=B, M=M, V=V, logit_dtype=dtype, parent=parent, P=P, Q=Q, tokens=tok, n_nodes=nn)
