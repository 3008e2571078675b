"""GPU parity of tree verification (spec_verify_tree) against the oracle's
recursive rejection over siblings, request by request with the band rule:
dense trees over several depths (f32 / bf16 rows, T = 1, 0.7, 1.3, 0), a
ragged vocabulary, caller uniforms, nodes in use per request (empty trees
draw the bonus from the root), invalid trees, and a 151936-token vocabulary;
plus a statistical check that the emitted tokens of the root follow p."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _softmax(l, T):
    z = np.asarray(l, dtype=np.float64) / T
    z -= z.max()
    w = np.exp(z)
    return w / w.sum()


def _drawn_tokens(orc, wl, T, rng, random_frac=0.2):
    """Each node's token drawn by the oracle from its parent's draft row (a
    share of random tokens, mostly rejected)."""
    B, M = wl["B"], wl["M"]
    dt = wl["logit_dtype"]
    tok = wl["tokens"].copy()
    for b in range(B):
        Qf = workloads.as_f64(wl["Q"][b], dt)
        for v in range(M):
            if rng.random() < random_frac:
                continue
            row = Qf[wl["parent"][b, v] + 1]
            if T == 0:
                tok[b, v] = orc.argmax(row)[0] if rng.random() < 0.7 else tok[b, v]
            else:
                w, Z, _ = orc.softmax_weights(row, T)
                tok[b, v] = orc.inverse_cdf(w, Z, rng.random())[0]
    return tok


def _run(sd, wl, tok, T, seed, uniforms=None, n_nodes=None, parent=None):
    dt = wl["logit_dtype"]
    par = wl["parent"] if parent is None else parent
    g = sd.spec_verify_tree(dev(wl["P"], dt), dev(wl["Q"], dt), dev(par), dev(tok), T,
                            n_nodes=None if n_nodes is None else dev(n_nodes),
                            uniforms=None if uniforms is None else dev(uniforms.astype(np.float32)),
                            seed=seed, offset=5)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _compare_all(orc, wl, tok, T, g, u, what, n_nodes=None, parent=None):
    dt = wl["logit_dtype"]
    par = wl["parent"] if parent is None else parent
    M = wl["M"]
    tally = compare.Tally()
    for b in range(wl["B"]):
        nb = M if n_nodes is None else int(n_nodes[b])
        P = workloads.as_f64(wl["P"][b], dt)
        Q = workloads.as_f64(wl["Q"][b], dt)
        gb = dict(accepted=g["accepted"][b], out_tokens=g["out_tokens"][b], path=g["path"][b])
        if n_nodes is not None:
            # nodes past n are not in the tree: compare against the oracle on the first n
            gb = dict(accepted=gb["accepted"], out_tokens=gb["out_tokens"][: nb + 1],
                      path=gb["path"][:nb])
        compare.compare_tree_request(P[: nb + 1], Q[: nb + 1], par[b, :nb], tok[b, :nb], T,
                                     u[b, :nb], u[b, M], gb, f"{what} b={b}", tally)
        if n_nodes is not None:
            assert np.all(g["out_tokens"][b, nb + 1:] == -1)
    return tally


@pytest.mark.parametrize("pdt,qdt_same,V,T,sigma", [
    ("f32", True, 3000, 1.0, 0.8), ("bf16", True, 4099, 0.7, 0.5), ("bf16", True, 5000, 1.3, 1.2),
    ("f32", True, 257, 1.0, 0.3), ("bf16", True, 3000, 0.0, 0.5), ("f32", True, 20000, 1.0, 1.5)])
def test_tree_verify_parity(orc, pdt, qdt_same, V, T, sigma):
    sd = require_gpu()
    B, M = 24, 14
    note(f"tree verify B={B} M={M} V={V} dtype={pdt} T={T} sigma={sigma}")
    wl = workloads.make_tree_verify(B, M, V, seed=300 + V, dtype=pdt, sigma=sigma, levels=4)
    tok = _drawn_tokens(orc, wl, T, np.random.default_rng(V))
    seed = 77
    g = _run(sd, wl, tok, T, seed)
    u = orc.tree_uniforms(seed, 5, B, M)
    tally = _compare_all(orc, wl, tok, T, g, u, f"V={V} T={T}")
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert g["accepted"].max() > 0


def test_tree_verify_mixed_dtypes_and_uniforms(orc):
    sd = require_gpu()
    B, M, V = 16, 10, 2000
    note(f"tree verify mixed dtypes, caller uniforms B={B} M={M} V={V}")
    wl = workloads.make_tree_verify(B, M, V, seed=41, dtype="bf16", sigma=0.6, levels=3)
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(4))
    rng = np.random.default_rng(9)
    u = rng.random((B, M + 1)).astype(np.float32).astype(np.float64)
    Qf32 = workloads.bf16_bits_to_f32(wl["Q"])
    g = sd.spec_verify_tree(dev(wl["P"], "bf16"), dev(Qf32), dev(wl["parent"]), dev(tok), 1.0,
                            uniforms=dev(u.astype(np.float32)))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    tally = _compare_all(orc, wl, tok, 1.0, g, u, "mixed")
    note(f"  {tally.as_dict()}")


def test_tree_verify_nodes_in_use_and_invalid(orc):
    sd = require_gpu()
    B, M, V = 20, 9, 1500
    note(f"tree verify ragged node counts and invalid trees B={B} M={M} V={V}")
    wl = workloads.make_tree_verify(B, M, V, seed=52, dtype="f32", sigma=0.7, levels=3,
                                    n_nodes=True)
    nn = wl["n_nodes"].copy()
    nn[0] = 0            # an empty tree: the bonus from the root
    nn[1] = M
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(5))
    parent = wl["parent"].copy()
    # invalid requests: a parent at or after its node, a token out of range,
    # a node count above M (each only within the nodes in use)
    nn[2] = M
    parent[2, 5] = 7
    nn[3] = M
    tok[3, 4] = V
    nn[4] = M + 1
    g = _run(sd, wl, tok, 1.0, 3, n_nodes=nn, parent=parent)
    u = orc.tree_uniforms(3, 5, B, M)
    for b in (2, 3, 4):
        assert g["accepted"][b] == -1 and np.all(g["out_tokens"][b] == -1), b
    assert g["accepted"][0] == 0 and g["out_tokens"][0, 0] >= 0
    nn_ok = nn.copy()
    keep = [b for b in range(B) if b not in (2, 3, 4)]
    sub = dict(wl, B=len(keep), P=wl["P"][keep], Q=wl["Q"][keep])
    gk = {k: v[keep] for k, v in g.items()}
    _compare_all(orc, sub, tok[keep], 1.0, gk, u[keep], "ragged", n_nodes=nn_ok[keep],
                 parent=parent[keep])


def test_tree_verify_large_vocab_sampled(orc):
    sd = require_gpu()
    B, M, V = 8, 16, 151936
    note(f"tree verify B={B} M={M} V={V} bf16")
    wl = workloads.make_tree_verify(B, M, V, seed=61, dtype="bf16", sigma=1.0, levels=4)
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(6))
    g = _run(sd, wl, tok, 1.0, 12)
    u = orc.tree_uniforms(12, 5, B, M)
    tally = _compare_all(orc, wl, tok, 1.0, g, u, "V=151936")
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")


def test_tree_verify_root_token_law(orc):
    """One tree repeated over 8192 requests: the first emitted token follows p
    of the root (chi-square, p > 1e-4), and not the draft law (p < 1e-8)."""
    st = pytest.importorskip("scipy.stats")
    sd = require_gpu()
    B, V = 8192, 64
    parent = np.array([-1, -1, -1, 0, 0, 1], dtype=np.int32)
    M = len(parent)
    rng = np.random.default_rng(17)
    Qr = 1.5 * rng.standard_normal((M + 1, V))
    Pr = Qr + 1.0 * rng.standard_normal((M + 1, V))
    # each request draws its own node tokens from its parent's draft row
    tok = np.empty((B, M), dtype=np.int32)
    for v in range(M):
        tok[:, v] = rng.choice(V, size=B, p=_softmax(Qr[parent[v] + 1], 1.0))
    P = np.broadcast_to(Pr.astype(np.float32), (B, M + 1, V)).copy()
    Q = np.broadcast_to(Qr.astype(np.float32), (B, M + 1, V)).copy()
    g = sd.spec_verify_tree(dev(P), dev(Q), dev(np.broadcast_to(parent, (B, M)).copy()), dev(tok),
                            1.0, seed=2026)
    torch.cuda.synchronize()
    first = g["out_tokens"][:, 0].cpu().numpy()
    counts = np.bincount(first, minlength=V).astype(np.float64)

    def pval(law):
        e = B * law
        keep = e >= 5
        c = np.append(counts[keep], counts[~keep].sum())
        e = np.append(e[keep], e[~keep].sum())
        return float(st.chi2.sf(((c - e) ** 2 / e).sum(), df=len(c) - 1))

    p_target = pval(_softmax(Pr[0].astype(np.float32).astype(np.float64), 1.0))
    p_draft = pval(_softmax(Qr[0].astype(np.float32).astype(np.float64), 1.0))
    note(f"  root token vs p: {p_target:.3g}; vs q: {p_draft:.3g}; "
         f"mean accepted {g['accepted'].float().mean().item():.3f}")
    assert p_target > 1e-4
    assert p_draft < 1e-8


def test_tree_verify_bench_shape_split(orc):
    """The bench's tree workload (32 trees x 16 nodes x 151936 tokens, bf16):
    eight workgroups per request on a 256-CU device, every request against the
    oracle."""
    sd = require_gpu()
    B, M, V = 32, 16, 151936
    note(f"tree verify split walk B={B} M={M} V={V} bf16")
    wl = workloads.make_tree_verify(B, M, V, seed=1234, dtype="bf16", sigma=1.0, levels=4)
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(9))
    g = _run(sd, wl, tok, 1.0, 31)
    u = orc.tree_uniforms(31, 5, B, M)
    tally = _compare_all(orc, wl, tok, 1.0, g, u, "bench shape")
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert g["accepted"].min() >= 0


def test_tree_verify_split_gives_up_cleanly(orc):
    """With a wait limit of two polls (set from the host) the split walk's
    exchanges give up: the launch still ends, every request is either valid
    (and agrees with the oracle) or reports accepted -1 with all-(-1) outputs,
    and the next call with the default limit agrees with the oracle again."""
    sd = require_gpu()
    B, M, V = 16, 12, 40000
    note(f"tree verify split walk, wait limit 2: B={B} M={M} V={V}")
    wl = workloads.make_tree_verify(B, M, V, seed=77, dtype="bf16", sigma=0.8, levels=3)
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(3))
    u = orc.tree_uniforms(8, 5, B, M)
    try:
        sd.spec_draft_set_poll_limit(2)
        bad = _run(sd, wl, tok, 1.0, 8)
    finally:
        sd.spec_draft_set_poll_limit(0)
    again = _run(sd, wl, tok, 1.0, 8)
    gave_up = bad["accepted"] == -1
    note(f"  requests that gave up: {int(gave_up.sum())} of {B}")
    assert np.all(bad["out_tokens"][gave_up] == -1)
    assert np.all(bad["path"][gave_up] == -1)
    keep = np.flatnonzero(~gave_up)
    if len(keep):
        sub = dict(wl, B=len(keep), P=wl["P"][keep], Q=wl["Q"][keep], parent=wl["parent"][keep])
        gk = {k: v[keep] for k, v in bad.items()}
        _compare_all(orc, sub, tok[keep], 1.0, gk, u[keep], "kept")
    tally = _compare_all(orc, wl, tok, 1.0, again, u, "again")
    assert again["accepted"].min() >= 0
    note(f"  again: {tally.as_dict()}")


def test_tree_verify_split_graph_replays(orc):
    """The split walk captured in a HIP graph and replayed three times, with
    direct calls on other uniforms between the replays: every replay and every
    direct call gives the direct call's result for its uniforms (each split
    call leaves the exchange area zeroed for the next, so a replay cannot see
    words of the one before), and the first agrees with the oracle."""
    sd = require_gpu()
    B, M, V = 16, 12, 40000
    note(f"tree verify split walk under graph replay: B={B} M={M} V={V}")
    wl = workloads.make_tree_verify(B, M, V, seed=91, dtype="bf16", sigma=0.8, levels=3)
    tok = _drawn_tokens(orc, wl, 1.0, np.random.default_rng(4))
    Pd, Qd = dev(wl["P"], "bf16"), dev(wl["Q"], "bf16")
    pard, tokd = dev(wl["parent"]), dev(tok)

    def call(seed, out=None):
        return sd.spec_verify_tree(Pd, Qd, pard, tokd, 1.0, seed=seed, offset=5, out=out)

    def host_of(g):
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in g.items()}

    want_a = host_of(call(21))
    want_b = host_of(call(22))
    _compare_all(orc, wl, tok, 1.0, want_a, orc.tree_uniforms(21, 5, B, M), "direct")
    out = {k: torch.empty((B,) if k == "accepted" else (B, M + (k == "out_tokens")),
                          dtype=torch.int32, device="cuda") for k in ("accepted", "out_tokens", "path")}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(21, out)   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(21, out)
    for rep in range(3):
        for v in out.values():
            v.fill_(-7)
        graph.replay()
        got = host_of(out)
        for k in want_a:
            assert np.array_equal(got[k], want_a[k]), (rep, k)
        between = host_of(call(22))
        for k in want_b:
            assert np.array_equal(between[k], want_b[k]), (rep, k)
