"""GPU parity of the timed q-free cycle at the size and in the launch
configuration the benchmark times, and of the edge paths around it.

* The whole batch (B = 128 or 64, gamma = 16, V = 151936, r = 256, bf16) runs
  the persistent draft (plain launch, W2 packed once) and spec_verify_markov
  exactly as one benchmark step does; six requests spread over both 64-row
  blocks are compared with the oracle's draft and verification of the same
  request, and every request is checked for the properties that hold at any
  size (tokens in range, 0 <= n <= gamma, -1 tail, completion word 0).
* The zero-mass residual fallback ([VESSL] "수락 규칙": after a rejection the
  residual max(0, p - q) has mass 1 - beta > 0 in exact arithmetic; a draw
  whose residual rounds to zero samples p_n instead) is driven by crafted
  rows and caller uniforms on both verification entry points.
* Outputs and workspaces the binding allocates belong to the stream the
  library runs on, so a call on a side stream is not disturbed by
  allocations on the main stream.
"""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu

NEG_INF_BF16 = np.uint16(0xFF80)


def _weights(wl):
    return workloads.as_f64(wl["W1"], "bf16"), workloads.as_f64(wl["W2"], "bf16")


@pytest.mark.parametrize("B,sigma,sample", [
    (128, 1.0, [0, 21, 63, 64, 100, 127]),
    (128, 0.3, [1, 40, 62, 65, 90, 126]),
    (64, 1.0, [0, 13, 31, 32, 50, 63]),
])
def test_qfree_cycle_timed_shape(orc, B, sigma, sample):
    sd = require_gpu()
    G, V, r, T = 16, 151936, 256, 1.0
    note(f"q-free cycle at the timed shape B={B} gamma={G} V={V} r={r} sigma={sigma}")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    cfg["sigma"] = sigma
    wl = workloads.make_markov(cfg, B=B)
    U, P = dev(wl["U"], "bf16"), dev(wl["P"], "bf16")
    W1d, x0 = dev(wl["W1"], "bf16"), dev(wl["x0"])
    was = sd.spec_draft_set_persistent(1)
    try:
        W2T = sd.spec_pack_w2(dev(wl["W2"], "bf16"))
        ws_d = torch.empty(sd.workspace_bytes("markov", B=B, gamma=G, V=V, r=r),
                           dtype=torch.uint8, device="cuda")
        ws_v = torch.empty(sd.workspace_bytes("verify_markov", B=B, gamma_max=G, V=V, r=r),
                           dtype=torch.uint8, device="cuda")
        status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        seed, step = 0, 3        # the benchmark's seed; its offset is the step index
        sd.spec_profile_enable("draft_persist")
        dr = sd.spec_draft_sample_markov(U, x0, W1d, None, T, W2T=W2T, q_free=True, seed=seed,
                                         offset=step, workspace=ws_d, status=status)
        vr = sd.spec_verify_markov(P, U, x0, W1d, None, dr["tokens"], dr["q_logZ"],
                                   dr["q_tok_prob"], T, W2T=W2T, seed=seed, offset=step,
                                   workspace=ws_v)
        gd, gv = host(dr), host(vr)
        launches, _ = sd.spec_profile_read()
        sd.spec_profile_enable(None)
    finally:
        sd.spec_draft_set_persistent(was)
    assert launches == 1, "the timed shape must run the persistent engine"
    assert int(status.item()) == 0
    # properties of every request
    assert np.all((gd["tokens"] >= 0) & (gd["tokens"] < V))
    assert np.all(np.isfinite(gd["q_logZ"])) and np.all(gd["q_tok_prob"] > 0)
    n = gv["accepted"]
    assert np.all((n >= 0) & (n <= G))
    for b in range(B):
        out = gv["out_tokens"][b]
        assert np.array_equal(out[:n[b]], gd["tokens"][b, :n[b]])
        assert 0 <= out[n[b]] < V and np.all(out[n[b] + 1:] == -1)
    # element-wise parity on the sampled requests
    W1, W2 = _weights(wl)
    ud = orc.draft_uniforms(seed, step, B, G)
    uv = orc.verify_uniforms(seed, step, B, G)
    Pf = workloads.as_f64(wl["P"][sample], "bf16")
    td, tv = compare.Tally(), compare.Tally()
    for i, b in enumerate(sample):
        Ub = workloads.as_f64(wl["U"][b], "bf16")
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, ud[b])
        same = compare.compare_draft_request(o, Ub, {k: v[b] for k, v in gd.items()}, T, ud[b],
                                             f"draft b={b}", td, check_logits=False)
        if not same:
            continue
        d = {k: v[b] for k, v in gv.items()}
        d["q_logZ"] = gd["q_logZ"][b]
        compare.compare_verify_request(Pf[i], o["q_logits"], o["tokens"], T, uv[b, :G], uv[b, G],
                                       d, f"verify b={b}", tv)
    note(f"  draft {td.as_dict()} verify {tv.as_dict()} mean tau {n.mean() + 1:.3f}")
    assert tv.requests >= len(sample) - 1
    assert td.boundary <= 1


def _crafted_fallback(B, G, V, r, dt, seed):
    """A workload whose requests 0, 1 and 2 reject at a position n whose
    target and draft rows are the same distribution and give the draft token
    no mass in either: the residual max(0, p_n - q_n) is zero, so the final
    draw falls back to p_n.  The bias at n is zero (the embedding row of the
    token before n is zero), so the draft row q_n is the base row U_n itself.
      request 0: n = 0, one finite logit (p_n = q_n = one-hot, exactly);
      request 1: n = 0, five equal finite logits (p_n = q_n uniform on them);
      request 2: n = 2 after two accepted tokens, one finite logit.
    The other requests are left as generated."""
    cfg = dict(workloads.CONFIGS["markov-32k-b32"])
    cfg.update(logit_dtype=dt, w_dtype="bf16", data_seed=seed, w_std=0.3)
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=r)
    rng = np.random.default_rng(seed)
    U, P, W1, x0 = wl["U"], wl["P"], wl["W1"], wl["x0"]
    ninf = NEG_INF_BF16 if dt == "bf16" else np.float32(-np.inf)

    def enc(x):
        x = np.float32(x)
        return workloads.f32_to_bf16_bits(np.array([x]))[0] if dt == "bf16" else x

    plan = {0: (0, [11]), 1: (0, [5, 77, 300, 301, 900]), 2: (2, [1234])}
    forced = {}
    for b, (n, keep) in plan.items():
        # the draft token at n: a token outside `keep`, -inf in both rows
        x = int(rng.integers(V))
        while x in keep:
            x = int(rng.integers(V))
        U[b, n, :] = ninf
        P[b, n, :] = ninf
        for t in keep:
            U[b, n, t] = enc(1.5)
            P[b, n, t] = enc(1.5)
        toks = rng.integers(0, V, size=G).astype(np.int32)
        toks[n] = x
        prev = x0[b] if n == 0 else int(toks[n - 1])
        W1[prev, :] = 0
        forced[b] = toks
    return wl, forced, plan


def _oracle_draft_outputs(orc, wl, forced, T, rng):
    """Draft tokens, the oracle's draft logits, log Z and q(x_k) per request:
    crafted requests use their forced tokens, the others the oracle's own
    draft with uniforms from rng."""
    B, G, dt = wl["B"], wl["gamma"], wl["logit_dtype"]
    W1, W2 = _weights(wl)
    draft = np.zeros((B, G), np.int32)
    lz = np.zeros((B, G), np.float32)
    qx = np.zeros((B, G), np.float32)
    Q = []
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], dt)
        u = rng.random(G)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, u, forced=forced.get(b))
        toks = forced.get(b, o["tokens"])
        for k in range(G):
            w, Z, logZ = orc.softmax_weights(o["q_logits"][k], T)
            lz[b, k] = logZ
            qx[b, k] = w[toks[k]] / Z
        draft[b] = toks
        Q.append(o["q_logits"])
    return draft, Q, lz, qx


@pytest.mark.parametrize("path,dt", [("qfree", "bf16"), ("qfree", "f32"),
                                     ("materialized", "f32")])
def test_residual_zero_mass_fallback(orc, path, dt):
    sd = require_gpu()
    B, G, V, r, T = 6, 4, 4096, 64, 1.0
    note(f"zero-mass residual fallback path={path} dtype={dt}")
    wl, forced, plan = _crafted_fallback(B, G, V, r, dt, 4321)
    draft, Q, lz, qx = _oracle_draft_outputs(orc, wl, forced, T, np.random.default_rng(5))
    # caller uniforms: ratio tests 0 (accept any token with p > 0) before the
    # crafted position, then just below 1; the final draw at 0.37
    uni = np.zeros((B, G + 1), np.float32)
    for b in range(B):
        n = plan[b][0] if b in plan else G
        uni[b, n:G] = np.float32(1.0 - 2**-24)
        uni[b, G] = np.float32(0.37)
    Pd, W1d, W2d, x0 = dev(wl["P"], dt), dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(wl["x0"])
    if path == "qfree":
        g = host(sd.spec_verify_markov(Pd, dev(wl["U"], dt), x0, W1d, W2d, dev(draft), dev(lz),
                                       dev(qx), T, uniforms=dev(uni)))
    else:
        Qd = dev(np.stack(Q).astype(np.float32))
        g = host(sd.spec_verify(Pd, Qd, dev(draft), T, uniforms=dev(uni)))
    Pf = workloads.as_f64(wl["P"], dt)
    if path == "materialized":        # the oracle gets the fp32 rows the GPU got
        Q = [q.astype(np.float32).astype(np.float64) for q in Q]
    tally = compare.Tally()
    u = uni.astype(np.float64)
    for b in range(B):
        d = {k: v[b] for k, v in g.items()}
        if path == "qfree":
            d["q_logZ"] = lz[b]
        compare.compare_verify_request(Pf[b], Q[b], draft[b], T, u[b, :G], u[b, G], d, f"b={b}",
                                       tally)
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert tally.fallbacks >= 3          # the oracle took the fallback on requests 0, 1, 2
    for b, (n, keep) in plan.items():
        assert g["accepted"][b] == n
        assert g["out_tokens"][b, n] in keep
    assert g["out_tokens"][0, 0] == 11 and g["out_tokens"][2, 2] == 1234
    assert tally.boundary == 0


def test_side_stream_allocations():
    """A draft and its verification on a side stream, with the binding
    allocating workspaces and outputs, interleaved with allocations and
    writes on the main stream: the results equal those of the same calls on
    the current stream."""
    sd = require_gpu()
    B, G, V, r = 96, 6, 40000, 128
    note(f"side-stream draft + verify B={B} gamma={G} V={V} r={r}")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=r)
    U, P = dev(wl["U"], "bf16"), dev(wl["P"], "bf16")
    W1, W2, x0 = dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(wl["x0"])

    def cycle(stream):
        d = sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, seed=8, stream=stream)
        v = sd.spec_verify_markov(P, U, x0, W1, W2, d["tokens"], d["q_logZ"], d["q_tok_prob"],
                                  1.0, seed=8, stream=stream)
        return d, v

    ref_d, ref_v = cycle(None)
    ref = {**host(ref_d), **host(ref_v)}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    results = []
    for rep in range(3):
        d, v = cycle(side)
        # main-stream traffic while the side stream still runs: allocations
        # of the sizes the binding freed, filled with garbage
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
                for n in (sd.workspace_bytes("markov", B=B, gamma=G, V=V, r=r),
                          sd.workspace_bytes("verify_markov", B=B, gamma_max=G, V=V, r=r),
                          1 << 20)]
        results.append((d, v, junk))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for d, v, _ in results:
        got = {**{k: x.cpu().numpy() for k, x in d.items()},
               **{k: x.cpu().numpy() for k, x in v.items()}}
        for k in ("tokens", "q_logZ", "q_tok_prob", "accepted", "out_tokens"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


def test_cycle_graph_replays():
    """One q-free cycle (persistent draft with the packed W2 image, then
    spec_verify_markov) captured in a HIP graph and replayed three times, with
    direct cycles on other uniforms between the replays: every replay gives
    the direct cycle's tokens, normalisers and verdicts bit for bit (every
    word a call reads is written or reset inside the call), and the draft
    status stays 0."""
    sd = require_gpu()
    B, G, V, r = 96, 6, 40000, 128
    note(f"graph-replayed draft + verify B={B} gamma={G} V={V} r={r}")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=r)
    U, P = dev(wl["U"], "bf16"), dev(wl["P"], "bf16")
    W1, W2, x0 = dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(wl["x0"])
    W2T = sd.spec_pack_w2(W2)
    status = torch.full((1,), -3, dtype=torch.int32, device="cuda")

    def cycle(seed):
        d = sd.spec_draft_sample_markov(U, x0, W1, None, 1.0, W2T=W2T, q_free=True, seed=seed,
                                        status=status)
        v = sd.spec_verify_markov(P, U, x0, W1, W2, d["tokens"], d["q_logZ"], d["q_tok_prob"],
                                  1.0, seed=seed)
        return d, v

    def host_of(d, v):
        torch.cuda.synchronize()
        return {**{k: x.cpu().numpy() for k, x in d.items()},
                **{k: x.cpu().numpy() for k, x in v.items()}}

    keys = ("tokens", "q_logZ", "q_tok_prob", "accepted", "out_tokens")
    ref_a = host_of(*cycle(8))
    ref_b = host_of(*cycle(9))
    assert not np.array_equal(ref_a["tokens"], ref_b["tokens"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cycle(8)   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gd, gv = cycle(8)
    for rep in range(3):
        for t in (*gd.values(), *gv.values()):
            t.fill_(-5)
        status.fill_(-3)
        graph.replay()
        got = host_of(gd, gv)
        assert int(status.cpu()[0]) == 0, rep
        for k in keys:
            np.testing.assert_array_equal(got[k], ref_a[k], err_msg=f"replay {rep}: {k}")
        between = host_of(*cycle(9))
        for k in keys:
            np.testing.assert_array_equal(between[k], ref_b[k], err_msg=f"direct {rep}: {k}")
