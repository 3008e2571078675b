"""GPU parity of the q-free Markov cycle against the oracle.

The q-free draft writes no draft-logit tensor: per position it returns the
token, the draft normaliser log Z and q(x_k), and locates the token from
8-token group sums plus a rebuild of one group's logits.  spec_verify_markov
takes those three outputs and rebuilds, for each request that needs a
residual draw, the single draft row q_n = U_n + W1[x_{n-1}] W2.  Both are
checked element by element against the oracle on the same seeded inputs;
the oracle never sees a GPU output."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _cfg(name, logit_dtype, seed, **kw):
    cfg = dict(workloads.CONFIGS[name])
    cfg.update(logit_dtype=logit_dtype, w_dtype="bf16", data_seed=seed, **kw)
    return cfg


def _weights(wl):
    return workloads.as_f64(wl["W1"], "bf16"), workloads.as_f64(wl["W2"], "bf16")


DRAFT_CASES = [
    # B, gamma, V, r, U dtype, T
    (3, 5, 5000, 64, "f32", 1.0),       # 32-row groups
    (40, 3, 3000, 32, "bf16", 1.0),     # 64-row groups
    (70, 3, 2000, 256, "f32", 0.8),     # 128-row groups
    (130, 2, 1500, 128, "bf16", 1.0),   # two row blocks
    (5, 4, 4099, 48, "f32", 1.3),       # ragged last tile (3 tokens)
    (4, 6, 131, 16, "f32", 1.0),        # two tiles
    (3, 4, 7, 16, "bf16", 1.0),         # one partial 8-token group
    (6, 4, 3000, 64, "bf16", 0.0),      # greedy
    # streaming tile (bf16 U, V % 8 == 0, B > 64, r in {64, 128, 256}):
    (130, 3, 3000, 256, "bf16", 1.0),   # two row blocks, one item per workgroup
    (100, 3, 40000, 128, "bf16", 1.0),  # three items per workgroup: full pipeline
    (200, 2, 20008, 64, "bf16", 0.9),   # row block changes inside a workgroup; 40-token tail
    (80, 3, 16384, 256, "bf16", 0.0),   # greedy
    # fp32 U on the persistent engine (4 KB units, 8 lanes per row piece):
    (32, 7, 32000, 256, "f32", 1.0),    # the 32k-vocabulary configuration's shape
    (130, 2, 3000, 128, "f32", 0.9),    # two row blocks
    (70, 3, 20008, 64, "f32", 1.0),     # 40-token tail, r = 64
    (9, 3, 3000, 256, "f32", 0.0),      # greedy
    # persistent draft (bf16 U, V % 8 == 0, r in {64, 128, 256}, W2 share fits):
    (1, 3, 5000, 64, "bf16", 1.0),      # one row: 31 absent rows in its group
    (33, 2, 8, 64, "bf16", 1.0),        # V = 8: one block, one workgroup
    (5, 2, 1000, 128, "bf16", 0.7),     # 32 blocks: one per workgroup, three idle waves
    (4, 2, 153600, 256, "bf16", 1.0),   # 20 blocks per workgroup: all register blocks in use
    (3, 1, 153608, 256, "bf16", 1.0),   # one block more than fits: per-position kernels
    (130, 3, 8192, 128, "bf16", 1.0),   # three 64-row blocks, the last one of 2 rows
    (65, 4, 9000, 256, "bf16", 1.0),    # a one-row second block: U of each block issued early
    (128, 5, 30000, 64, "bf16", 0.0),   # two full blocks at r = 64, greedy
]


def persist_eligible(B, gamma, V, r, udt):
    """Shapes the library runs as one persistent launch (256 CUs, 16 of them
    finalizing: at most 20 / 40 / 80 blocks of 32 tokens per unit workgroup
    for r = 256 / 128 / 64)."""
    if udt not in ("bf16", "f32") or V % 8 or r not in (64, 128, 256) or B < 1 or gamma < 1:
        return False
    nblk = (V + 31) // 32
    ng = min(240, nblk)
    return -(-nblk // ng) <= 4 * {256: 5, 128: 10, 64: 20}[r]


@pytest.fixture(params=["persistent", "per_position"])
def engine(request):
    sd = require_gpu()
    was = sd.spec_draft_set_persistent(request.param == "persistent")
    yield request.param
    sd.spec_draft_set_persistent(was)


@pytest.mark.parametrize("B,gamma,V,r,udt,T", DRAFT_CASES)
def test_qfree_draft_parity(orc, engine, B, gamma, V, r, udt, T):
    sd = require_gpu()
    eligible = persist_eligible(B, gamma, V, r, udt)
    if engine == "per_position" and not eligible:
        pytest.skip("same kernels as the persistent engine for this shape")
    note(f"q-free draft B={B} gamma={gamma} V={V} r={r} U={udt} T={T} engine={engine}")
    wl = workloads.make_markov(_cfg("markov-32k-b32", udt, 300 + B + V, w_std=0.3), B=B,
                               gamma=gamma, V=V, r=r)
    seed, offset = 17, 5
    sd.spec_profile_enable("draft_persist")
    g = host(sd.spec_draft_sample_markov(dev(wl["U"], udt), dev(wl["x0"]), dev(wl["W1"], "bf16"),
                                         dev(wl["W2"], "bf16"), T, q_free=True, seed=seed,
                                         offset=offset))
    launches, _ = sd.spec_profile_read()
    sd.spec_profile_enable(None)
    assert launches == (1 if engine == "persistent" and eligible else 0)
    assert "q_logits" not in g
    W1, W2 = _weights(wl)
    u = orc.draft_uniforms(seed, offset, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], udt)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, T, u[b], f"b={b}",
                                      tally, check_logits=False)
    note(f"  {tally.as_dict()}")
    assert tally.boundary <= max(1, tally.draws // 50)


def packed_image(W2, r, V):
    """The packed W2 layout as the header documents it, built element by
    element from W2 [r, V] (uint16 bf16 bits)."""
    ntile = (V + 127) // 128
    img = np.zeros(ntile * 128 * r, dtype=np.uint16)
    nchunk = r // 8
    F = min(16, nchunk & -nchunk)
    for v in range(V):
        u = v % 128
        s = ((u & 3) | ((((u >> 4) ^ (u >> 2)) & 3) << 2)) & (F - 1)
        for kc in range(nchunk):
            dst = v * r + 8 * (kc ^ s)
            img[dst:dst + 8] = W2[8 * kc:8 * kc + 8, v]
    return img


@pytest.mark.parametrize("r,V", [(64, 6001), (48, 300), (256, 1000), (16, 129)])
def test_pack_w2_layout(r, V):
    sd = require_gpu()
    W2 = workloads.f32_to_bf16_bits(
        np.random.default_rng(r + V).standard_normal((r, V)).astype(np.float32))
    img = sd.spec_pack_w2(dev(W2, "bf16"))
    torch.cuda.synchronize()
    got = img.cpu().numpy().view(np.uint16)
    assert got.nbytes == sd.spec_pack_w2_bytes(r, V)
    assert np.array_equal(got, packed_image(W2, r, V))


def test_qfree_draft_full_size_sampled(orc, engine):
    """B = 128, gamma = 16, V = 151936, r = 256, bf16: both draft engines at the
    size they are timed at; four requests are checked against the oracle."""
    sd = require_gpu()
    note(f"full-size q-free draft engine={engine}")
    B, gamma, V, r = 128, 16, 151936, 256
    sample = [0, 45, 96, 127]
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=gamma, V=V, r=r)
    seed = 77
    W2T = sd.spec_pack_w2(dev(wl["W2"], "bf16"))
    g = host(sd.spec_draft_sample_markov(dev(wl["U"], "bf16"), dev(wl["x0"]),
                                         dev(wl["W1"], "bf16"), None, 1.0, W2T=W2T, q_free=True,
                                         seed=seed))
    W1, W2 = _weights(wl)
    u = orc.draft_uniforms(seed, 0, B, gamma)
    tally = compare.Tally()
    for b in sample:
        Ub = workloads.as_f64(wl["U"][b], "bf16")
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], 1.0, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, 1.0, u[b],
                                      f"b={b}", tally, check_logits=False)
    note(f"  {tally.as_dict()}")
    assert np.all((g["tokens"] >= 0) & (g["tokens"] < V))
    assert np.all(np.isfinite(g["q_logZ"])) and np.all(g["q_tok_prob"] > 0)


@pytest.mark.parametrize("B,gamma,V,r", [(128, 16, 151936, 256), (130, 3, 8192, 128)])
def test_qfree_draft_launch_modes(B, gamma, V, r):
    """The persistent draft under a plain launch (mode 1) and a cooperative
    launch (mode 2) is the same kernel: identical tokens, log Z and q(x_k)."""
    sd = require_gpu()
    assert persist_eligible(B, gamma, V, r, "bf16")
    note(f"persistent draft launch modes B={B} gamma={gamma} V={V} r={r}")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=gamma, V=V, r=r)
    args = (dev(wl["U"], "bf16"), dev(wl["x0"]), dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), 1.0)
    res = {}
    was = sd.spec_draft_set_persistent(1)
    try:
        for mode in (1, 2):
            sd.spec_draft_set_persistent(mode)
            sd.spec_profile_enable("draft_persist")
            res[mode] = host(sd.spec_draft_sample_markov(*args, q_free=True, seed=5, offset=2))
            launches, _ = sd.spec_profile_read()
            sd.spec_profile_enable(None)
            assert launches == 1
    finally:
        sd.spec_draft_set_persistent(was)
    for k in ("tokens", "q_logZ", "q_tok_prob"):
        np.testing.assert_array_equal(res[1][k], res[2][k], err_msg=k)
    assert np.all((res[1]["tokens"] >= 0) & (res[1]["tokens"] < V))


def test_persistent_draft_gives_up_cleanly():
    """With a wait limit of two polls (set from the host) the persistent draft
    gives up on its waits: the launch still ends, every token is -1 or a valid
    id and some rows stay -1, verification marks the requests holding a -1
    invalid (accepted -1), and the next call with the default limit matches a
    call made before."""
    sd = require_gpu()
    B, gamma, V, r = 128, 4, 32000, 256
    assert persist_eligible(B, gamma, V, r, "bf16")
    note(f"persistent draft wait limit B={B} gamma={gamma} V={V} r={r}")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=gamma, V=V, r=r)
    U, x0 = dev(wl["U"], "bf16"), dev(wl["x0"])
    W1, W2 = dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16")
    was_mode = sd.spec_draft_set_persistent(1)
    try:
        st_ref, st_bad, st_again = (torch.full((1,), 7, dtype=torch.int32, device="cuda")
                                    for _ in range(3))
        ref = host(sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, seed=3,
                                               status=st_ref))
        sd.spec_draft_set_poll_limit(2)
        d = sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, seed=3, status=st_bad)
        torch.cuda.synchronize()
        sd.spec_draft_set_poll_limit(0)
        bad = host(d)
        again = host(sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, seed=3,
                                                 status=st_again))
        v = host(sd.spec_verify_markov(dev(wl["P"], "bf16"), U, x0, W1, W2, d["tokens"],
                                       d["q_logZ"], d["q_tok_prob"], 1.0, seed=3))
    finally:
        sd.spec_draft_set_poll_limit(0)
        sd.spec_draft_set_persistent(was_mode)
    # the completion word reports the give-up, and only it
    assert (int(st_ref.item()), int(st_bad.item()), int(st_again.item())) == (0, 1, 0)
    tok = bad["tokens"]
    assert np.all((tok == -1) | ((tok >= 0) & (tok < V)))
    assert (tok == -1).any()
    undrawn = (tok == -1).any(axis=1)
    note(f"  requests with an undrawn token: {int(undrawn.sum())} of {B}")
    assert np.all(v["accepted"][undrawn] == -1)
    assert np.all(v["accepted"][~undrawn] >= 0)
    for k in ("tokens", "q_logZ", "q_tok_prob"):
        np.testing.assert_array_equal(ref[k], again[k], err_msg=k)


def test_draft_status_other_engines():
    """The per-position engine and the materialised draft have no waits: after
    a persistent call that gave up, a call on either engine with the same
    workspace reads complete (0) again."""
    sd = require_gpu()
    B, gamma, V, r = 70, 3, 8192, 128
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=gamma, V=V, r=r)
    U, x0 = dev(wl["U"], "bf16"), dev(wl["x0"])
    W1, W2 = dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16")
    ws = torch.empty(sd.workspace_bytes("markov", B=B, gamma=gamma, V=V, r=r), dtype=torch.uint8,
                     device="cuda")
    st = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    was = sd.spec_draft_set_persistent(1)
    try:
        sd.spec_draft_set_poll_limit(2)
        sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, workspace=ws, status=st)
        sd.spec_draft_set_poll_limit(0)
        assert int(st.item()) == 1
        sd.spec_draft_set_persistent(0)
        d = sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, workspace=ws, status=st)
        assert int(st.item()) == 0
        assert bool((d["tokens"] >= 0).all())
        sd.spec_draft_set_persistent(1)
        sd.spec_draft_set_poll_limit(2)
        sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, q_free=True, workspace=ws, status=st)
        sd.spec_draft_set_poll_limit(0)
        assert int(st.item()) == 1
        sd.spec_draft_sample_markov(U, x0, W1, W2, 1.0, workspace=ws, status=st)   # q logits
        assert int(st.item()) == 0
        st2 = sd.spec_draft_status(ws, B, gamma, V, r)
        assert int(st2.item()) == 0
    finally:
        sd.spec_draft_set_poll_limit(0)
        sd.spec_draft_set_persistent(was)


def test_qfree_draft_packed_w2_and_uniforms(orc):
    """A W2T packed once by spec_pack_w2 gives the same result as W2, and
    caller uniforms replace the counter stream."""
    sd = require_gpu()
    B, gamma, V, r = 9, 5, 6001, 64
    wl = workloads.make_markov(_cfg("markov-32k-b32", "f32", 77, w_std=0.3), B=B, gamma=gamma,
                               V=V, r=r)
    W2d = dev(wl["W2"], "bf16")
    W2T = sd.spec_pack_w2(W2d)
    uni = np.random.default_rng(8).random((B, gamma)).astype(np.float32)
    args = (dev(wl["U"]), dev(wl["x0"]), dev(wl["W1"], "bf16"))
    a = host(sd.spec_draft_sample_markov(*args, W2d, 1.0, q_free=True, uniforms=dev(uni)))
    b = host(sd.spec_draft_sample_markov(*args, None, 1.0, W2T=W2T, q_free=True,
                                         uniforms=dev(uni)))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    W1, W2 = _weights(wl)
    tally = compare.Tally()
    for i in range(B):
        Ub = workloads.as_f64(wl["U"][i], "f32")
        ui = uni[i].astype(np.float64)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][i], 1.0, ui)
        compare.compare_draft_request(o, Ub, {k: v[i] for k, v in a.items()}, 1.0, ui, f"b={i}",
                                      tally, check_logits=False)
    note(f"  {tally.as_dict()}")


def test_qfree_draft_invalid_anchor_persistent(orc):
    """An anchor outside [0, V) in the persistent engine: that request gets -1
    tokens and NaN normalisers; the other requests still match the oracle."""
    sd = require_gpu()
    B, gamma, V, r = 40, 3, 2000, 64
    wl = workloads.make_markov(_cfg("markov-32k-b32", "bf16", 6, w_std=0.3), B=B, gamma=gamma,
                               V=V, r=r)
    x0 = wl["x0"].copy()
    x0[7] = V
    x0[33] = -2
    g = host(sd.spec_draft_sample_markov(dev(wl["U"], "bf16"), dev(x0), dev(wl["W1"], "bf16"),
                                         dev(wl["W2"], "bf16"), 1.0, q_free=True, seed=4))
    for b in (7, 33):
        assert np.all(g["tokens"][b] == -1) and np.all(np.isnan(g["q_logZ"][b]))
    W1, W2 = _weights(wl)
    u = orc.draft_uniforms(4, 0, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        if b in (7, 33):
            continue
        Ub = workloads.as_f64(wl["U"][b], "bf16")
        o = orc.draft_markov(Ub, W1, W2, x0[b], 1.0, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, 1.0, u[b],
                                      f"b={b}", tally, check_logits=False)
    note(f"  {tally.as_dict()}")


def test_qfree_draft_invalid_anchor():
    sd = require_gpu()
    B, gamma, V, r = 3, 3, 500, 16
    wl = workloads.make_markov(_cfg("markov-32k-b32", "f32", 5), B=B, gamma=gamma, V=V, r=r)
    x0 = wl["x0"].copy()
    x0[1] = V + 3
    g = host(sd.spec_draft_sample_markov(dev(wl["U"]), dev(x0), dev(wl["W1"], "bf16"),
                                         dev(wl["W2"], "bf16"), 1.0, q_free=True, seed=2))
    assert np.all(g["tokens"][1] == -1) and np.all(np.isnan(g["q_logZ"][1]))
    assert np.all(g["tokens"][[0, 2]] >= 0)


# ---------------------------------------------------------------------------
# spec_verify_markov on drafts the oracle produced
# ---------------------------------------------------------------------------

def _oracle_block(orc, wl, udt, T, u, rng, random_frac):
    """The oracle's draft of every request, with a fraction of requests given
    one random token (re-drafted with that prefix forced).  Returns the draft
    tokens, the oracle's draft logits and the draft normaliser and q(x_k) in
    fp32 as the draft would hand them over."""
    B, G = wl["B"], wl["gamma"]
    W1, W2 = _weights(wl)
    draft = np.zeros((B, G), dtype=np.int32)
    Q, lz, qx = [], np.zeros((B, G), np.float32), np.zeros((B, G), np.float32)
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], udt)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, u[b])
        toks = o["tokens"].copy()
        if G and rng.random() < random_frac:
            toks[rng.integers(G)] = rng.integers(wl["V"])
            o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, u[b], forced=toks)
        for k in range(G):
            if T == 0:
                qx[b, k] = 1.0 if toks[k] == orc.argmax(o["q_logits"][k])[0] else 0.0
            else:
                w, Z, _ = orc.softmax_weights(o["q_logits"][k], T)
                qx[b, k] = w[toks[k]] / Z
        draft[b] = toks
        lz[b] = o["logZ"]
        Q.append(o["q_logits"])
    return draft, Q, lz, qx


def _verify_rows(g, b, lz):
    d = {k: v[b] for k, v in g.items()}
    d["q_logZ"] = lz[b]
    return d


@pytest.mark.parametrize("B,G,V,r,pdt,udt,T,sigma", [
    (12, 5, 5000, 64, "f32", "f32", 1.0, 0.6),
    (12, 4, 4099, 48, "bf16", "f32", 0.7, 0.3),
    (70, 3, 3000, 256, "bf16", "bf16", 1.0, 1.2),    # 128-row residual groups
    (130, 2, 1500, 128, "f32", "bf16", 1.0, 1.5),    # two row blocks
    (8, 4, 131, 16, "f32", "f32", 1.0, 0.8),
    (10, 5, 2000, 64, "f32", "f32", 0.0, 0.6),       # greedy
    # streamed final draw (bf16 P and U, V % 8 == 0, r in {64, 128, 256}):
    (140, 3, 4104, 128, "bf16", "bf16", 0.8, 1.0),   # two row blocks, 8-token tail slice
    (20, 4, 3000, 256, "bf16", "bf16", 1.3, 0.4),
])
def test_verify_markov_parity(orc, B, G, V, r, pdt, udt, T, sigma):
    sd = require_gpu()
    note(f"verify_markov B={B} G={G} V={V} r={r} P={pdt} U={udt} T={T}")
    cfg = _cfg("markov-32k-b32", udt, 500 + B + V, w_std=0.3, sigma=sigma)
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=r)
    rng = np.random.default_rng(V)
    ud = orc.draft_uniforms(3, 1, B, G)
    draft, Q, lz, qx = _oracle_block(orc, wl, udt, T, ud, rng, 0.3)
    P32 = workloads.as_f64(wl["P"], cfg["logit_dtype"]).astype(np.float32)
    P = workloads.f32_to_bf16_bits(P32) if pdt == "bf16" else P32
    # request 0: the first draft token has no target mass -> n = 0
    P[0, 0, draft[0, 0]] = np.float32(-np.inf) if pdt == "f32" else np.uint16(0xFF80)
    # request 1: target rows equal the draft rows -> every token accepted
    Pq = np.concatenate([Q[1], workloads.as_f64(P[1, G:], pdt)], axis=0).astype(np.float32)
    P[1] = workloads.f32_to_bf16_bits(Pq) if pdt == "bf16" else Pq
    Pf = workloads.as_f64(P, pdt)
    seed = 23
    g = host(sd.spec_verify_markov(dev(P, pdt), dev(wl["U"], udt), dev(wl["x0"]),
                                   dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(draft),
                                   dev(lz), dev(qx), T, seed=seed))
    u = orc.verify_uniforms(seed, 0, B, G)
    tally = compare.Tally()
    for b in range(B):
        compare.compare_verify_request(Pf[b], Q[b], draft[b], T, u[b, :G], u[b, G],
                                       _verify_rows(g, b, lz), f"b={b}", tally)
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert g["accepted"][0] == 0
    if pdt == "f32" and T > 0:
        assert g["accepted"][1] == G
    assert tally.boundary <= max(1, tally.draws // 50)


def test_verify_markov_ragged_packed(orc):
    """Ragged lengths (one empty draft) with packed target rows and a W2T
    packed by spec_pack_w2."""
    sd = require_gpu()
    B, G, V, r = 10, 6, 3000, 64
    cfg = _cfg("ragged-128k-b256", "bf16", 41, w_std=0.3)
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=r)
    lens = wl["lens"].copy()
    p_off0 = workloads.packed_offsets(lens + 1)
    lens[3] = 0
    Pp = np.concatenate([wl["P"][p_off0[b]:p_off0[b] + lens[b] + 1] for b in range(B)], axis=0)
    p_off = workloads.packed_offsets(lens + 1)
    ud = orc.draft_uniforms(6, 0, B, G)
    draft, Q, lz, qx = _oracle_block(orc, wl, "bf16", 1.0, ud, np.random.default_rng(2), 0.3)
    for b in range(B):
        draft[b, lens[b]:] = -7            # slots past L are never read
    W2T = sd.spec_pack_w2(dev(wl["W2"], "bf16"))
    seed = 9
    g = host(sd.spec_verify_markov(dev(Pp, "bf16"), dev(wl["U"], "bf16"), dev(wl["x0"]),
                                   dev(wl["W1"], "bf16"), None, dev(draft), dev(lz), dev(qx), 1.0,
                                   W2T=W2T, gamma_max=G, lens=dev(lens), p_row_off=dev(p_off),
                                   seed=seed))
    Pf = workloads.as_f64(Pp, "bf16")
    u = orc.verify_uniforms(seed, 0, B, G)
    tally = compare.Tally()
    for b in range(B):
        L = int(lens[b])
        d = {k: v[b] for k, v in g.items()}
        d["q_logZ"] = lz[b]
        compare.compare_verify_request(Pf[p_off[b]:p_off[b] + L + 1], Q[b][:L], draft[b, :L],
                                       1.0, u[b, :L], u[b, G], d, f"b={b} L={L}", tally)
        assert 0 <= g["accepted"][b] <= L
    assert g["accepted"][3] == 0
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")


def test_verify_markov_bonus_only_bf16(orc):
    """gamma_max = 0 with bf16 rows: every request draws its bonus token from
    its single target row (no residual, so the streamed draw is not used; the
    library must not touch a packed W2 it never built)."""
    sd = require_gpu()
    B, V, r = 5, 4000, 64
    rng = np.random.default_rng(12)
    P32 = (rng.standard_normal((B, 1, V)) * 3).astype(np.float32)
    P = workloads.f32_to_bf16_bits(P32)
    W1 = workloads.f32_to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32))
    W2 = workloads.f32_to_bf16_bits(rng.standard_normal((r, V)).astype(np.float32))
    empty_f = torch.zeros((B, 0), dtype=torch.float32, device="cuda")
    g = host(sd.spec_verify_markov(
        dev(P, "bf16"), torch.zeros((B, 0, V), dtype=torch.bfloat16, device="cuda"),
        dev(np.zeros(B, np.int32)), dev(W1, "bf16"), dev(W2, "bf16"),
        torch.zeros((B, 0), dtype=torch.int32, device="cuda"), empty_f, empty_f, 1.0, seed=6))
    u = orc.verify_uniforms(6, 0, B, 0)
    Pf = workloads.as_f64(P, "bf16")
    tally = compare.Tally()
    for b in range(B):
        w, Z, _ = orc.softmax_weights(Pf[b, 0], 1.0)
        want = orc.inverse_cdf(w, Z, u[b, 0])[0]
        assert g["accepted"][b] == 0
        if g["out_tokens"][b, 0] != want:
            compare._check_draw(w, want, int(g["out_tokens"][b, 0]), u[b, 0], f"b={b}")
            tally.boundary += 1
    assert tally.boundary <= 1


def test_verify_markov_bonus_only(orc):
    sd = require_gpu()
    B, V, r = 3, 500, 16
    rng = np.random.default_rng(5)
    P = rng.standard_normal((B, 1, V)).astype(np.float32)
    W1 = workloads.f32_to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32))
    W2 = workloads.f32_to_bf16_bits(rng.standard_normal((r, V)).astype(np.float32))
    empty_f = torch.zeros((B, 0), dtype=torch.float32, device="cuda")
    g = host(sd.spec_verify_markov(
        dev(P), torch.zeros((B, 0, V), device="cuda"), dev(np.zeros(B, np.int32)),
        dev(W1, "bf16"), dev(W2, "bf16"), torch.zeros((B, 0), dtype=torch.int32, device="cuda"),
        empty_f, empty_f, 1.0, seed=3))
    u = orc.verify_uniforms(3, 0, B, 0)
    for b in range(B):
        w, Z, _ = orc.softmax_weights(P[b, 0].astype(np.float64), 1.0)
        assert g["accepted"][b] == 0
        assert g["out_tokens"][b, 0] == orc.inverse_cdf(w, Z, u[b, 0])[0]


# ---------------------------------------------------------------------------
# The whole q-free cycle on the GPU against the oracle's cycle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,B,G,V,T", [
    ("markov-32k-b32", 16, 7, 32000, 1.0),
    ("markov-152k-b128", 4, 16, 151936, 1.0),
    ("ragged-128k-b256", 6, 8, 20000, 0.9),
])
def test_qfree_cycle_against_oracle(orc, name, B, G, V, T):
    """GPU q-free draft -> spec_verify_markov, compared with the oracle's draft
    and verification of the same request.  Requests whose draft met a
    boundary draw are counted and their verification skipped (the two sides
    then condition on different prefixes)."""
    sd = require_gpu()
    note(f"q-free cycle {name} B={B} G={G} V={V} T={T}")
    cfg = dict(workloads.CONFIGS[name])
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V)
    ldt = cfg["logit_dtype"]
    lens = wl["lens"]
    p_off = None if lens is None else workloads.packed_offsets(lens + 1)
    U, W1d, W2d, x0 = dev(wl["U"], ldt), dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(wl["x0"])
    seed = 1234
    dr = sd.spec_draft_sample_markov(U, x0, W1d, W2d, T, q_free=True, seed=seed, offset=0)
    vr = sd.spec_verify_markov(dev(wl["P"], ldt), U, x0, W1d, W2d, dr["tokens"], dr["q_logZ"],
                               dr["q_tok_prob"], T, lens=None if lens is None else dev(lens),
                               p_row_off=None if p_off is None else dev(p_off), seed=seed,
                               offset=1)
    gd, gv = host(dr), host(vr)
    W1, W2 = _weights(wl)
    ud = orc.draft_uniforms(seed, 0, B, G)
    uv = orc.verify_uniforms(seed, 1, B, G)
    Pf = workloads.as_f64(wl["P"], ldt)
    td, tv = compare.Tally(), compare.Tally()
    for b in range(B):
        L = G if lens is None else int(lens[b])
        Ub = workloads.as_f64(wl["U"][b], ldt)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, ud[b])
        same = compare.compare_draft_request(o, Ub, {k: v[b] for k, v in gd.items()}, T, ud[b],
                                             f"draft b={b}", td, check_logits=False)
        if not same and not np.array_equal(gd["tokens"][b, :L], o["tokens"][:L]):
            continue
        Pb = Pf[b] if lens is None else Pf[p_off[b]:p_off[b] + L + 1]
        d = {k: v[b] for k, v in gv.items()}
        d["q_logZ"] = gd["q_logZ"][b]
        compare.compare_verify_request(Pb, o["q_logits"][:L], o["tokens"][:L], T, uv[b, :L],
                                       uv[b, G], d, f"verify b={b}", tv)
    note(f"  draft {td.as_dict()} verify {tv.as_dict()} accepted={gv['accepted'].tolist()}")
    assert tv.requests >= B - 1
