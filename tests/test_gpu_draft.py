"""GPU parity of the sequential draft stage (Markov and RNN heads) against the
oracle, on every tile configuration of the kernels (row groups of 32/64/128,
several row blocks, vocabulary tails, both weight paths, greedy)."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu


def _markov_cfg(logit_dtype, w_dtype, seed, w_std=0.3):
    cfg = dict(workloads.CONFIGS["markov-32k-b32"])
    cfg.update(logit_dtype=logit_dtype, w_dtype=w_dtype, w_std=w_std, data_seed=seed)
    return cfg


CASES = [
    # B, gamma, V, r, U dtype, W dtype, T
    (1, 4, 1000, 16, "f32", "f32", 1.0),       # fp32 weights: vector-ALU tile
    (3, 5, 5000, 64, "f32", "bf16", 1.0),      # 32-row groups, 4 waves along V
    (40, 3, 3000, 32, "bf16", "bf16", 1.0),    # 64-row groups
    (70, 3, 2000, 256, "f32", "bf16", 0.8),    # 128-row groups
    (130, 2, 1500, 128, "bf16", "bf16", 1.0),  # two row blocks
    (5, 4, 4099, 48, "f32", "bf16", 1.0),      # V % 8 != 0: scalar edges
    (6, 4, 3000, 64, "f32", "bf16", 0.0),      # greedy
    (2, 3, 777, 16, "bf16", "f32", 0.0),       # greedy, fp32 weights
    (4, 6, 131, 16, "f32", "bf16", 1.0),       # two tiles, ragged
]


@pytest.mark.parametrize("B,gamma,V,r,udt,wdt,T", CASES)
def test_markov_draft_parity(orc, B, gamma, V, r, udt, wdt, T):
    sd = require_gpu()
    note(f"markov draft B={B} gamma={gamma} V={V} r={r} U={udt} W={wdt} T={T}")
    wl = workloads.make_markov(_markov_cfg(udt, wdt, 100 + B + V), B=B, gamma=gamma, V=V, r=r)
    seed, offset = 21, 3
    g = host(sd.spec_draft_sample_markov(dev(wl["U"], udt), dev(wl["x0"]), dev(wl["W1"], wdt),
                                         dev(wl["W2"], wdt), T, seed=seed, offset=offset))
    W1 = workloads.as_f64(wl["W1"], wdt)
    W2 = workloads.as_f64(wl["W2"], wdt)
    u = orc.draft_uniforms(seed, offset, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], udt)
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][b], T, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, T, u[b], f"b={b}",
                                      tally)
    note(f"  {tally.as_dict()}")
    assert tally.boundary <= max(1, tally.draws // 50)


def test_markov_caller_uniforms_and_determinism(orc):
    sd = require_gpu()
    B, gamma, V, r = 8, 5, 6000, 64
    wl = workloads.make_markov(_markov_cfg("f32", "bf16", 9), B=B, gamma=gamma, V=V, r=r)
    uni = np.random.default_rng(4).random((B, gamma)).astype(np.float32)
    args = (dev(wl["U"]), dev(wl["x0"]), dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), 1.0)
    a = host(sd.spec_draft_sample_markov(*args, uniforms=dev(uni)))
    b = host(sd.spec_draft_sample_markov(*args, uniforms=dev(uni)))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    W1, W2 = workloads.as_f64(wl["W1"], "bf16"), workloads.as_f64(wl["W2"], "bf16")
    tally = compare.Tally()
    for i in range(B):
        Ub = workloads.as_f64(wl["U"][i], "f32")
        o = orc.draft_markov(Ub, W1, W2, wl["x0"][i], 1.0, uni[i].astype(np.float64))
        compare.compare_draft_request(o, Ub, {k: v[i] for k, v in a.items()}, 1.0,
                                      uni[i].astype(np.float64), f"b={i}", tally)


def test_markov_invalid_anchor(orc):
    sd = require_gpu()
    B, gamma, V, r = 3, 3, 500, 16
    wl = workloads.make_markov(_markov_cfg("f32", "bf16", 5), B=B, gamma=gamma, V=V, r=r)
    x0 = wl["x0"].copy()
    x0[1] = V + 3
    g = host(sd.spec_draft_sample_markov(dev(wl["U"]), dev(x0), dev(wl["W1"], "bf16"),
                                         dev(wl["W2"], "bf16"), 1.0, seed=2))
    assert np.all(g["tokens"][1] == -1)
    assert np.all(g["tokens"][[0, 2]] >= 0)


def _rnn_cfg(seed, w_std):
    cfg = dict(workloads.CONFIGS["rnn-32k-b64"])
    cfg.update(data_seed=seed, w_std=w_std)
    return cfg


@pytest.mark.parametrize("B,gamma,V,r,d,udt,T,w_std", [
    (5, 4, 3000, 32, 64, "f32", 1.0, 0.3),
    (70, 3, 2500, 256, 512, "bf16", 1.0, 0.05),
    (3, 3, 1200, 16, 8, "f32", 0.0, 0.3),
])
def test_rnn_draft_parity(orc, B, gamma, V, r, d, udt, T, w_std):
    sd = require_gpu()
    note(f"rnn draft B={B} gamma={gamma} V={V} r={r} d={d} T={T}")
    cfg = _rnn_cfg(200 + B, w_std)
    cfg["logit_dtype"] = udt
    wl = workloads.make_rnn(cfg, B=B, gamma=gamma, V=V, r=r, d=d)
    seed = 31
    g = host(sd.spec_draft_sample_rnn(
        dev(wl["U"], udt), dev(wl["x0"]), dev(wl["H"], "bf16"), dev(wl["W1"], "bf16"),
        dev(wl["W2"], "bf16"), dev(wl["Wg"], "bf16"), dev(wl["Wc"], "bf16"), dev(wl["Wo"], "bf16"),
        T, seed=seed))
    f = {n: workloads.as_f64(wl[n], "bf16") for n in ("W1", "W2", "Wg", "Wc", "Wo")}
    u = orc.draft_uniforms(seed, 0, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], udt)
        hb = workloads.as_f64(wl["H"][b], "bf16")
        o = orc.draft_rnn(Ub, hb, f["W1"], f["W2"], f["Wg"], f["Wc"], f["Wo"], wl["x0"][b], T, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, T, u[b], f"b={b}",
                                      tally)
    note(f"  {tally.as_dict()}")
