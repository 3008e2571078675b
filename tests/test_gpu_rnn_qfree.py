"""GPU parity of the q-free RNN draft ("[논문리뷰] DSpark", §1.2 RNN-head
equation: the bias W2^T o_k with o_k from the gated state) and of its
verification (spec_verify_rnn), against the oracle's RNN draft and chain
verification on the same seeded inputs: tokens with the band rule, log Z_k
and q(x_k) against the oracle's, and the cycle's accepted counts and tokens
for requests whose draft matched."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _rnn_cfg(seed, w_std):
    cfg = dict(workloads.CONFIGS["rnn-32k-b64"])
    cfg.update(data_seed=seed, w_std=w_std)
    return cfg


def _device(wl, udt):
    return dict(U=dev(wl["U"], udt), x0=dev(wl["x0"]), H=dev(wl["H"], "bf16"),
                W1=dev(wl["W1"], "bf16"), W2=dev(wl["W2"], "bf16"), Wg=dev(wl["Wg"], "bf16"),
                Wc=dev(wl["Wc"], "bf16"), Wo=dev(wl["Wo"], "bf16"))


@pytest.mark.parametrize("B,gamma,V,r,d,udt,T,w_std", [
    (5, 4, 3000, 32, 64, "f32", 1.0, 0.3),
    (70, 3, 2500, 256, 512, "bf16", 1.0, 0.05),
    (9, 5, 4099, 64, 128, "bf16", 0.7, 0.2),
    (3, 3, 1200, 16, 8, "f32", 0.0, 0.3),
])
def test_rnn_qfree_draft_parity(orc, B, gamma, V, r, d, udt, T, w_std):
    sd = require_gpu()
    note(f"q-free rnn draft B={B} gamma={gamma} V={V} r={r} d={d} T={T}")
    cfg = _rnn_cfg(400 + B, w_std)
    cfg["logit_dtype"] = udt
    wl = workloads.make_rnn(cfg, B=B, gamma=gamma, V=V, r=r, d=d)
    t = _device(wl, udt)
    seed = 37
    g = host({k: v for k, v in sd.spec_draft_sample_rnn(
        t["U"], t["x0"], t["H"], t["W1"], t["W2"], t["Wg"], t["Wc"], t["Wo"], T, q_free=True,
        seed=seed).items() if k != "cond"})
    assert "q_logits" not in g
    f = {n: workloads.as_f64(wl[n], "bf16") for n in ("W1", "W2", "Wg", "Wc", "Wo")}
    u = orc.draft_uniforms(seed, 0, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], udt)
        hb = workloads.as_f64(wl["H"][b], "bf16")
        o = orc.draft_rnn(Ub, hb, f["W1"], f["W2"], f["Wg"], f["Wc"], f["Wo"], wl["x0"][b], T, u[b])
        compare.compare_draft_request(o, Ub, {k: v[b] for k, v in g.items()}, T, u[b], f"b={b}",
                                      tally, check_logits=False)
    note(f"  {tally.as_dict()}")


def test_rnn_qfree_matches_materialised_draft():
    """Same inputs and uniforms: the q-free draft's tokens equal the
    materialised draft's (both sample the same fp32 logits), q_logZ and q(x)
    agree to fp32 rounding."""
    sd = require_gpu()
    B, gamma, V, r, d = 33, 4, 5000, 128, 256
    note(f"q-free vs materialised rnn draft B={B} gamma={gamma} V={V}")
    wl = workloads.make_rnn(_rnn_cfg(77, 0.1), B=B, gamma=gamma, V=V, r=r, d=d)
    t = _device(wl, "f32")
    args = (t["U"], t["x0"], t["H"], t["W1"], t["W2"], t["Wg"], t["Wc"], t["Wo"], 1.0)
    a = host(sd.spec_draft_sample_rnn(*args, seed=5))
    bq = sd.spec_draft_sample_rnn(*args, q_free=True, seed=5)
    b = host({k: v for k, v in bq.items() if k != "cond"})
    same = (a["tokens"] == b["tokens"]).mean()
    note(f"  token agreement {same:.4f}")
    assert same > 0.97            # a draw may sit on a CDF boundary; later positions follow it
    first = a["tokens"][:, 0] == b["tokens"][:, 0]
    assert first.mean() > 0.99
    np.testing.assert_allclose(b["q_logZ"][:, 0], a["q_logZ"][:, 0], atol=2e-5, rtol=0)
    ok = first
    np.testing.assert_allclose(b["q_tok_prob"][ok, 0], a["q_tok_prob"][ok, 0], rtol=2e-5, atol=0)


@pytest.mark.parametrize("B,G,V,r,d,T,pdt", [
    (24, 4, 3000, 64, 128, 1.0, "bf16"),
    (16, 5, 4096, 128, 256, 0.8, "f32"),
    (12, 3, 2000, 32, 64, 0.0, "bf16"),
])
def test_rnn_qfree_cycle_against_oracle(orc, B, G, V, r, d, T, pdt):
    """q-free RNN draft -> spec_verify_rnn, compared with the oracle's draft
    and chain verification (the oracle's own draft logits stand for q)."""
    sd = require_gpu()
    note(f"q-free rnn cycle B={B} G={G} V={V} r={r} d={d} T={T} P={pdt}")
    cfg = _rnn_cfg(900 + V, 0.15)
    cfg["logit_dtype"] = pdt
    wl = workloads.make_rnn(cfg, B=B, gamma=G, V=V, r=r, d=d)
    t = _device(wl, pdt)
    seed = 4321
    dr = sd.spec_draft_sample_rnn(t["U"], t["x0"], t["H"], t["W1"], t["W2"], t["Wg"], t["Wc"],
                                  t["Wo"], T, q_free=True, seed=seed, offset=0)
    vr = sd.spec_verify_rnn(dev(wl["P"], pdt), t["U"], dr["cond"], t["W2"], dr["tokens"],
                            dr["q_logZ"], dr["q_tok_prob"], T, seed=seed, offset=1)
    gd = host({k: v for k, v in dr.items() if k != "cond"})
    gv = host(vr)
    f = {n: workloads.as_f64(wl[n], "bf16") for n in ("W1", "W2", "Wg", "Wc", "Wo")}
    ud = orc.draft_uniforms(seed, 0, B, G)
    uv = orc.verify_uniforms(seed, 1, B, G)
    Pf = workloads.as_f64(wl["P"], pdt)
    td, tv = compare.Tally(), compare.Tally()
    for b in range(B):
        Ub = workloads.as_f64(wl["U"][b], pdt)
        hb = workloads.as_f64(wl["H"][b], "bf16")
        o = orc.draft_rnn(Ub, hb, f["W1"], f["W2"], f["Wg"], f["Wc"], f["Wo"], wl["x0"][b], T,
                          ud[b])
        same = compare.compare_draft_request(o, Ub, {k: v[b] for k, v in gd.items()}, T, ud[b],
                                             f"draft b={b}", td, check_logits=False)
        if not same and not np.array_equal(gd["tokens"][b], o["tokens"]):
            continue
        d_ = {k: v[b] for k, v in gv.items()}
        d_["q_logZ"] = gd["q_logZ"][b]
        compare.compare_verify_request(Pf[b], o["q_logits"], o["tokens"], T, uv[b, :G], uv[b, G],
                                       d_, f"verify b={b}", tv)
    note(f"  draft {td.as_dict()} verify {tv.as_dict()} accepted={gv['accepted'].tolist()}")
    assert tv.requests >= B - 1
    if T > 0:
        assert (gv["accepted"] < G).any()     # some residual draws happened
