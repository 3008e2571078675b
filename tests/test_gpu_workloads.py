"""GPU parity of the whole cycle (draft then verify) on the named workloads at
their full sizes, in the launch configuration the benchmark times.  The
oracle checks every request of the small workloads and a sample of requests
of the large ones; properties that hold at any size are checked on all."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _check_properties(gd, gv, V, lens, gamma):
    toks = gd["tokens"]
    assert np.all((toks >= 0) & (toks < V))
    n = gv["accepted"]
    L = np.full(len(n), gamma) if lens is None else lens
    assert np.all(n >= 0) and np.all(n <= L)                      # 1 <= tau <= L + 1
    for b in range(len(n)):
        row = gv["out_tokens"][b]
        assert np.array_equal(row[:n[b]], toks[b, :n[b]])
        assert 0 <= row[n[b]] < V
        assert np.all(row[n[b] + 1:] == -1)


def _run_markov_cycle(orc, wl, T, seed, sample, p_packed=False):
    sd = require_gpu()
    B, gamma, V = wl["B"], wl["gamma"], wl["V"]
    lb, wb = wl["logit_dtype"], wl["w_dtype"]
    U, P = dev(wl["U"], lb), dev(wl["P"], lb)
    W1, W2, x0 = dev(wl["W1"], wb), dev(wl["W2"], wb), dev(wl["x0"])
    lens = wl["lens"]
    d = sd.spec_draft_sample_markov(U, x0, W1, W2, T, seed=seed)
    if lens is None:
        v = sd.spec_verify(P, d["q_logits"], d["tokens"], T, seed=seed)
    else:
        v = sd.spec_verify(P, d["q_logits"], d["tokens"], T, lens=dev(lens),
                           p_row_off=dev(workloads.packed_offsets(lens + 1)), seed=seed)
    gd, gv = host(d), host(v)
    _check_properties(gd, gv, V, lens, gamma)
    # determinism of the whole cycle
    d2 = sd.spec_draft_sample_markov(U, x0, W1, W2, T, seed=seed)
    assert torch.equal(d2["tokens"], d["tokens"]) and torch.equal(d2["q_logits"], d["q_logits"])
    del U, P, d, d2, v
    torch.cuda.empty_cache()

    W1f, W2f = workloads.as_f64(wl["W1"], wb), workloads.as_f64(wl["W2"], wb)
    ud = orc.draft_uniforms(seed, 0, B, gamma)
    uv = orc.verify_uniforms(seed, 0, B, gamma)
    p_off = None if lens is None else workloads.packed_offsets(lens + 1)
    tally_d, tally_v = compare.Tally(), compare.Tally()
    for b in sample:
        Ub = workloads.as_f64(wl["U"][b], lb)
        o = orc.draft_markov(Ub, W1f, W2f, wl["x0"][b], T, ud[b])
        same = compare.compare_draft_request(o, Ub, {k: x[b] for k, x in gd.items()}, T, ud[b],
                                             f"draft b={b}", tally_d)
        if not same:
            continue
        L = gamma if lens is None else int(lens[b])
        Pb = workloads.as_f64(wl["P"][b] if lens is None else wl["P"][p_off[b]:p_off[b] + L + 1], lb)
        compare.compare_verify_request(Pb, o["q_logits"][:L], o["tokens"][:L], T, uv[b, :L],
                                       uv[b, gamma], {k: x[b] for k, x in gv.items()},
                                       f"verify b={b}", tally_v)
    note(f"  draft {tally_d.as_dict()}\n  verify {tally_v.as_dict()}\n"
         f"  mean tau {float(gv['accepted'].mean() + 1):.3f}")
    return gv


@pytest.mark.parametrize("name,T,sample", [
    ("markov-tiny", 1.0, "all"),
    ("markov-32k-b32", 1.0, "all"),
    ("markov-32k-b32", 0.0, "all"),
])
def test_small_workloads_every_request(orc, name, T, sample):
    wl = workloads.make_markov(workloads.CONFIGS[name], T=T)
    note(f"{name} T={T} B={wl['B']}")
    _run_markov_cycle(orc, wl, T, seed=0, sample=range(wl["B"]))


@pytest.mark.parametrize("B,sigma", [(128, 1.0), (32, 0.3)])
def test_markov_152k_sampled(orc, B, sigma):
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    cfg["sigma"] = sigma
    wl = workloads.make_markov(cfg, B=B)
    note(f"markov-152k B={B} sigma={sigma}")
    _run_markov_cycle(orc, wl, 1.0, seed=0, sample=[0, B // 2 + 1, B - 1])


def test_ragged_128k_sampled(orc):
    wl = workloads.make_markov(workloads.CONFIGS["ragged-128k-b256"])
    note(f"ragged-128k B={wl['B']} lens mean {wl['lens'].mean():.2f}")
    _run_markov_cycle(orc, wl, 1.0, seed=0, sample=[0, 101, 255])


def test_rnn_32k_sampled(orc):
    sd = require_gpu()
    wl = workloads.make_rnn(workloads.CONFIGS["rnn-32k-b64"])
    B, gamma, V = wl["B"], wl["gamma"], wl["V"]
    note(f"rnn-32k B={B}")
    lb = wl["logit_dtype"]
    d = sd.spec_draft_sample_rnn(dev(wl["U"], lb), dev(wl["x0"]), dev(wl["H"], "bf16"),
                                 dev(wl["W1"], "bf16"), dev(wl["W2"], "bf16"), dev(wl["Wg"], "bf16"),
                                 dev(wl["Wc"], "bf16"), dev(wl["Wo"], "bf16"), 1.0, seed=0)
    v = sd.spec_verify(dev(wl["P"], lb), d["q_logits"], d["tokens"], 1.0, seed=0)
    gd, gv = host(d), host(v)
    _check_properties(gd, gv, V, None, gamma)
    f = {n: workloads.as_f64(wl[n], "bf16") for n in ("W1", "W2", "Wg", "Wc", "Wo")}
    ud = orc.draft_uniforms(0, 0, B, gamma)
    uv = orc.verify_uniforms(0, 0, B, gamma)
    td, tv = compare.Tally(), compare.Tally()
    for b in [0, 31, 63]:
        Ub = workloads.as_f64(wl["U"][b], lb)
        o = orc.draft_rnn(Ub, workloads.as_f64(wl["H"][b], "bf16"), f["W1"], f["W2"], f["Wg"],
                          f["Wc"], f["Wo"], wl["x0"][b], 1.0, ud[b])
        if compare.compare_draft_request(o, Ub, {k: x[b] for k, x in gd.items()}, 1.0, ud[b],
                                         f"draft b={b}", td):
            compare.compare_verify_request(workloads.as_f64(wl["P"][b], lb), o["q_logits"],
                                           o["tokens"], 1.0, uv[b, :gamma], uv[b, gamma],
                                           {k: x[b] for k, x in gv.items()}, f"verify b={b}", tv)
    note(f"  draft {td.as_dict()}\n  verify {tv.as_dict()}")


def test_rnn_32k_qfree_sampled(orc):
    """The RNN workload at full size on the q-free path (the benchmark's
    cycle): q-free draft, then spec_verify_rnn; requests spread over the
    batch compared with the oracle's draft and verification."""
    sd = require_gpu()
    wl = workloads.make_rnn(workloads.CONFIGS["rnn-32k-b64"])
    B, gamma, V = wl["B"], wl["gamma"], wl["V"]
    note(f"rnn-32k q-free B={B}")
    lb = wl["logit_dtype"]
    U, W2 = dev(wl["U"], lb), dev(wl["W2"], "bf16")
    d = sd.spec_draft_sample_rnn(U, dev(wl["x0"]), dev(wl["H"], "bf16"), dev(wl["W1"], "bf16"),
                                 W2, dev(wl["Wg"], "bf16"), dev(wl["Wc"], "bf16"),
                                 dev(wl["Wo"], "bf16"), 1.0, q_free=True, seed=7)
    v = sd.spec_verify_rnn(dev(wl["P"], lb), U, d["cond"], W2, d["tokens"], d["q_logZ"],
                           d["q_tok_prob"], 1.0, seed=7, offset=1)
    gd = host({k: x for k, x in d.items() if k != "cond"})
    gv = host(v)
    _check_properties(gd, gv, V, None, gamma)
    f = {n: workloads.as_f64(wl[n], "bf16") for n in ("W1", "W2", "Wg", "Wc", "Wo")}
    ud = orc.draft_uniforms(7, 0, B, gamma)
    uv = orc.verify_uniforms(7, 1, B, gamma)
    td, tv = compare.Tally(), compare.Tally()
    for b in [0, 9, 31, 50, 63]:
        Ub = workloads.as_f64(wl["U"][b], lb)
        o = orc.draft_rnn(Ub, workloads.as_f64(wl["H"][b], "bf16"), f["W1"], f["W2"], f["Wg"],
                          f["Wc"], f["Wo"], wl["x0"][b], 1.0, ud[b])
        if compare.compare_draft_request(o, Ub, {k: x[b] for k, x in gd.items()}, 1.0, ud[b],
                                         f"draft b={b}", td, check_logits=False):
            gvb = {k: x[b] for k, x in gv.items()}
            gvb["q_logZ"] = gd["q_logZ"][b]
            compare.compare_verify_request(workloads.as_f64(wl["P"][b], lb), o["q_logits"],
                                           o["tokens"], 1.0, uv[b, :gamma], uv[b, gamma], gvb,
                                           f"verify b={b}", tv)
    note(f"  draft {td.as_dict()}\n  verify {tv.as_dict()}")
    assert tv.requests >= 4
