"""GPU statistical check of the lossless theorem ("Speculative Decoding Part 1",
section on the acceptance rule: a token drawn from q, kept when u q(x) < p(x)
and otherwise replaced by a draw from the normalised residual max(0, p - q),
follows p).

The timed path (q-free Markov draft, then spec_verify_markov) runs on a batch
of requests that all carry the same target rows p_0..p_gamma, which do not
depend on the context, so the batch is the trial axis:

* whatever the draft law, the token emitted at position j (by rows that reach
  j) follows p_j: chi-square of the emitted counts against p_j, at every
  position, for a draft whose rows depend on the previous token (random W1);
* with draft rows that do not depend on the context either (W1 = 0) the ratio
  tests are independent with chance alpha_k = sum min(p_k, q_k) (the oracle's
  closed form), so the accepted count n follows P(n = j) = alpha_0 ..
  alpha_{j-1} (1 - alpha_j) (j < gamma), P(n = gamma) = alpha_0 .. alpha_{gamma-1}:
  chi-square of n's histogram and a z-test of E[tau] = 1 + E[n].

The same counts tested against the draft law q instead of p must fail, so the
test can tell the two apart.  Inputs and uniforms are seeded; every p-value
is deterministic.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, note, require_gpu, torch

pytestmark = pytest.mark.gpu

scipy_stats = pytest.importorskip("scipy.stats")

PMIN = 1e-4      # a correct sampler passes at this level (fixed seeds: no flakiness)


def _chi2_pvalue(counts, probs):
    """Pearson chi-square p-value of counts against probs; categories with an
    expected count below 5 are pooled into one."""
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    exp = n * np.asarray(probs, dtype=np.float64)
    small = exp < 5.0
    c = np.append(counts[~small], counts[small].sum())
    e = np.append(exp[~small], exp[small].sum())
    keep = e > 0
    if (c[~keep] > 0).any():
        return 0.0            # mass where the law has none
    c, e = c[keep], e[keep]
    stat = float(((c - e) ** 2 / e).sum())
    return float(scipy_stats.chi2.sf(stat, df=len(c) - 1))


def _law(orc, row, T):
    w, Z, _ = orc.softmax_weights(row, T)
    return w / Z


def _cycle(sd, wl, T, seed):
    lb = wl["logit_dtype"]
    U, P = dev(wl["U"], lb), dev(wl["P"], lb)
    W1, W2, x0 = dev(wl["W1"], lb), dev(wl["W2"], lb), dev(wl["x0"])
    W2T = sd.spec_pack_w2(W2)
    d = sd.spec_draft_sample_markov(U, x0, W1, None, T, W2T=W2T, q_free=True, seed=seed, offset=1)
    v = sd.spec_verify_markov(P, U, x0, W1, None, d["tokens"], d["q_logZ"], d["q_tok_prob"], T,
                              W2T=W2T, seed=seed, offset=2)
    torch.cuda.synchronize()
    return (d["tokens"].cpu().numpy(), v["accepted"].cpu().numpy(), v["out_tokens"].cpu().numpy())


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_emitted_tokens_follow_target(orc, T):
    sd = require_gpu()
    B, gamma, V, r = 16384, 4, 256, 64
    note(f"lossless stats: emitted law, B={B} gamma={gamma} V={V} T={T}")
    wl = workloads.make_repeated_markov(B, gamma, V, r, seed=71, sigma=1.0, w_std=0.3)
    tokens, acc, out = _cycle(sd, wl, T, seed=2024)
    assert (acc >= 0).all() and (acc <= gamma).all()
    P1 = workloads.as_f64(wl["P1"], "bf16")
    U1 = workloads.as_f64(wl["U1"], "bf16")
    for j in range(gamma + 1):
        reach = acc >= j                       # rows that emit a token at position j
        toks = out[reach, j]
        assert (toks >= 0).all() and (toks < V).all()
        counts = np.bincount(toks, minlength=V)
        pv = _chi2_pvalue(counts, _law(orc, P1[j], T))
        note(f"  position {j}: {int(reach.sum())} tokens, chi-square p = {pv:.3g}")
        assert pv > PMIN, (j, pv)
    # power: position 0's emitted tokens are not drawn from the draft's law
    # (which, with the context-dependent head, is a mixture over the anchors;
    # the draft tokens themselves are)
    q0 = np.zeros(V)
    W1 = workloads.as_f64(wl["W1"], "bf16")
    W2 = workloads.as_f64(wl["W2"], "bf16")
    for x, cnt in zip(*np.unique(wl["x0"], return_counts=True)):
        q0 += cnt * _law(orc, U1[0] + W1[x] @ W2, T)
    q0 /= q0.sum()
    pv_draft = _chi2_pvalue(np.bincount(tokens[:, 0], minlength=V), q0)
    pv_wrong = _chi2_pvalue(np.bincount(out[:, 0], minlength=V), q0)
    note(f"  draft tokens vs q: p = {pv_draft:.3g}; emitted vs q: p = {pv_wrong:.3g}")
    assert pv_draft > PMIN
    assert pv_wrong < 1e-8


@pytest.mark.parametrize("T", [1.0, 1.3])
def test_accepted_length_law_iid(orc, T):
    sd = require_gpu()
    B, gamma, V, r = 16384, 6, 256, 64
    note(f"lossless stats: accepted-length law, B={B} gamma={gamma} V={V} T={T}")
    wl = workloads.make_repeated_markov(B, gamma, V, r, seed=73, sigma=0.8, w1_zero=True)
    _, acc, out = _cycle(sd, wl, T, seed=99)
    P1 = workloads.as_f64(wl["P1"], "bf16")
    U1 = workloads.as_f64(wl["U1"], "bf16")
    alpha = np.array([orc.alpha_tv(P1[k], U1[k], T)[0] for k in range(gamma)])
    law = np.empty(gamma + 1)
    run = 1.0
    for j in range(gamma):
        law[j] = run * (1.0 - alpha[j])
        run *= alpha[j]
    law[gamma] = run
    counts = np.bincount(acc, minlength=gamma + 1)
    pv = _chi2_pvalue(counts, law)
    e_tau = 1.0 + float((np.arange(gamma + 1) * law).sum())
    sd_n = float(np.sqrt(((np.arange(gamma + 1) - (e_tau - 1.0)) ** 2 * law).sum()))
    z = (1.0 + acc.mean() - e_tau) / (sd_n / np.sqrt(B))
    note(f"  alpha = {np.round(alpha, 4).tolist()}, counts = {counts.tolist()}")
    note(f"  chi-square p = {pv:.3g}; E[tau] {e_tau:.4f} vs mean {1.0 + acc.mean():.4f} (z = {z:.2f})")
    assert pv > PMIN
    assert abs(z) < 4.0
    # every emitted position still follows p_j
    for j in range(gamma + 1):
        reach = acc >= j
        assert _chi2_pvalue(np.bincount(out[reach, j], minlength=V), _law(orc, P1[j], T)) > PMIN
    # power: the law with the acceptance chances one notch higher is rejected
    alt = np.empty(gamma + 1)
    run = 1.0
    a2 = np.minimum(alpha + 0.05, 1.0)
    for j in range(gamma):
        alt[j] = run * (1.0 - a2[j])
        run *= a2[j]
    alt[gamma] = run
    assert _chi2_pvalue(counts, alt) < 1e-8
