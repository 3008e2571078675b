"""Pins of the oracle's row primitives: softmax normaliser, inverse-CDF draw,
greedy argmax and CDF intervals, against scipy/numpy library routines,
closed forms and brute force."""
import numpy as np
import pytest
from scipy import special, stats


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_logz_matches_logsumexp(orc, T):
    rng = np.random.default_rng(1)
    for V in [1, 7, 1000, 32000]:
        l = rng.standard_normal(V) * 4 - 1.1 * np.log(np.arange(1, V + 1))
        w, Z, logZ = orc.softmax_weights(l, T)
        assert abs(logZ - special.logsumexp(l / T)) <= 1e-12 * max(1.0, abs(logZ))
        assert np.allclose(w / Z, special.softmax(l / T), rtol=1e-12, atol=0)


def test_softmax_special_cases(orc):
    V = 513
    w, Z, logZ = orc.softmax_weights(np.full(V, 2.5), 1.0)
    assert Z == V and np.all(w == 1.0)
    assert abs(logZ - (2.5 + np.log(V))) < 1e-12
    l = np.zeros(V)
    l[17] = 1000.0
    w, Z, _ = orc.softmax_weights(l, 1.0)
    assert w[17] / Z == 1.0 and np.all(np.delete(w, 17) == 0.0)
    l = np.array([-np.inf, 0.0, -np.inf, 0.0])
    w, Z, _ = orc.softmax_weights(l, 1.0)
    assert w.tolist() == [0.0, 1.0, 0.0, 1.0]
    w, Z, logZ = orc.softmax_weights(np.full(4, -np.inf), 1.0)
    assert Z == 0.0 and logZ == -np.inf


def test_inverse_cdf_matches_searchsorted(orc):
    rng = np.random.default_rng(2)
    for V in [1, 2, 9, 1000, 20000]:
        l = rng.standard_normal(V) * 3
        w, Z, _ = orc.softmax_weights(l, 1.0)
        cs = np.cumsum(w)
        for u in list(rng.random(200)) + [0.0, 1 - 2**-24]:
            tok, thr, margin = orc.inverse_cdf(w, Z, u)
            want = int(np.searchsorted(cs, u * Z, side="right"))
            assert tok == want
            assert 0.0 <= margin <= 0.5 * w[tok] / Z + 1e-15
            lo, hi = orc.cdf_interval(w, tok)
            assert lo <= thr < hi or (lo <= thr and abs(thr - hi) < 1e-15)


def test_inverse_cdf_skips_zero_weight_tokens(orc):
    w = np.array([0.0, 1.0, 0.0, 0.0, 3.0, 0.0])
    seen = set()
    for u in np.linspace(0, 1, 101)[:-1]:
        tok, _, _ = orc.inverse_cdf(w, w.sum(), u)
        seen.add(tok)
    assert seen == {1, 4}


def test_inverse_cdf_draws_follow_p(orc):
    # brute force on a tiny vocabulary: Philox uniforms, chi-square vs p
    l = np.array([0.3, -1.0, 2.0, 0.0, -3.0, 1.1, 0.7, -0.2])
    w, Z, _ = orc.softmax_weights(l, 1.0)
    p = special.softmax(l)
    n = 40000
    counts = np.zeros(8)
    for i in range(n):
        tok, _, _ = orc.inverse_cdf(w, Z, orc.uniform(99, 0, i, 0, 0))
        counts[tok] += 1
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_argmax_lowest_index_on_ties(orc):
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 50))
        l = rng.integers(-3, 3, size=V).astype(float)
        tok, gap = orc.argmax(l)
        assert tok == int(np.argmax(l))
        others = np.delete(l, tok)
        assert gap == (l[tok] - others.max() if V > 1 else np.inf)
