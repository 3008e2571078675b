"""Pins of the oracle's lossless verification (VESSL "Speculative Decoding
Part 1": one speculative cycle, acceptance rule, residual distribution,
lossless theorem, closed form of alpha, expected tokens per cycle).

* Lossless theorem: the exact law of each emitted token, obtained by
  brute-force enumeration of the draft token and fine uniform grids, equals
  the target distribution p (computed with scipy).
* Closed form of alpha: Monte-Carlo acceptance frequency equals
  sum_u min(p(u), q(u)) computed with numpy; the TV identity holds.
* E[tau] = (1 - alpha^(gamma+1)) / (1 - alpha) and the truncated geometric
  law under i.i.d. acceptance.
* tau >= 1, tau <= L + 1; temperature 0 reduces to a top-1 match; p == q
  accepts everything; disjoint supports accept nothing.
"""
import numpy as np
import pytest
from scipy import special, stats


def _q_probs(l, T=1.0):
    return special.softmax(np.asarray(l, dtype=np.float64) / T)


def _accept_measure(orc, P, Q, draft, pos, grid, prefix_u=0.0, T=1.0):
    """Fraction of ratio-test uniforms on a midpoint grid that accept the
    draft token at position pos (earlier positions forced to accept with
    u = prefix_u = 0, which accepts any token with p > 0)."""
    L = len(draft)
    acc = 0
    for i in range(grid):
        ut = np.full(L, prefix_u)
        ut[pos] = (i + 0.5) / grid
        ut[pos + 1:] = 1.0 - 2**-24
        res = orc.verify(P, Q, draft, T, ut, 0.5)
        acc += res["n"] > pos
    return acc / grid


def _final_law(orc, P, Q, draft, ut, grid, V, T=1.0):
    """Law of the final (corrected or bonus) token over a uniform grid."""
    law = np.zeros(V)
    for j in range(grid):
        res = orc.verify(P, Q, draft, T, ut, (j + 0.5) / grid)
        law[res["out"][res["n"]]] += 1.0 / grid
    return law


# Temperatures other than 1 (the sampling temperature applies to p and q
# alike: the theorem holds for the two distributions at whatever temperature
# both are taken), so that dropping T from either normaliser, from q in the
# ratio test or from q in the residual fails a pin.
TEMPS = [1.0, 0.5, 0.7, 1.3, 2.0]


@pytest.mark.parametrize("T", TEMPS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lossless_by_enumeration_single_position(orc, seed, T):
    rng = np.random.default_rng(seed)
    V = 5
    P = rng.standard_normal((2, V)) * 1.5
    Q = rng.standard_normal((1, V)) * 1.5
    p0, q0 = _q_probs(P[0], T), _q_probs(Q[0], T)
    grid = 1 << 12
    law = np.zeros(V)
    for x in range(V):
        a = _accept_measure(orc, P, Q, [x], 0, grid, T=T)
        corr = _final_law(orc, P, Q, [x], np.array([1.0 - 2**-24]), grid, V, T) if a < 1 else 0
        law[x] += q0[x] * a
        law += q0[x] * (1 - a) * corr
    # grid error: <= 1/grid for the acceptance measure, <= V/grid for the law
    assert np.max(np.abs(law - p0)) < (V + 2) / grid
    # and the acceptance probability is the closed form sum min(p, q)
    acc = sum(q0[x] * _accept_measure(orc, P, Q, [x], 0, grid, T=T) for x in range(V))
    assert abs(acc - np.minimum(p0, q0).sum()) < 2 / grid


@pytest.mark.parametrize("T", TEMPS)
def test_lossless_second_position_and_bonus(orc, T):
    rng = np.random.default_rng(4)
    V = 4
    P = rng.standard_normal((3, V))
    Q = rng.standard_normal((2, V))
    p1, q1, p2 = _q_probs(P[1], T), _q_probs(Q[1], T), _q_probs(P[2], T)
    grid = 1 << 11
    x0 = int(np.argmax(_q_probs(P[0])))   # p(x0) > 0, accepted when u = 0
    law1 = np.zeros(V)
    bonus = None
    for x in range(V):
        draft = [x0, x]
        a = _accept_measure(orc, P, Q, draft, 1, grid, T=T)
        if a < 1:
            corr = _final_law(orc, P, Q, draft, np.array([0.0, 1.0 - 2**-24]), grid, V, T)
            law1 += q1[x] * (1 - a) * corr
        law1[x] += q1[x] * a
        if bonus is None and a > 0:
            bonus = _final_law(orc, P, Q, draft, np.array([0.0, 0.0]), grid, V, T)
    assert np.max(np.abs(law1 - p1)) < (V + 2) / grid
    # all accepted: the bonus token follows p at slot L (not slot L-1)
    assert np.max(np.abs(bonus - p2)) < (V + 1) / grid


@pytest.mark.parametrize("T", [0.5, 0.7, 1.3, 2.0])
def test_verify_outputs_at_temperature(orc, T):
    """Normalisers and acceptance probabilities at T != 1 against scipy's
    logsumexp and numpy softmax ratios of the rows divided by T."""
    rng = np.random.default_rng(41)
    V, L = 300, 5
    P = rng.standard_normal((L + 1, V)) * 3
    Q = P[:L] + rng.standard_normal((L, V))
    draft = rng.integers(0, V, size=L)
    res = orc.verify(P, Q, draft, T, np.zeros(L), 0.5)
    assert np.allclose(res["logZp"], special.logsumexp(P / T, axis=1), rtol=0, atol=1e-12)
    assert np.allclose(res["logZq"], special.logsumexp(Q / T, axis=1), rtol=0, atol=1e-12)
    p = special.softmax(P[:L] / T, axis=1)[np.arange(L), draft]
    q = special.softmax(Q / T, axis=1)[np.arange(L), draft]
    assert np.allclose(res["accept_prob"], np.minimum(1.0, p / q), rtol=1e-12, atol=0)
    # the first rejection follows the ratio tests: u = 0 accepts all, u just
    # below 1 rejects the first position whose min(1, p/q) < 1 - 2^-24
    res1 = orc.verify(P, Q, draft, T, np.full(L, 1.0 - 2**-24), 0.5)
    want = next((k for k in range(L) if (1.0 - 2**-24) * q[k] >= p[k]), L)
    assert res1["n"] == want
    assert res["n"] == L


@pytest.mark.parametrize("T", [0.5, 0.7, 1.3, 2.0])
def test_residual_weights_at_temperature(orc, T):
    rng = np.random.default_rng(43)
    V = 200
    lp = rng.standard_normal(V) * 2
    lq = lp + rng.standard_normal(V)
    w, R = orc.residual_weights(lp, lq, T, special.logsumexp(lp / T), special.logsumexp(lq / T))
    want = np.maximum(0.0, special.softmax(lp / T) - special.softmax(lq / T))
    assert np.allclose(w, want, rtol=1e-12, atol=1e-16)
    assert abs(R - want.sum()) < 1e-13
    # the residual mass is the total variation at that temperature
    assert abs(R - 0.5 * np.abs(special.softmax(lp / T) - special.softmax(lq / T)).sum()) < 1e-13


def test_lossless_monte_carlo_chi_square(orc):
    rng = np.random.default_rng(17)
    V = 8
    P = rng.standard_normal((2, V)) * 2
    Q = rng.standard_normal((1, V)) * 2
    q0 = _q_probs(Q[0])
    cq = np.cumsum(q0)
    n = 20000
    counts = np.zeros(V)
    for t in range(n):
        x = int(np.searchsorted(cq, orc.uniform(3, 0, t, 0, 0) * cq[-1], side="right"))
        res = orc.verify(P, Q, [x], 1.0, [orc.uniform(3, 0, t, 0, 1)], orc.uniform(3, 0, t, 0, 2))
        counts[res["out"][0]] += 1
    assert stats.chisquare(counts, _q_probs(P[0]) * n).pvalue > 1e-4


@pytest.mark.parametrize("T", [0.5, 0.7, 1.3, 2.0])
def test_alpha_tv_at_temperature(orc, T):
    rng = np.random.default_rng(45)
    V = 400
    lp = rng.standard_normal(V) * 2
    lq = lp + rng.standard_normal(V)
    p, q = special.softmax(lp / T), special.softmax(lq / T)
    alpha, tv = orc.alpha_tv(lp, lq, T)
    assert abs(alpha - np.minimum(p, q).sum()) < 1e-13
    assert abs(tv - 0.5 * np.abs(p - q).sum()) < 1e-13
    # temperature moves alpha: at T = 1 it differs from the value at T
    a1, _ = orc.alpha_tv(lp, lq, 1.0)
    assert abs(a1 - alpha) > 1e-3


def test_alpha_identity_and_frequency(orc):
    rng = np.random.default_rng(21)
    V = 50
    lp = rng.standard_normal(V) * 2
    lq = lp + rng.standard_normal(V)
    p, q = _q_probs(lp), _q_probs(lq)
    alpha, tv = orc.alpha_tv(lp, lq)
    assert abs(alpha - np.minimum(p, q).sum()) < 1e-13
    assert abs(alpha - (1 - tv)) < 1e-13
    assert abs(tv - 0.5 * np.abs(p - q).sum()) < 1e-13
    n = 20000
    cq = np.cumsum(q)
    acc = 0
    P = np.stack([lp, lp])
    Q = lq[None, :]
    for t in range(n):
        x = int(np.searchsorted(cq, orc.uniform(5, 0, t, 0, 0) * cq[-1], side="right"))
        res = orc.verify(P, Q, [x], 1.0, [orc.uniform(5, 0, t, 0, 1)], 0.5)
        acc += res["n"]
    sd = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(acc / n - alpha) < 4 * sd


def test_expected_tau_iid_acceptance(orc):
    # identical p rows and identical q rows at every position, draft tokens
    # drawn independently from q: acceptance is i.i.d. Bernoulli(alpha).
    rng = np.random.default_rng(23)
    V, gamma = 30, 5
    lp = rng.standard_normal(V) * 2
    lq = lp + 0.8 * rng.standard_normal(V)
    p, q = _q_probs(lp), _q_probs(lq)
    alpha = np.minimum(p, q).sum()
    P = np.tile(lp, (gamma + 1, 1))
    Q = np.tile(lq, (gamma, 1))
    n = 6000
    cq = np.cumsum(q)
    tau = np.zeros(n, dtype=int)
    for t in range(n):
        draft = [int(np.searchsorted(cq, orc.uniform(8, 0, t, k, 0) * cq[-1], side="right"))
                 for k in range(gamma)]
        ut = [orc.uniform(8, 0, t, k, 1) for k in range(gamma)]
        res = orc.verify(P, Q, draft, 1.0, ut, orc.uniform(8, 0, t, 0, 2))
        tau[t] = res["n"] + 1
    assert tau.min() >= 1 and tau.max() <= gamma + 1
    e_tau = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(tau.mean() - e_tau) < 4 * tau.std() / np.sqrt(n)
    law = np.array([alpha ** (j - 1) * (1 - alpha) for j in range(1, gamma + 1)] + [alpha ** gamma])
    counts = np.bincount(tau, minlength=gamma + 2)[1:]
    assert stats.chisquare(counts, law * n).pvalue > 1e-4


def test_greedy_is_top1_match_and_seed_free(orc):
    rng = np.random.default_rng(31)
    V, L = 40, 6
    for trial in range(30):
        P = rng.integers(-4, 4, size=(L + 1, V)).astype(float)   # exact ties happen
        Q = rng.standard_normal((L, V))
        draft = [int(np.argmax(P[k])) if rng.random() < 0.7 else int(rng.integers(V))
                 for k in range(L)]
        want_n = L
        for k in range(L):
            if draft[k] != int(np.argmax(P[k])):
                want_n = k
                break
        outs = []
        for s in range(3):
            res = orc.verify(P, Q, draft, 0.0, rng.random(L), rng.random())
            assert res["n"] == want_n
            assert res["out"][want_n] == int(np.argmax(P[want_n]))
            assert list(res["out"][:want_n]) == draft[:want_n]
            outs.append(res["out"].tolist())
        assert outs[0] == outs[1] == outs[2]


def test_identical_distributions_accept_everything(orc):
    rng = np.random.default_rng(33)
    V, L = 64, 7
    Q = rng.standard_normal((L, V)) * 3
    P = np.vstack([Q, rng.standard_normal((1, V))])
    for t in range(50):
        draft = rng.integers(0, V, size=L)
        res = orc.verify(P, Q, draft, 1.0, rng.random(L), rng.random())
        assert res["n"] == L
        assert np.all(res["accept_prob"] == 1.0)
        assert list(res["out"][:L]) == draft.tolist()


def test_disjoint_supports_accept_nothing(orc):
    V, L = 10, 3
    P = np.full((L + 1, V), -np.inf)
    Q = np.full((L, V), -np.inf)
    P[:, :5] = np.arange(5) * 0.3
    Q[:, 5:] = 0.0
    p0 = _q_probs(P[0])
    n = 4000
    counts = np.zeros(V)
    for t in range(n):
        draft = [5 + (t + k) % 5 for k in range(L)]
        res = orc.verify(P, Q, draft, 1.0, [orc.uniform(1, 0, t, k, 1) for k in range(L)],
                         orc.uniform(1, 0, t, 0, 2))
        assert res["n"] == 0 and res["out"][1] == -1
        counts[res["out"][0]] += 1
    assert counts[5:].sum() == 0
    assert stats.chisquare(counts[:5], p0[:5] * n).pvalue > 1e-4


def test_zero_length_gives_bonus_from_first_row(orc):
    rng = np.random.default_rng(35)
    P = rng.standard_normal((1, 6))
    w = np.exp(P[0] - P[0].max())
    for u in rng.random(50):
        res = orc.verify(P, None, [], 1.0, [], u)
        assert res["n"] == 0
        assert res["out"][0] == int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))


def test_tau_bounds_on_random_requests(orc):
    rng = np.random.default_rng(37)
    for t in range(100):
        V = int(rng.integers(2, 30))
        L = int(rng.integers(0, 6))
        P = rng.standard_normal((L + 1, V)) * 2
        Q = rng.standard_normal((L, V)) * 2 if L else None
        draft = rng.integers(0, V, size=L)
        res = orc.verify(P, Q, draft, 1.0, rng.random(L), rng.random())
        tau = res["n"] + 1
        assert 1 <= tau <= L + 1
        assert res["out"][res["n"]] >= 0
        assert np.all(res["out"][res["n"] + 1:] == -1)
