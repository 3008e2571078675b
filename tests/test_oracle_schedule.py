"""Pins of the oracle's confidence head and hardware-aware prefix scheduler
(DSpark review, §2.1 "Confidence Head" and §2.2 "Hardware-Aware Prefix
Scheduler").

* Confidence head: zero weights give 1/2; a one-hot weight on one input of
  either block (hidden state or Markov embedding) gives scipy's expit of that
  input; negating w gives 1 - c; logits add over disjoint weight supports.
* Scheduler: on tiny cases whose best throughput over the admitted count is
  unimodal (log-concave SPS, or flat then 1/B), the chosen lengths reach the
  maximum of tau * SPS(B) over EVERY assignment of lengths, found by brute
  force; the admitted candidates are the global top-t by survival
  probability; constant SPS admits everything; an SPS table that is zero past
  B = R admits nothing; a hand-worked example; and on a table whose
  throughput falls then rises again, the search stops at the first fall.
"""
import itertools

import numpy as np
import pytest
from scipy import special


def test_confidence_zero_weights_is_half(orc):
    rng = np.random.default_rng(0)
    assert orc.confidence(rng.normal(size=7), rng.normal(size=3), np.zeros(10)) == 0.5


@pytest.mark.parametrize("i", [0, 4, 6, 7, 9])
def test_confidence_one_hot_weight_is_expit(orc, i):
    rng = np.random.default_rng(i)
    h, e = rng.normal(size=7) * 3, rng.normal(size=3) * 3
    w = np.zeros(10)
    w[i] = 1.0
    x = h[i] if i < 7 else e[i - 7]
    assert orc.confidence(h, e, w) == pytest.approx(special.expit(x), rel=1e-15, abs=0)


def test_confidence_symmetry_and_additive_logits(orc):
    rng = np.random.default_rng(3)
    h, e = rng.normal(size=64), rng.normal(size=16)
    w = rng.normal(size=80) * 0.2
    c = orc.confidence(h, e, w)
    assert orc.confidence(h, e, -w) == pytest.approx(1.0 - c, rel=1e-14)
    w1, w2 = w.copy(), w.copy()
    w1[40:] = 0.0
    w2[:40] = 0.0
    logit = special.logit
    assert logit(c) == pytest.approx(logit(orc.confidence(h, e, w1)) + logit(orc.confidence(h, e, w2)),
                                     rel=1e-12)


# --------------------------------------------------------------------------

def _survival(c):
    """a[r, j] = prod_{i <= j} c[r, i] from the float32 confidences, in fp64."""
    return np.cumprod(np.asarray(c, dtype=np.float64), axis=1)


def _theta(a, lens, sps):
    R = a.shape[0]
    B = R + int(np.sum(lens))
    tau = R + sum(a[r, :lens[r]].sum() for r in range(R))
    return tau * (sps[B] if B < len(sps) else 0.0), B, tau


def _brute_best(a, sps):
    R, g = a.shape
    best = -1.0
    for lens in itertools.product(range(g + 1), repeat=R):
        best = max(best, _theta(a, lens, sps)[0])
    return best


def _sps_tables(R, g):
    n = R * (g + 1) + 1
    B = np.arange(n, dtype=np.float64)
    yield 1000.0 * np.exp(-0.04 * B**2 / R)          # log-concave
    yield np.clip(900.0 - 35.0 * B, 1.0, None)        # linear (log-concave where positive)
    B0 = R + 1.5 * R
    yield np.where(B <= B0, 800.0, 800.0 * B0 / np.maximum(B, 1))   # memory- then compute-bound
    yield np.full(n, 500.0)                          # constant


@pytest.mark.parametrize("R,g,seed", [(1, 4, 0), (2, 3, 1), (3, 2, 2), (3, 3, 3), (4, 2, 4)])
def test_schedule_matches_brute_force(orc, R, g, seed):
    rng = np.random.default_rng(seed)
    for trial in range(6):
        c = rng.uniform(0.05, 1.0, size=(R, g)).astype(np.float32)
        if trial == 5:
            c[:, 1:] = 1.0   # equal survival along a request
        a = _survival(c)
        for sps in _sps_tables(R, g):
            lens, B, tau = orc.prefix_schedule(c, sps)
            th, B2, tau2 = _theta(a, lens, sps)
            assert B == B2
            assert tau == pytest.approx(tau2, rel=1e-7)
            assert th >= _brute_best(a, sps) * (1 - 1e-7)


def test_schedule_admits_global_top_t(orc):
    rng = np.random.default_rng(7)
    R, g = 24, 8
    c = rng.uniform(0.3, 1.0, size=(R, g)).astype(np.float32)
    sps = 1000.0 * np.exp(-0.002 * np.arange(R * (g + 1) + 1) ** 2 / R)
    lens, B, tau = orc.prefix_schedule(c, sps)
    a = _survival(c)
    taken = np.concatenate([a[r, :lens[r]] for r in range(R)])
    left = np.concatenate([a[r, lens[r]:] for r in range(R)])
    assert 0 < taken.size < R * g
    assert taken.min() >= left.max() * (1 - 1e-6)
    assert B == R + taken.size


def test_schedule_constant_sps_admits_everything(orc):
    rng = np.random.default_rng(8)
    c = rng.uniform(0.0, 1.0, size=(5, 6)).astype(np.float32)
    c[0] = 0.0   # zero survival is still no fall in throughput
    lens, B, tau = orc.prefix_schedule(c, np.full(5 * 7 + 1, 10.0))
    assert list(lens) == [6] * 5 and B == 35


def test_schedule_sps_zero_past_r_admits_nothing(orc):
    c = np.full((4, 3), 0.99, dtype=np.float32)
    lens, B, tau = orc.prefix_schedule(c, np.array([0, 0, 0, 0, 50.0]))
    assert list(lens) == [0] * 4 and B == 4 and tau == 4.0
    # the same with the table ending at B = R
    lens, B, tau = orc.prefix_schedule(c, np.array([0, 0, 0, 0, 50.0, 0.0, 0.0]))
    assert list(lens) == [0] * 4


def test_schedule_hand_worked_example(orc):
    # a = [[0.9, 0.45], [0.6, 0.54]]; order 0.9, 0.6, 0.54, 0.45.
    # Theta: B=2: 2*100 = 200; B=3: 2.9*100 = 290; B=4: 3.5*90 = 315;
    # B=5: 4.04*70 = 282.8 < 315 -> stop with lengths [1, 1].
    c = np.array([[0.9, 0.5], [0.6, 0.9]], dtype=np.float32)
    sps = np.array([0, 0, 100.0, 100.0, 90.0, 70.0, 60.0])
    lens, B, tau = orc.prefix_schedule(c, sps)
    assert list(lens) == [1, 1] and B == 4
    assert tau == pytest.approx(3.5, rel=1e-7)


def test_schedule_stops_at_first_fall(orc):
    # Throughput falls at B=3 then would rise again: the greedy search stops.
    c = np.ones((2, 3), dtype=np.float32)
    sps = np.array([0, 0, 100.0, 100.0, 60.0, 60.0, 60.0, 60.0])
    # tau = 2, 3, 4, 5, 6, 7 for B = 2..7: Theta = 200, 300, 240, 300, 360, 420
    lens, B, tau = orc.prefix_schedule(c, sps)
    assert B == 3 and tau == 3.0 and sorted(lens) == [0, 1]
    assert list(lens) == [1, 0]   # equal survival: the lower request first


def test_schedule_empty(orc):
    lens, B, tau = orc.prefix_schedule(np.zeros((3, 0), dtype=np.float32), np.full(4, 5.0))
    assert list(lens) == [0, 0, 0] and B == 3 and tau == 3.0
