"""The comparison's per-logit error bound for the Markov head
(oracle/compare.markov_logit_bound, gamma_{r+1} (|U| + |W1[x]| . |W2|))
holds for fp32 arithmetic on bf16 inputs whatever the summation order: an
fp32 emulation in numpy of the kernels' sums stays within it on random
inputs, with U added last (the per-position tiles) or used as the
accumulator's starting value (the persistent draft), the rank summed forward,
reversed or pairwise.  With U in the accumulator from the start, the worst
case is gamma_{r+1} |U| ~ 1.5e-5 |U| at r = 256, which is why a fixed band of
1e-6 * max(1, |l|) would not be a bound at this rank."""
import numpy as np

import workloads
from oracle import compare


def _bf16(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x.astype(np.float32)))


def _fp32_sum(terms, order, start=None):
    """Sum of the rows of terms (fp32, each row one term per token) in fp32."""
    acc = np.zeros(terms.shape[1], np.float32) if start is None else start.astype(np.float32)
    if order == "pairwise":
        t = terms.astype(np.float32)
        while t.shape[0] > 1:
            if t.shape[0] % 2:
                t = np.vstack([t, np.zeros((1, t.shape[1]), np.float32)])
            t = (t[0::2] + t[1::2]).astype(np.float32)
        return (acc + t[0]).astype(np.float32)
    idx = range(terms.shape[0]) if order == "forward" else reversed(range(terms.shape[0]))
    for j in idx:
        acc = (acc + terms[j]).astype(np.float32)
    return acc


def test_markov_logit_bound_covers_fp32_sums():
    rng = np.random.default_rng(3)
    for r, V, w_std in ((256, 3000, 0.02), (64, 2000, 0.3), (16, 500, 1.0)):
        W1 = _bf16(w_std * rng.standard_normal((50, r))).astype(np.float64)
        W2 = _bf16(w_std * rng.standard_normal((r, V))).astype(np.float64)
        U = (4.0 * rng.standard_normal(V)).astype(np.float32).astype(np.float64)
        x = 7
        exact = U + W1[x] @ W2
        bound = compare.markov_logit_bound(U, W1, W2, x)
        prods = (W1[x][:, None].astype(np.float32) * W2.astype(np.float32)).astype(np.float32)
        for order in ("forward", "reverse", "pairwise"):
            last = (U.astype(np.float32) + _fp32_sum(prods, order)).astype(np.float32)
            first = _fp32_sum(prods, order, start=U)
            for l32 in (last, first):
                assert np.all(np.abs(l32.astype(np.float64) - exact) <= bound), (r, order)
        assert np.all(bound > 0)
        # the bound is gamma_{r+1} times the sum of the magnitudes
        mag = np.abs(U) + np.abs(W1[x]) @ np.abs(W2)
        np.testing.assert_allclose(bound / mag, (r + 1) * 2.0 ** -24, rtol=1e-3)


def test_greedy_band_uses_bound():
    l = np.array([1.0, 1.0 - 2e-7, 0.5])
    err = np.full(3, 1.5e-7)
    assert compare._check_greedy(l, 0, 1, "tie", err)            # within 3e-7: a tie
    try:
        compare._check_greedy(l, 0, 2, "far", err)
    except AssertionError:
        pass
    else:
        raise AssertionError("a 0.5 gap must not pass as a tie")
