"""Pin of the E[tau] closed form against values printed on the VESSL AI page
("Speculative Decoding Part 1", speedup-equation section).  The same closed
form is the expectation the oracle's Monte-Carlo tau law is tested against
(test_oracle_verify.test_expected_tau_iid_acceptance)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "speedup_points.txt")


def _e_tau_sum(alpha, gamma):
    return sum(alpha ** k for k in range(gamma + 1))


def _e_tau_closed(alpha, gamma):
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


def _speedup(alpha, c, gamma):
    return _e_tau_closed(alpha, gamma) / (c * gamma + 1)


def _rows():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            f = line.split()
            yield float(f[0]), float(f[1]), f[2:]


def test_closed_form_equals_geometric_sum():
    for alpha in (0.1, 0.5, 0.8, 0.95):
        for gamma in range(0, 30):
            assert abs(_e_tau_sum(alpha, gamma) - _e_tau_closed(alpha, gamma)) < 1e-12


def test_printed_speedup_values():
    gammas = np.arange(1, 200)
    seen = 0
    for alpha, c, f in _rows():
        S = np.array([_speedup(alpha, c, g) for g in gammas])
        best = S.max()
        assert np.all(S <= min(1 / c, 1 / (1 - alpha)) + 1e-12)
        if f[0] == "plateau_within_3pct":
            lo, hi = int(f[1]), int(f[2])
            for g in range(lo, hi + 1):
                assert S[g - 1] >= 0.97 * best
            seen += 1
        elif f[0] == "max_speedup":
            assert round(best, 1) == float(f[1])
            if len(f) > 2:
                assert int(gammas[S.argmax()]) == int(f[3])
            seen += 1
        elif f[0] == "upper_bound_inv_c":
            assert 1 / c == float(f[1])
            seen += 1
    assert seen == 4
