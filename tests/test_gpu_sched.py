"""GPU parity of the DSpark confidence head (spec_confidence_head) and the
hardware-aware prefix scheduler (spec_prefix_schedule) against the oracle.

* Confidence head: every position, element by element, against the oracle's
  fp64 c = sigmoid(w . [h; W1[prev]]) on the same inputs.  Tolerance derived
  from the kernel's arithmetic: each lane sums about (d + r) / 64 fp32
  products in sequence, then a 6-level tree adds the lanes, so the logit
  error is at most (n / 64 + 8) 2^-24 sum |w_i x_i| (n = d + r); sigmoid's
  slope is at most 1/4, and the fp32 sigmoid adds a few ulps of c.
* Scheduler: lengths, batch size and tau bit-exact (both sides fix a in
  fp32 products and tau in exact integer sums), on random, tied and
  degenerate confidences and on several SPS tables, up to the 8192-candidate
  limit.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _conf_oracle(orc, wl, rows=None):
    R, G, d, r, V = wl["R"], wl["gamma"], wl["d"], wl["r"], wl["V"]
    H = workloads.as_f64(wl["h"], wl["h_dtype"])
    W1 = workloads.as_f64(wl["W1"], wl["w_dtype"])
    w = wl["w"].astype(np.float64)
    out = {}
    for b, k in (rows if rows is not None else [(b, k) for b in range(R) for k in range(G)]):
        prev = int(wl["x0"][b]) if k == 0 else int(wl["draft"][b, k - 1])
        if prev < 0 or prev >= V:
            out[(b, k)] = (0.0, 0.0)
            continue
        c = orc.confidence(H[b, k], W1[prev], w)
        S = float(np.abs(w[:d] * H[b, k]).sum() + np.abs(w[d:] * W1[prev]).sum())
        out[(b, k)] = (c, S)
    return out


def _conf_run(sd, wl):
    return sd.spec_confidence_head(dev(wl["h"], wl["h_dtype"]), dev(wl["x0"]), dev(wl["draft"]),
                                   dev(wl["W1"], wl["w_dtype"]), dev(wl["w"]))


def _conf_check(got, want, n):
    for (b, k), (c, S) in want.items():
        tol = 0.25 * (n / 64 + 8) * 2.0**-24 * S + 8 * 2.0**-24 * c + 1e-12
        assert abs(float(got[b, k]) - c) <= tol, (b, k, float(got[b, k]), c, tol)


@pytest.mark.parametrize("R,gamma,d,r,V,hdt,wdt", [
    (3, 4, 64, 16, 100, "f32", "f32"),
    (5, 3, 4096, 256, 1000, "bf16", "bf16"),   # 16-byte loads
    (4, 5, 100, 12, 50, "bf16", "f32"),        # d % 8 != 0: element loads
    (2, 2, 8, 8, 10, "f32", "bf16"),
    (7, 1, 520, 24, 300, "bf16", "bf16"),
])
def test_confidence_parity(orc, R, gamma, d, r, V, hdt, wdt):
    sd = require_gpu()
    note(f"confidence head R={R} gamma={gamma} d={d} r={r} V={V} h={hdt} W1={wdt}")
    wl = workloads.make_confidence(R, gamma, V, r, d, 60 + d, h_dtype=hdt, w_dtype=wdt)
    got = host({"c": _conf_run(sd, wl)})["c"]
    _conf_check(got, _conf_oracle(orc, wl), d + r)


def test_confidence_undrawn_previous_token(orc):
    sd = require_gpu()
    note("confidence head with undrawn / out-of-range previous tokens")
    wl = workloads.make_confidence(4, 4, 200, 16, 64, 77)
    wl["x0"][1] = -1
    wl["x0"][2] = 200
    wl["draft"][0, 1] = -1      # position 2 of request 0 follows an undrawn token
    wl["draft"][3, 3] = -1      # last draft token is never read
    got = host({"c": _conf_run(sd, wl)})["c"]
    want = _conf_oracle(orc, wl)
    assert got[1, 0] == 0.0 and got[2, 0] == 0.0 and got[0, 2] == 0.0
    _conf_check(got, want, 64 + 16)


def test_confidence_full_size(orc):
    """R = 128 requests, gamma = 16, hidden size 4096, r = 256, V = 151936:
    every position."""
    sd = require_gpu()
    note("confidence head full size R=128 gamma=16 d=4096")
    wl = workloads.make_confidence(128, 16, 151936, 256, 4096, 91)
    got = host({"c": _conf_run(sd, wl)})["c"]
    _conf_check(got, _conf_oracle(orc, wl), 4096 + 256)
    assert got.std() > 0.15 and 0.3 < got.mean() < 0.7   # the weights spread c over (0, 1)


# --------------------------------------------------------------------------

def _sched_check(orc, sd, c, sps, what):
    note(f"prefix schedule {what} R={c.shape[0]} gamma={c.shape[1]} nsps={sps.size}")
    want_l, want_B, want_tau = orc.prefix_schedule(c, sps)
    out = sd.spec_prefix_schedule(dev(np.ascontiguousarray(c, dtype=np.float32)),
                                  dev(np.ascontiguousarray(sps, dtype=np.float64)))
    got = host(out)
    np.testing.assert_array_equal(got["lens"], want_l)
    assert int(got["B"][0]) == want_B
    assert float(got["tau"][0]) == want_tau
    return want_l, want_B


def _tables(R, gamma, seed):
    n = R * (gamma + 1) + 1
    B = np.arange(n, dtype=np.float64)
    knee = 3 * R
    yield "knee", 1.0 / (1.0 + np.maximum(0.0, B - knee) / knee)
    yield "log-concave", 1000.0 * np.exp(-0.5 * (B / (2.0 * R)) ** 2)
    yield "constant", np.full(n, 7.0)
    rng = np.random.default_rng(seed)
    yield "noisy", np.sort(rng.uniform(0.5, 1.0, n))[::-1] * (1 + 0.02 * rng.standard_normal(n))
    yield "short", np.array([3.0] * min(n, R))    # zero at every B >= R


@pytest.mark.parametrize("R,gamma", [(1, 1), (3, 4), (7, 13), (100, 3), (128, 16), (1024, 8),
                                     (8192, 1), (512, 16)])
def test_schedule_parity(orc, R, gamma):
    sd = require_gpu()
    wl = workloads.make_schedule(R, gamma, 500 + R + gamma)
    for name, sps in _tables(R, gamma, R):
        _sched_check(orc, sd, wl["c"], sps, name)
    _sched_check(orc, sd, wl["c"], wl["sps"], "workload")


def test_schedule_ties(orc):
    """Many equal survival products across and along requests: the order of
    equal keys (lower request, then lower position) decides who is admitted."""
    sd = require_gpu()
    rng = np.random.default_rng(11)
    for R, gamma in ((9, 5), (200, 16), (1000, 8)):
        c = rng.choice(np.array([1.0, 0.5, 0.25, 0.75], dtype=np.float32), size=(R, gamma))
        for name, sps in _tables(R, gamma, 3):
            _sched_check(orc, sd, c, sps, "ties/" + name)
        c[:, :] = 1.0
        _sched_check(orc, sd, c, next(_tables(R, gamma, 3))[1], "all-ones")


def test_schedule_degenerate(orc):
    sd = require_gpu()
    c = np.zeros((6, 4), dtype=np.float32)
    c[1] = -0.0
    c[2, 0] = 1.0
    sps = np.linspace(10.0, 1.0, 6 * 5 + 1)
    _sched_check(orc, sd, c, sps, "zeros")
    _sched_check(orc, sd, c, np.full(31, 2.0), "zeros/constant")
    # no drafted positions: every length 0, B = R, tau = R
    l, B = _sched_check(orc, sd, np.zeros((5, 0), dtype=np.float32), np.full(6, 1.0), "gamma=0")
    assert B == 5 and not l.any()
    # empty SPS table: Theta is 0 everywhere, so nothing ever falls
    l, B = _sched_check(orc, sd, np.full((3, 2), 0.5, dtype=np.float32), np.zeros(0), "nsps=0")
    assert B == 9


def test_schedule_no_requests():
    sd = require_gpu()
    note("prefix schedule R=0")
    out = sd.spec_prefix_schedule(torch.zeros((0, 4), dtype=torch.float32, device="cuda"),
                                  torch.ones(4, dtype=torch.float64, device="cuda"))
    got = host(out)
    assert got["lens"].size == 0 and int(got["B"][0]) == 0 and float(got["tau"][0]) == 0.0


def test_schedule_admits_prefixes():
    """Survival products are non-increasing along a request, so every
    request's admitted set is a prefix and lengths stay within [0, gamma]."""
    sd = require_gpu()
    wl = workloads.make_schedule(128, 16, 9)
    got = host(sd.spec_prefix_schedule(dev(wl["c"]), dev(wl["sps"])))
    assert got["lens"].min() >= 0 and got["lens"].max() <= 16
    assert int(got["B"][0]) == 128 + int(got["lens"].sum())
