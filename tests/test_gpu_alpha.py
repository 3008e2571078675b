"""GPU parity of the per-position acceptance rate alpha = sum min(p, q) and
total variation 1/2 sum |p - q| (spec_acceptance_rate) against the oracle's
fp64 definition, on dense and packed rows, bf16 and fp32 logits, ragged
lengths and T = 0.  Tolerance: the benchmark spec's 1e-5 relative on
probabilities, with an absolute floor of 1e-6 (alpha and TV are sums of
normalised weights)."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _tol(x):
    return 1e-5 * abs(x) + 1e-6


def _want(orc, lp, lq, T):
    if T == 0.0:   # one-hot at the argmax (lowest id on ties)
        a = 1.0 if orc.argmax(lp)[0] == orc.argmax(lq)[0] else 0.0
        return a, 1.0 - a
    return orc.alpha_tv(lp, lq, T)


def _rows(B, gamma, V, seed, pdt, qdt):
    """Target rows P [B, gamma+1, V] and draft rows Q [B, gamma, V] of the
    seeded Zipf + Gaussian generator (Q: the draft base logits)."""
    cfg = dict(workloads.CONFIGS["markov-32k-b32"])
    cfg["logit_dtype"] = "bf16"
    cfg["data_seed"] = seed
    wl = workloads.make_markov(cfg, B=B, gamma=gamma, V=V, r=16)
    P = workloads.as_f64(wl["P"], "bf16")
    Q = workloads.as_f64(wl["U"], "bf16")

    def store(x, dt):
        x32 = x.astype(np.float32)
        return (x32, dev(x32)) if dt == "f32" else (x32, dev(workloads.f32_to_bf16_bits(x32), "bf16"))

    return store(P, pdt), store(Q, qdt)


@pytest.mark.parametrize("B,gamma,V,pdt,qdt,T", [
    (3, 4, 1000, "f32", "f32", 1.0),
    (5, 3, 4099, "bf16", "f32", 0.8),     # V % 8 != 0: element loads
    (4, 5, 3000, "bf16", "bf16", 1.3),
    (6, 4, 2000, "f32", "bf16", 0.0),     # greedy
    (2, 2, 8, "bf16", "f32", 1.0),        # one 8-token vector per row
])
def test_alpha_dense_parity(orc, B, gamma, V, pdt, qdt, T):
    sd = require_gpu()
    note(f"acceptance rate dense B={B} gamma={gamma} V={V} P={pdt} Q={qdt} T={T}")
    (Ph, Pd), (Qh, Qd) = _rows(B, gamma, V, 40 + V, pdt, qdt)
    g = host(sd.spec_acceptance_rate(Pd, Qd, T))
    for b in range(B):
        for k in range(gamma):
            a, t = _want(orc, Ph[b, k].astype(np.float64), Qh[b, k].astype(np.float64), T)
            assert abs(g["alpha"][b, k] - a) <= _tol(a), (b, k, g["alpha"][b, k], a)
            assert abs(g["tv"][b, k] - t) <= _tol(t), (b, k, g["tv"][b, k], t)
            assert abs(g["alpha"][b, k] + g["tv"][b, k] - 1.0) <= 2e-6


@pytest.mark.parametrize("B,gamma,V,T", [
    (4, 5, 3000, 1.3),
    (61, 13, 3000, 1.0),     # 793 positions
    (3, 2, 64, 0.7),
    (2, 3, 8, 1.0),          # one 8-token vector per row
    (5, 7, 184320, 1.0),
])
def test_alpha_bf16_pairs_parity(orc, B, gamma, V, T):
    """bf16 P and Q rows under sampling: every position against the oracle,
    and against the same values given as fp32 Q rows (a second kernel
    instantiation)."""
    sd = require_gpu()
    note(f"acceptance rate bf16 pairs B={B} gamma={gamma} V={V} T={T}")
    (Ph, Pd), (Qh, Qd) = _rows(B, gamma, V, 90 + V, "bf16", "bf16")
    g = host(sd.spec_acceptance_rate(Pd, Qd, T))
    g2 = host(sd.spec_acceptance_rate(Pd, Qd.float().contiguous(), T))
    for b in range(B):
        for k in range(gamma):
            a, t = _want(orc, Ph[b, k].astype(np.float64), Qh[b, k].astype(np.float64), T)
            assert abs(g["alpha"][b, k] - a) <= _tol(a), (b, k, g["alpha"][b, k], a)
            assert abs(g["tv"][b, k] - t) <= _tol(t), (b, k, g["tv"][b, k], t)
            assert abs(g["alpha"][b, k] - g2["alpha"][b, k]) <= 2 * _tol(a), (b, k)


def test_alpha_bf16_packed_ragged(orc):
    """Packed bf16 P and Q rows with per-request lengths (0, gamma_max and one
    out of range): positions with no rows are NaN (the last request has none,
    so its offsets point at the end of both tensors)."""
    sd = require_gpu()
    B, G, V, T = 9, 6, 6000, 1.0
    lens = np.array([3, 0, 6, 1, 9, 5, 2, 6, 0], dtype=np.int32)   # lens[4] > G: invalid
    (Ph, _), (Qh, _) = _rows(B, G, V, 78, "f32", "f32")
    prow, qrow, p_off, q_off = [], [], [], []
    for b in range(B):
        L = int(lens[b]) if lens[b] <= G else 0
        p_off.append(len(prow))
        q_off.append(len(qrow))
        prow += [Ph[b, k] for k in range(L + 1 if L else 0)]
        qrow += [Qh[b, k] for k in range(L)]
    Pb = workloads.f32_to_bf16_bits(np.stack(prow).astype(np.float32))
    Qb = workloads.f32_to_bf16_bits(np.stack(qrow).astype(np.float32))
    g = host(sd.spec_acceptance_rate(
        dev(Pb, "bf16"), dev(Qb, "bf16"), T, gamma_max=G, lens=dev(lens),
        p_row_off=dev(np.array(p_off, np.int64)), q_row_off=dev(np.array(q_off, np.int64))))
    P64, Q64 = workloads.as_f64(Pb, "bf16"), workloads.as_f64(Qb, "bf16")
    for b in range(B):
        for k in range(G):
            if lens[b] > G or k >= lens[b]:
                assert np.isnan(g["alpha"][b, k]) and np.isnan(g["tv"][b, k]), (b, k)
                continue
            a, t = _want(orc, P64[p_off[b] + k], Q64[q_off[b] + k], T)
            assert abs(g["alpha"][b, k] - a) <= _tol(a), (b, k)
            assert abs(g["tv"][b, k] - t) <= _tol(t), (b, k)


def test_alpha_packed_ragged(orc):
    """Packed rows with per-request lengths (0 and gamma_max included, one
    out of range): positions past L_b and the bad request are NaN."""
    sd = require_gpu()
    B, G, V, T = 7, 6, 5000, 1.0
    lens = np.array([3, 0, 6, 1, 7, 5, 2], dtype=np.int32)   # lens[4] > G: invalid
    (Ph, _), (Qh, _) = _rows(B, G, V, 77, "f32", "f32")
    prow, qrow, p_off, q_off = [], [], [], []
    for b in range(B):
        L = min(int(lens[b]), G)
        p_off.append(len(prow))
        q_off.append(len(qrow))
        prow += [Ph[b, k] for k in range(L + 1)]
        qrow += [Qh[b, k] for k in range(L)]
    Pp = np.stack(prow).astype(np.float32)
    Qp = np.stack(qrow).astype(np.float32)
    Pd = dev(workloads.f32_to_bf16_bits(Pp), "bf16")
    Qd = dev(Qp)
    g = host(sd.spec_acceptance_rate(
        Pd, Qd, T, gamma_max=G, lens=dev(lens), p_row_off=dev(np.array(p_off, np.int64)),
        q_row_off=dev(np.array(q_off, np.int64))))
    Pb = workloads.as_f64(workloads.f32_to_bf16_bits(Pp), "bf16")
    for b in range(B):
        for k in range(G):
            if lens[b] > G or k >= lens[b]:
                assert np.isnan(g["alpha"][b, k]) and np.isnan(g["tv"][b, k]), (b, k)
                continue
            a, t = _want(orc, Pb[p_off[b] + k], Qp[q_off[b] + k].astype(np.float64), T)
            assert abs(g["alpha"][b, k] - a) <= _tol(a), (b, k)
            assert abs(g["tv"][b, k] - t) <= _tol(t), (b, k)


def test_alpha_special_cases(orc):
    """p == q gives alpha 1; rows whose mass sits on disjoint tokens give 0."""
    sd = require_gpu()
    V = 512
    x = np.random.default_rng(3).standard_normal(V).astype(np.float32) * 3
    far = np.full(V, -1e4, dtype=np.float32)
    p_disj, q_disj = far.copy(), far.copy()
    p_disj[:8] = 0.0
    q_disj[-8:] = 0.0
    P = np.stack([np.stack([x, x]), np.stack([p_disj, p_disj])])       # [2, 2, V]
    Q = np.stack([x[None], q_disj[None]])                               # [2, 1, V]
    g = host(sd.spec_acceptance_rate(dev(P), dev(Q), 1.0))
    assert abs(g["alpha"][0, 0] - 1.0) <= 2e-6 and abs(g["tv"][0, 0]) <= 2e-6
    assert abs(g["alpha"][1, 0]) <= 1e-6 and abs(g["tv"][1, 0] - 1.0) <= 2e-6


def test_alpha_full_size_sampled(orc):
    """B = 128, gamma = 16, V = 151936: bf16 target rows against fp32 draft
    rows at the timed size; six positions are checked against the oracle."""
    sd = require_gpu()
    B, G, V = 128, 16, 151936
    note("acceptance rate full size")
    cfg = dict(workloads.CONFIGS["markov-152k-b128"])
    wl = workloads.make_markov(cfg, B=B, gamma=G, V=V, r=16)
    Pd = dev(wl["P"], "bf16")
    Qf = torch.from_numpy(wl["U"]).view(torch.bfloat16).to("cuda").float().contiguous()
    g = host(sd.spec_acceptance_rate(Pd, Qf, 1.0))
    assert np.all(np.isfinite(g["alpha"])) and np.all((g["alpha"] > 0) & (g["alpha"] <= 1 + 1e-6))
    for b, k in [(0, 0), (17, 5), (64, 15), (100, 9), (127, 0), (127, 15)]:
        a, t = _want(orc, workloads.as_f64(wl["P"][b, k], "bf16"),
                     workloads.as_f64(wl["U"][b, k], "bf16"), 1.0)
        assert abs(g["alpha"][b, k] - a) <= _tol(a), (b, k, g["alpha"][b, k], a)
        assert abs(g["tv"][b, k] - t) <= _tol(t), (b, k)
