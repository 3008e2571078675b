"""GPU parity: device Philox stream and lossless verification against the
oracle on identical inputs (dense, packed/ragged, greedy, caller uniforms)."""
import numpy as np
import pytest

import workloads
from oracle import compare
from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,offset", [(0, 0), (12345678901234, 7), (2**64 - 1, 2**32 - 1)])
def test_device_philox_equals_oracle(orc, seed, offset):
    sd = require_gpu()
    B, K = 37, 33
    for stream in (0, 1, 2):
        note(f"philox seed={seed} offset={offset} stream={stream}")
        g = sd.spec_philox_uniforms(seed, offset, stream, B, K).cpu().numpy()
        want = np.array([[orc.uniform(seed, offset, b, k, stream) for k in range(K)]
                         for b in range(B)])
        assert np.array_equal(g.astype(np.float64), want)


def _oracle_drafts(orc, Qf, T, rng, random_frac=0.2):
    """Draft tokens drawn by the oracle from the draft rows (plus some random
    tokens, which are mostly rejected)."""
    B, gamma, V = Qf.shape
    draft = np.zeros((B, gamma), dtype=np.int32)
    for b in range(B):
        for k in range(gamma):
            if rng.random() < random_frac:
                draft[b, k] = rng.integers(V)
            elif T == 0:
                draft[b, k] = orc.argmax(Qf[b, k])[0]
            else:
                w, Z, _ = orc.softmax_weights(Qf[b, k], T)
                draft[b, k] = orc.inverse_cdf(w, Z, rng.random())[0]
    return draft


def _gpu_rows(g, b):
    return {k: v[b] for k, v in g.items()}


@pytest.mark.parametrize("dtype,V,T,sigma", [
    ("f32", 5000, 1.0, 0.6), ("bf16", 5000, 1.0, 0.3), ("bf16", 4099, 0.7, 0.6),
    ("f32", 257, 1.3, 1.0), ("f32", 1000, 0.0, 0.6), ("bf16", 12345, 0.0, 0.3),
    ("bf16", 20000, 1.0, 1.5)])
def test_verify_dense_parity(orc, dtype, V, T, sigma):
    sd = require_gpu()
    B, gamma = 12, 5
    note(f"verify dense dtype={dtype} V={V} T={T}")
    vw = workloads.make_verify_only(B, gamma, V, seed=1000 + V, dtype=dtype, sigma=sigma)
    Pf, Qf = workloads.as_f64(vw["P"], dtype), workloads.as_f64(vw["Q"], dtype)
    draft = _oracle_drafts(orc, Qf, T, np.random.default_rng(V))
    seed = 11
    g = host(sd.spec_verify(dev(vw["P"], dtype), dev(vw["Q"], dtype), dev(draft), T, seed=seed))
    u = orc.verify_uniforms(seed, 0, B, gamma)
    tally = compare.Tally()
    for b in range(B):
        compare.compare_verify_request(Pf[b], Qf[b], draft[b], T, u[b, :gamma], u[b, gamma],
                                       _gpu_rows(g, b), f"b={b}", tally)
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert g["accepted"].max() > 0          # some acceptances happen


@pytest.mark.parametrize("pdt,qdt", [("bf16", "f32"), ("f32", "f32"), ("bf16", "bf16")])
def test_verify_ragged_packed_parity(orc, pdt, qdt):
    sd = require_gpu()
    B, G, V = 10, 6, 3000
    lens = np.array([0, 6, 1, 3, 6, 2, 0, 5, 4, 6], dtype=np.int32)
    note(f"verify ragged p={pdt} q={qdt}")
    vw = workloads.make_verify_only(B, G, V, seed=77, dtype=pdt, sigma=0.5, lens=lens)
    Pf = workloads.as_f64(vw["P"], pdt)                      # packed [sum(L+1), V]
    q32 = workloads.as_f64(vw["Q"], pdt).astype(np.float32)  # dense [B, G, V]
    qstore = workloads.f32_to_bf16_bits(q32) if qdt == "bf16" else q32
    Qf_dense = workloads.as_f64(qstore, qdt)
    # pack the draft rows of each request: rows q_off[b] .. q_off[b] + L - 1
    q_off = workloads.packed_offsets(lens)
    Qpacked = np.concatenate([qstore[b, :lens[b]] for b in range(B)], axis=0)
    p_off = workloads.packed_offsets(lens + 1)
    draft = _oracle_drafts(orc, Qf_dense, 1.0, np.random.default_rng(3), random_frac=0.1)
    seed = 4
    g = host(sd.spec_verify(dev(vw["P"], pdt), dev(Qpacked, qdt), dev(draft), 1.0, gamma_max=G,
                            lens=dev(lens), p_row_off=dev(p_off), q_row_off=dev(q_off), seed=seed))
    u = orc.verify_uniforms(seed, 0, B, G)
    tally = compare.Tally()
    for b in range(B):
        L = int(lens[b])
        Pb = Pf[p_off[b]:p_off[b] + L + 1]
        compare.compare_verify_request(Pb, Qf_dense[b, :L], draft[b, :L], 1.0, u[b, :L], u[b, G],
                                       _gpu_rows(g, b), f"b={b} L={L}", tally)
        assert 1 <= g["accepted"][b] + 1 <= L + 1
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")


def test_verify_caller_uniforms_and_identical_rows(orc):
    sd = require_gpu()
    B, G, V = 6, 4, 2048
    rng = np.random.default_rng(9)
    Q = (rng.standard_normal((B, G, V)) * 3).astype(np.float32)
    P = np.concatenate([Q, (rng.standard_normal((B, 1, V)) * 3).astype(np.float32)], axis=1)
    P[3:] = (rng.standard_normal((3, G + 1, V)) * 3).astype(np.float32)   # 3 requests differ
    draft = _oracle_drafts(orc, Q.astype(np.float64), 1.0, rng, random_frac=0.0)
    uni = rng.random((B, G + 1)).astype(np.float32)
    g = host(sd.spec_verify(dev(P), dev(Q), dev(draft), 1.0, uniforms=dev(uni)))
    tally = compare.Tally()
    for b in range(B):
        compare.compare_verify_request(P[b].astype(np.float64), Q[b].astype(np.float64), draft[b],
                                       1.0, uni[b, :G].astype(np.float64), float(uni[b, G]),
                                       _gpu_rows(g, b), f"b={b}", tally)
    assert np.all(g["accepted"][:3] == G)              # p == q accepts everything
    assert np.all(g["accept_prob"][:3] == 1.0)


def test_verify_invalid_requests_are_flagged(orc):
    sd = require_gpu()
    B, G, V = 4, 3, 600
    rng = np.random.default_rng(2)
    P = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    Q = rng.standard_normal((B, G, V)).astype(np.float32)
    draft = rng.integers(0, V, size=(B, G)).astype(np.int32)
    draft[1, 2] = V            # out of range token
    draft[2, 0] = -5
    P[3, 1, :] = -np.inf       # a target row without mass
    g = host(sd.spec_verify(dev(P), dev(Q), dev(draft), 1.0, seed=1))
    assert g["accepted"][1] == -1 and g["accepted"][2] == -1 and g["accepted"][3] == -1
    assert np.all(g["out_tokens"][1:] == -1)
    assert g["accepted"][0] >= 0 and g["out_tokens"][0][g["accepted"][0]] >= 0


@pytest.mark.parametrize("dtype,V,T", [
    ("f32", 24584, 1.0), ("bf16", 24584, 0.0), ("bf16", 16387, 1.0), ("f32", 16387, 0.0)])
def test_verify_segmented_rows(orc, dtype, V, T):
    """Rows split into several segments: a ragged split of the 16-byte
    vectors (V = 8 * 3073) or of single values (V odd), rows whose finite
    logits all sit in one segment, and more than 64 positions per request so
    the decision runs over several chunks; request 2 has an out-of-range
    draft token at position 66 (second chunk) and must come back invalid."""
    sd = require_gpu()
    B, G = 3, 70
    note(f"verify segmented dtype={dtype} V={V} T={T}")
    vw = workloads.make_verify_only(B, G, V, seed=31 + V, dtype=dtype, sigma=0.5)
    P, Q = vw["P"], vw["Q"]
    ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    P[1, 3, :V - 100] = ninf        # mass only in the last segment
    Q[0, 2, 50:] = ninf             # mass only in the first segment
    P[0, 40, V // 3:] = ninf        # mass only in the first segments
    Pf, Qf = workloads.as_f64(P, dtype), workloads.as_f64(Q, dtype)
    draft = _oracle_drafts(orc, Qf, T, np.random.default_rng(V), random_frac=0.05)
    draft[2, 66] = V
    seed = 19
    g = host(sd.spec_verify(dev(P, dtype), dev(Q, dtype), dev(draft), T, seed=seed))
    u = orc.verify_uniforms(seed, 0, B, G)
    tally = compare.Tally()
    for b in range(2):
        compare.compare_verify_request(Pf[b], Qf[b], draft[b], T, u[b, :G], u[b, G],
                                       _gpu_rows(g, b), f"b={b}", tally)
    note(f"  {tally.as_dict()} accepted={g['accepted'].tolist()}")
    assert g["accepted"][2] == -1 and np.all(g["out_tokens"][2] == -1)
    assert np.all(g["p_logZ"][2] == 0.0) and np.all(g["accept_prob"][2] == 0.0)


def test_verify_zero_sizes(orc):
    sd = require_gpu()
    V = 100
    P = torch.zeros((0, 3, V), device="cuda")
    Q = torch.zeros((0, 2, V), device="cuda")
    d = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    out = sd.spec_verify(P, Q, d, 1.0)
    assert out["accepted"].numel() == 0
    # gamma_max = 0: only the bonus draw from the single target row
    rng = np.random.default_rng(5)
    P1 = rng.standard_normal((3, 1, V)).astype(np.float32)
    g = host(sd.spec_verify(dev(P1), None, torch.zeros((3, 0), dtype=torch.int32, device="cuda"),
                            1.0, seed=3))
    u = orc.verify_uniforms(3, 0, 3, 0)
    for b in range(3):
        w, Z, _ = orc.softmax_weights(P1[b, 0].astype(np.float64), 1.0)
        want = orc.inverse_cdf(w, Z, u[b, 0])[0]
        assert g["accepted"][b] == 0 and g["out_tokens"][b, 0] == want


def test_verify_deterministic(orc):
    sd = require_gpu()
    B, G, V = 16, 7, 32000
    vw = workloads.make_verify_only(B, G, V, seed=5, dtype="f32", sigma=0.8)
    Pd, Qd = dev(vw["P"]), dev(vw["Q"])
    draft = dev(_oracle_drafts(orc, workloads.as_f64(vw["Q"], "f32"), 1.0,
                               np.random.default_rng(1)))
    a = host(sd.spec_verify(Pd, Qd, draft, 1.0, seed=8))
    b = host(sd.spec_verify(Pd, Qd, draft, 1.0, seed=8))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
