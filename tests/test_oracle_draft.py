"""Pins of the oracle's sequential stage (DSpark review, §1.2: block
factorisation, Markov-head and RNN-head equations).

Markov: the bias equals the numpy product W1[x_{k-1}] @ W2; with W2 = 0 the
draws reduce to independent inverse-CDF draws from softmax(U_k) computed
with numpy; T = 0 reduces to numpy argmax.  RNN: limits of the gate that
reduce the update to closed forms (sigmoid -> 1 keeps s = 0; sigmoid -> 0
gives s_k = tanh(W_c z_k)), W_o = 0 gives no bias, and a block-structured
case whose bias is a hand-derived composition.
"""
import numpy as np
import pytest
from scipy import special

import workloads


def _numpy_draw(l, u):
    w = np.exp(l - l.max())
    return int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))


@pytest.fixture(scope="module")
def tiny():
    wl = workloads.make_markov(workloads.CONFIGS["markov-tiny"])
    return wl


def _inputs(wl, b=0):
    U = workloads.as_f64(wl["U"][b], wl["logit_dtype"])
    W1 = workloads.as_f64(wl["W1"], wl["w_dtype"])
    W2 = workloads.as_f64(wl["W2"], wl["w_dtype"])
    return U, W1, W2


def test_markov_bias_is_embedding_times_projection(orc):
    # amplified weights so that a wrong row, token or transpose is visible
    rng = np.random.default_rng(5)
    gamma, V, r = 6, 300, 8
    U = rng.standard_normal((gamma, V)) * 3
    W1 = rng.standard_normal((V, r)) * 0.5
    W2 = rng.standard_normal((r, V)) * 0.5
    u = rng.random(gamma)
    o = orc.draft_markov(U, W1, W2, x0=17, T=1.0, u=u)
    prev = [17] + o["tokens"][:-1].tolist()
    for k in range(gamma):
        bias = W1[prev[k]] @ W2
        assert np.allclose(o["q_logits"][k] - U[k], bias, rtol=0, atol=1e-12)
        assert abs(o["logZ"][k] - special.logsumexp(U[k] + bias)) < 1e-12
        assert o["tokens"][k] == _numpy_draw(U[k] + bias, u[k])
        assert abs(o["q_tok"][k] - special.softmax(U[k] + bias)[o["tokens"][k]]) < 1e-14


def test_markov_w2_zero_gives_independent_draws(orc, tiny):
    U, W1, W2 = _inputs(tiny)
    u = orc.draft_uniforms(0, 0, 1, tiny["gamma"])[0]
    o = orc.draft_markov(U, W1, np.zeros_like(W2), tiny["x0"][0], 1.0, u)
    for k in range(tiny["gamma"]):
        assert o["tokens"][k] == _numpy_draw(U[k], u[k])
        assert np.array_equal(o["q_logits"][k], U[k])


def test_markov_greedy_is_argmax(orc):
    rng = np.random.default_rng(6)
    U = rng.standard_normal((5, 400))
    W1 = rng.standard_normal((400, 4))
    W2 = rng.standard_normal((4, 400))
    o = orc.draft_markov(U, W1, W2, x0=3, T=0.0, u=None)
    prev = [3] + o["tokens"][:-1].tolist()
    for k in range(5):
        assert o["tokens"][k] == int(np.argmax(U[k] + W1[prev[k]] @ W2))


def test_markov_temperature(orc):
    rng = np.random.default_rng(8)
    U = rng.standard_normal((3, 200)) * 2
    W1 = rng.standard_normal((200, 4)) * 0.3
    W2 = rng.standard_normal((4, 200)) * 0.3
    u = rng.random(3)
    for T in (0.5, 2.0):
        o = orc.draft_markov(U, W1, W2, x0=0, T=T, u=u)
        prev = [0] + o["tokens"][:-1].tolist()
        for k in range(3):
            l = U[k] + W1[prev[k]] @ W2
            assert np.allclose(o["q_logits"][k], l, atol=1e-12)   # stored before temperature
            assert abs(o["logZ"][k] - special.logsumexp(l / T)) < 1e-12
            assert o["tokens"][k] == _numpy_draw(l / T, u[k])


def test_markov_depends_only_on_previous_token(orc):
    rng = np.random.default_rng(9)
    U = rng.standard_normal((4, 100))
    W1 = rng.standard_normal((100, 4))
    W2 = rng.standard_normal((4, 100))
    u = rng.random(4)
    a = orc.draft_markov(U, W1, W2, 5, 1.0, u, forced=[10, 20, 30, 40])
    b = orc.draft_markov(U, W1, W2, 5, 1.0, u, forced=[11, 20, 30, 40])
    assert not np.allclose(a["q_logits"][1], b["q_logits"][1])
    assert np.array_equal(a["q_logits"][2], b["q_logits"][2])
    assert np.array_equal(a["q_logits"][3], b["q_logits"][3])
    assert np.allclose(a["q_logits"][2] - U[2], W1[20] @ W2)


def _rnn_case(rng, gamma=4, V=120, r=3, d=5):
    U = rng.standard_normal((gamma, V)) * 2
    h = rng.standard_normal((gamma, d))
    W1 = rng.standard_normal((V, r))
    W2 = rng.standard_normal((r, V))
    return U, h, W1, W2


def test_rnn_output_zero_gives_no_bias(orc):
    rng = np.random.default_rng(10)
    U, h, W1, W2 = _rnn_case(rng)
    r, d = 3, 5
    Wg = rng.standard_normal((r, 2 * r + d))
    Wc = rng.standard_normal((r, 2 * r + d))
    Wo = np.zeros((r, 2 * r + d))
    u = rng.random(4)
    o = orc.draft_rnn(U, h, W1, W2, Wg, Wc, Wo, 7, 1.0, u)
    assert np.array_equal(o["q_logits"], U)
    for k in range(4):
        assert o["tokens"][k] == _numpy_draw(U[k], u[k])


def test_rnn_gate_open_keeps_state_zero(orc):
    # W_g drives sigmoid to exactly 1 in fp64, so s_k = s_{k-1} = 0 for all k;
    # W_o reads only the state block, so the bias stays 0 at every position.
    rng = np.random.default_rng(11)
    U, h, W1, W2 = _rnn_case(rng)
    r, d = 3, 5
    h = np.abs(h) + 1.0
    Wg = np.zeros((r, 2 * r + d))
    Wg[:, 2 * r:] = 1e4
    Wc = rng.standard_normal((r, 2 * r + d)) * 2
    Wo = np.zeros((r, 2 * r + d))
    Wo[:, :r] = rng.standard_normal((r, r)) * 3
    o = orc.draft_rnn(U, h, W1, W2, Wg, Wc, Wo, 7, 1.0, rng.random(4))
    assert np.array_equal(o["q_logits"], U)


def test_rnn_gate_closed_gives_candidate_state(orc):
    # sigmoid -> 0: s_k = tanh(W_c z_k).  With W_c reading only the hidden
    # block (C) and W_o reading only the state block (A):
    #   position 1: z_1 holds s_0 = 0, so the bias is 0;
    #   position 2: bias = W2^T tanh(A tanh(C h_1)).
    rng = np.random.default_rng(12)
    U, h, W1, W2 = _rnn_case(rng)
    r, d = 3, 5
    h = np.abs(h) + 1.0
    Wg = np.zeros((r, 2 * r + d))
    Wg[:, 2 * r:] = -1e4
    C = rng.standard_normal((r, d))
    A = rng.standard_normal((r, r)) * 2
    Wc = np.zeros((r, 2 * r + d))
    Wc[:, 2 * r:] = C
    Wo = np.zeros((r, 2 * r + d))
    Wo[:, :r] = A
    o = orc.draft_rnn(U, h, W1, W2, Wg, Wc, Wo, 7, 1.0, rng.random(4))
    assert np.array_equal(o["q_logits"][0], U[0])
    s1 = np.tanh(C @ h[0])
    want = np.tanh(A @ s1) @ W2
    assert np.allclose(o["q_logits"][1] - U[1], want, atol=1e-12)
    s2 = np.tanh(C @ h[1])
    assert np.allclose(o["q_logits"][2] - U[2], np.tanh(A @ s2) @ W2, atol=1e-12)


def test_rnn_embedding_block_reads_previous_token(orc):
    # gate open (s = 0); W_o reads only the embedding block (E), so the bias
    # of position k is W2^T tanh(E W1[x_{k-1}]), a Markov-like dependence.
    rng = np.random.default_rng(13)
    U, h, W1, W2 = _rnn_case(rng)
    r, d = 3, 5
    h = np.abs(h) + 1.0
    Wg = np.zeros((r, 2 * r + d))
    Wg[:, 2 * r:] = 1e4
    Wc = rng.standard_normal((r, 2 * r + d))
    E = rng.standard_normal((r, r))
    Wo = np.zeros((r, 2 * r + d))
    Wo[:, r:2 * r] = E
    o = orc.draft_rnn(U, h, W1, W2, Wg, Wc, Wo, 7, 1.0, rng.random(4))
    prev = [7] + o["tokens"][:-1].tolist()
    for k in range(4):
        assert np.allclose(o["q_logits"][k] - U[k], np.tanh(E @ W1[prev[k]]) @ W2, atol=1e-12)


def test_rnn_hidden_block_feeds_every_position(orc):
    # gate open, W_o reads only the hidden block (Hh): bias_k = W2^T tanh(Hh h_k)
    rng = np.random.default_rng(14)
    U, h, W1, W2 = _rnn_case(rng)
    r, d = 3, 5
    Wg = np.zeros((r, 2 * r + d))
    Wg[:, r:2 * r] = 0.0
    Wg[:, 2 * r:] = 0.0
    Hh = rng.standard_normal((r, d))
    Wo = np.zeros((r, 2 * r + d))
    Wo[:, 2 * r:] = Hh
    Wc = np.zeros((r, 2 * r + d))   # c = 0, g = 1/2: s_k = s_{k-1}/2 = 0
    o = orc.draft_rnn(U, h, W1, W2, Wg, Wc, Wo, 7, 1.0, rng.random(4))
    for k in range(4):
        assert np.allclose(o["q_logits"][k] - U[k], np.tanh(Hh @ h[k]) @ W2, atol=1e-12)
