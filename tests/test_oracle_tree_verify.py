"""Pins of the oracle's tree verification (orc_verify_tree).

"Speculative Decoding Part 1", section on redistributing the draft budget as a
tree instead of a chain: several continuations are verified in one target
pass; the acceptance rule (same page, section on the acceptance rule) keeps
the output lossless.  The oracle reads this as recursive rejection over the
siblings of a node; these tests pin it without re-deriving its arithmetic:

* exact output law: the draft tokens of every node's children are enumerated
  with their draft probabilities (i.i.d. from the parent's draft law), and the
  uniforms are integrated exactly by bisecting the oracle's own decisions
  (each ratio test is monotone in its uniform, the final draw in u_final).
  The law of the emitted sequence must be the target's: the first token
  follows p at the root, and given the emitted prefix and that the walk went
  on, the next token follows p of that context;
* a chain-shaped tree gives exactly the chain verification's outputs;
* T = 0 emits the target's greedy sequence, as far as the tree holds it;
* invalid trees and tokens are refused.
"""
import itertools

import numpy as np
import pytest


def _softmax(l, T):
    z = np.asarray(l, dtype=np.float64) / T
    z = z - z.max()
    w = np.exp(z)
    return w / w.sum()


class Contexts:
    """Target and draft logits per token context (tuple of tokens after the
    root), drawn on first use: a consistent model of a target and a draft."""

    def __init__(self, V, seed, sigma=1.5):
        self.V = V
        self.rng = np.random.default_rng(seed)
        self.sigma = sigma
        self.p, self.q = {}, {}

    def rows(self, ctx):
        if ctx not in self.p:
            self.p[ctx] = 1.5 * self.rng.standard_normal(self.V)
            self.q[ctx] = self.p[ctx] + self.sigma * self.rng.standard_normal(self.V)
        return self.p[ctx], self.q[ctx]


def _paths(parent, tok):
    """Token context (tuple) of every node: the tokens from the root's child
    down to the node itself."""
    ctx = []
    for v, pa in enumerate(parent):
        ctx.append((ctx[pa] if pa >= 0 else ()) + (int(tok[v]),))
    return ctx


def _rows(cx, parent, tok):
    ctx = _paths(parent, tok)
    P = [cx.rows(())[0]] + [cx.rows(c)[0] for c in ctx]
    Q = [cx.rows(())[1]] + [cx.rows(c)[1] for c in ctx]
    return np.array(P), np.array(Q)


def _final_law(call, lo=0.0, hi=1.0 - 2.0 ** -53):
    """Lengths of the u_final intervals of each final token (the inverse CDF
    is non-decreasing in u): recursive bisection of the step function."""
    law = {}

    def rec(a, ta, b, tb):
        if ta == tb:
            law[ta] = law.get(ta, 0.0) + (b - a)
            return
        if b - a < 1e-15:
            law[tb] = law.get(tb, 0.0) + (b - a)
            return
        m = 0.5 * (a + b)
        tm = call(m)
        rec(a, ta, m, tm)
        rec(m, tm, b, tb)

    rec(lo, call(lo), hi, call(hi))
    return law


def _exact_law(orc, cx, parent, T):
    """Law of the emitted sequence (accepted tokens, then the final token) of
    orc.verify_tree on tree `parent`, over the draft tokens and every uniform."""
    V, M = cx.V, len(parent)
    law = {}
    for tok in itertools.product(range(V), repeat=M):
        ctx = _paths(parent, tok)
        wtok = 1.0
        for v, pa in enumerate(parent):
            q = _softmax(cx.rows(ctx[pa] if pa >= 0 else ())[1], T)
            wtok *= q[tok[v]]
        if wtok == 0.0:
            continue
        P, Q = _rows(cx, parent, tok)

        def run(u, uf):
            r = orc.verify_tree(P, Q, parent, tok, T, u, uf)
            assert r is not None
            return r

        def explore(ufix, prob):
            u = np.array([ufix.get(v, 0.5) for v in range(M)])
            r = run(u, 0.5)
            tested = [v for v in range(M) if np.isfinite(r["test_ratio"][v])]
            open_ = [v for v in tested if v not in ufix]
            if not open_:
                n = r["n"]
                head = tuple(int(x) for x in r["out"][:n])
                fl = _final_law(lambda uf: int(run(u, uf)["out"][n]))
                for y, w in fl.items():
                    key = head + (y,)
                    law[key] = law.get(key, 0.0) + prob * w
                return
            c = open_[0]          # tests happen in increasing node index

            def passes(x):
                uu = u.copy()
                uu[c] = x
                return c in run(uu, 0.5)["path"][: M]

            lo, hi = 0.0, 1.0     # passes(lo) unless the threshold is 0
            if not passes(0.0):
                t = 0.0
            else:
                for _ in range(55):
                    mid = 0.5 * (lo + hi)
                    if passes(mid):
                        lo = mid
                    else:
                        hi = mid
                t = hi
            if t > 0.0:
                explore({**ufix, c: 0.5 * t}, prob * t)
            if t < 1.0:
                explore({**ufix, c: 0.5 * (1.0 + t)}, prob * (1.0 - t))

        explore({}, wtok)
    return law


def _check_target_law(cx, law, T, tol=1e-9):
    """Every emitted position follows p of its context, given the emitted
    prefix and that the walk reached it."""
    assert abs(sum(law.values()) - 1.0) < tol
    depth = max(len(k) for k in law)
    for j in range(depth):
        # mass of (prefix s of length j, next token y) among outputs longer than j
        cond = {}
        for key, w in law.items():
            if len(key) > j:
                cond.setdefault(key[:j], np.zeros(cx.V))[key[j]] += w
        for pre, mass in cond.items():
            tot = mass.sum()
            if tot < 1e-12:
                continue
            want = _softmax(cx.rows(pre)[0], T)
            assert np.allclose(mass / tot, want, atol=tol / max(tot, 1e-3)), (j, pre, mass / tot, want)


TREES = {
    "star2": [-1, -1],
    "star3": [-1, -1, -1],
    "fork": [-1, -1, 0, 0],
    "chain_and_sibling": [-1, 0, -1],
    "deep": [-1, 0, 1, -1],
}


@pytest.mark.parametrize("name", sorted(TREES))
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_tree_output_law_is_target(orc, name, T):
    cx = Contexts(V=3, seed=sum(map(ord, name)) + int(10 * T))
    law = _exact_law(orc, cx, TREES[name], T)
    _check_target_law(cx, law, T)


def test_tree_law_check_has_power(orc):
    """The law check notices 1% of the mass moved from one output to another."""
    cx = Contexts(V=3, seed=5)
    law = _exact_law(orc, cx, TREES["star2"], 1.0)
    # tamper: move 1% of the mass of one output to another
    keys = sorted(law)
    law[keys[0]] -= 0.01
    law[keys[-1]] += 0.01
    with pytest.raises(AssertionError):
        _check_target_law(cx, law, 1.0)


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_chain_tree_equals_chain_verify(orc, T):
    rng = np.random.default_rng(11 + int(10 * T))
    for trial in range(150):
        L = int(rng.integers(1, 6))
        V = int(rng.integers(2, 40))
        P = 2.0 * rng.standard_normal((L + 1, V))
        Q = P[:L] + rng.standard_normal((L, V))
        draft = rng.integers(0, V, size=L).astype(np.int32)
        if trial % 2 == 0 and T > 0:     # draws from q, mostly accepted
            for k in range(L):
                draft[k] = rng.choice(V, p=_softmax(Q[k], T))
        u = rng.random(L)
        uf = float(rng.random())
        want = orc.verify(P, Q, draft, T, u, uf)
        Qt = np.vstack([Q, np.zeros((1, V))])      # a leaf's draft row is never read
        got = orc.verify_tree(P, Qt, list(range(-1, L - 1)), draft, T, u, uf)
        if T > 0 and min(want["final_margin"], got["final_margin"]) < 1e-12:
            continue                                # a final draw on a CDF boundary
        assert got["n"] == want["n"], trial
        assert np.array_equal(got["out"], want["out"]), trial
        assert np.array_equal(got["path"][: got["n"]], np.arange(got["n"]))


def test_greedy_emits_target_greedy_sequence(orc):
    rng = np.random.default_rng(3)
    for trial in range(100):
        V = int(rng.integers(2, 6))
        M = int(rng.integers(1, 9))
        parent = [int(rng.integers(-1, v)) for v in range(M)]
        tok = rng.integers(0, V, size=M).astype(np.int32)
        cx = Contexts(V, seed=100 + trial)
        P, Q = _rows(cx, parent, tok)
        r = orc.verify_tree(P, Q, parent, tok, 0.0, np.full(M, 0.5), 0.5)
        n, out = r["n"], r["out"]
        # the emitted tokens are the target's greedy sequence
        pre = ()
        for j in range(n + 1):
            assert out[j] == int(np.argmax(cx.rows(pre)[0])), (trial, j)
            pre = pre + (int(out[j]),)
        # and the walk stopped where no child holds the greedy token
        last = r["path"][n - 1] if n > 0 else -1
        kids = [v for v in range(M) if parent[v] == last]
        assert all(tok[v] != out[n] for v in kids)


def test_invalid_tree_or_token_refused(orc):
    V = 4
    P = np.zeros((4, V))
    Q = np.zeros((4, V))
    u = np.full(3, 0.5)
    assert orc.verify_tree(P, Q, [-1, 1, 0], [0, 1, 2], 1.0, u, 0.5) is None     # parent >= v
    assert orc.verify_tree(P, Q, [-1, -2, 0], [0, 1, 2], 1.0, u, 0.5) is None    # parent < -1
    assert orc.verify_tree(P, Q, [-1, 0, 0], [0, 4, 2], 1.0, u, 0.5) is None     # token >= V
    assert orc.verify_tree(P, Q, [-1, 0, 0], [0, 1, -1], 0.0, u, 0.5) is None    # token < 0


def test_empty_tree_draws_bonus_from_root(orc):
    rng = np.random.default_rng(8)
    P = rng.standard_normal((1, 7))
    law = {}
    for uf in (np.arange(4096) + 0.5) / 4096:
        y = orc.verify_tree(P, np.zeros((1, 7)), [], [], 1.0, [], uf)["out"][0]
        law[y] = law.get(y, 0) + 1 / 4096
    want = _softmax(P[0], 1.0)
    got = np.array([law.get(v, 0.0) for v in range(7)])
    assert np.abs(got - want).max() < 2 / 4096


def test_siblings_tested_in_index_order(orc):
    """With the draft law equal to the target law every ratio is 1, so the
    first child tested passes: it is the lowest-index child of the root, then
    the lowest-index child of that node."""
    rng = np.random.default_rng(21)
    V = 6
    row = rng.standard_normal(V)
    parent = [-1, -1, 1, 1, 0, -1]
    tok = [3, 1, 4, 2, 0, 5]
    P = np.tile(row, (7, 1))
    for _ in range(20):
        u = rng.random(6)
        r = orc.verify_tree(P, P.copy(), parent, tok, 1.0, u, float(rng.random()))
        assert r["n"] == 2 and list(r["path"][:2]) == [0, 4]
        assert list(r["out"][:2]) == [3, 0]
