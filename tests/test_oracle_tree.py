"""Pins of the oracle's tree-draft node selection (VESSL "Speculative
Decoding Part 1", section "γ 재배분: 체인 대신 트리": score every node by its
survival probability a_v, take the global top n with ties to the shallower
node; the choice is closed under prefixes and optimal for a fixed budget).

* Brute force over every prefix-closed node set of size n on tiny random
  trees: the chosen set is prefix-closed and reaches the largest summed
  survival.
* Chain (every node the child of the one before): the first n nodes.
* Star (every node a child of the root): numpy's stable top-n of c.
* All c = 1: breadth-first order (depth, then id).
* A forest of chains is a batch of requests: the chosen nodes are the first
  n candidates of the prefix scheduler's order on the same confidences.
"""
import itertools

import numpy as np
import pytest


def _random_tree(rng, M):
    parent = np.array([-1] + [int(rng.integers(-1, v)) for v in range(1, M)], dtype=np.int32)
    c = rng.uniform(0.05, 1.0, M).astype(np.float32)
    return parent, c


def _survival(parent, c):
    a = np.zeros(len(c))
    for v in range(len(c)):
        a[v] = (1.0 if parent[v] < 0 else a[parent[v]]) * np.float64(c[v])
    return a


def _closed(parent, S):
    return all(parent[v] < 0 or parent[v] in S for v in S)


@pytest.mark.parametrize("seed", range(8))
def test_tree_select_brute_force(orc, seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(3, 9))
    parent, c = _random_tree(rng, M)
    if seed == 7:
        c[:] = np.float32(0.5)   # many ties
    a = _survival(parent, c)
    for n in range(0, M + 1):
        sel, score = orc.tree_select(parent, c, n)
        S = set(int(v) for v in sel)
        assert len(S) == n and _closed(parent, S)
        best = max(sum(a[list(T)]) for T in itertools.combinations(range(M), n)
                   if _closed(parent, set(T)))
        assert sum(a[list(S)]) >= best * (1 - 1e-6) - 1e-12
        assert score == pytest.approx(sum(a[list(S)]), rel=1e-6, abs=1e-12)


def test_tree_select_chain(orc):
    M = 12
    parent = np.arange(-1, M - 1, dtype=np.int32)
    c = np.random.default_rng(1).uniform(0.2, 1.0, M).astype(np.float32)
    for n in (0, 1, 5, 12, 15):
        sel, _ = orc.tree_select(parent, c, n)
        assert list(sel[:min(n, M)]) == list(range(min(n, M)))
        assert (sel[M:] == -1).all()


def test_tree_select_star(orc):
    rng = np.random.default_rng(2)
    M = 40
    c = rng.choice(np.array([0.9, 0.5, 0.7, 0.2], dtype=np.float32), M)
    sel, score = orc.tree_select(np.full(M, -1, dtype=np.int32), c, 17)
    want = np.argsort(-c.astype(np.float64), kind="stable")[:17]
    assert list(sel) == list(want)
    assert score == pytest.approx(float(np.sort(c.astype(np.float64))[::-1][:17].sum()), rel=1e-9)


def test_tree_select_all_ones_is_breadth_first(orc):
    rng = np.random.default_rng(3)
    M = 30
    parent, _ = _random_tree(rng, M)
    depth = np.zeros(M, dtype=int)
    for v in range(M):
        depth[v] = 1 if parent[v] < 0 else depth[parent[v]] + 1
    sel, score = orc.tree_select(parent, np.ones(M, dtype=np.float32), M)
    assert list(sel) == sorted(range(M), key=lambda v: (depth[v], v))
    assert score == M


def test_tree_select_forest_of_chains_matches_scheduler(orc):
    """Requests with gamma drafted positions each are a forest of chains; with
    distinct survival values the top-n nodes are the scheduler's first n."""
    rng = np.random.default_rng(4)
    R, g = 6, 5
    c = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
    parent = np.array([-1 if j == 0 else r * g + j - 1 for r in range(R) for j in range(g)],
                      dtype=np.int32)
    a = np.cumprod(c.astype(np.float32), axis=1, dtype=np.float32).ravel()
    assert len(set(a.tolist())) == a.size
    for n in range(R * g + 1):
        sel, _ = orc.tree_select(parent, c.ravel(), n)
        sps = np.concatenate([np.full(R + n + 1, 1.0), np.zeros(R * g)])   # flat, then zero
        lens, B, _ = orc.prefix_schedule(c, sps)
        assert B == R + n
        want = sorted(r * g + j for r in range(R) for j in range(lens[r]))
        assert sorted(sel.tolist()) == want


def test_tree_select_bad_parent(orc):
    sel, score = orc.tree_select(np.array([-1, 1, 0], dtype=np.int32),
                                 np.full(3, 0.5, dtype=np.float32), 2)
    assert (sel == -1).all() and np.isnan(score)
