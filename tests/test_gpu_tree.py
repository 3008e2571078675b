"""GPU parity of the tree-draft node selection (spec_tree_select) against the
oracle: selected ids and scores bit-exact (both sides form survival as fp32
products down the tree and sum it exactly in 2^-48 units), on random trees of
several shapes and sizes up to 4096 nodes, chains, stars, ties, budgets above
the tree size, empty trees and a tree with an invalid parent id next to valid
ones."""
import numpy as np
import pytest

from tests.gpu_util import dev, host, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _random_trees(rng, R, M, branch=None):
    """Parents first; branch bounds how far back a parent may be (None: any)."""
    par = np.empty((R, M), dtype=np.int32)
    for t in range(R):
        for v in range(M):
            lo = -1 if branch is None else max(-1, v - branch)
            par[t, v] = rng.integers(lo, v) if v > 0 else -1
    return par


def _check(orc, sd, par, c, n, what):
    note(f"tree select {what} R={par.shape[0]} M={par.shape[1]} n={n}")
    got = host(sd.spec_tree_select(dev(par), dev(np.ascontiguousarray(c, dtype=np.float32)), n))
    for t in range(par.shape[0]):
        sel, score = orc.tree_select(par[t], c[t], n)
        np.testing.assert_array_equal(got["sel"][t], sel, err_msg=f"tree {t}")
        if np.isnan(score):
            assert np.isnan(got["score"][t])
        else:
            assert got["score"][t] == score, (t, got["score"][t], score)
    return got


@pytest.mark.parametrize("R,M,n,branch", [
    (4, 1, 1, None), (8, 7, 3, None), (16, 64, 16, 4), (8, 100, 40, None),
    (4, 1000, 60, 8), (2, 4096, 512, 16), (3, 4096, 4096, None), (5, 33, 50, 2),
])
def test_tree_select_parity(orc, R, M, n, branch):
    sd = require_gpu()
    rng = np.random.default_rng(M + n)
    par = _random_trees(rng, R, M, branch)
    c = rng.beta(4.0, 1.2, size=(R, M)).astype(np.float32)
    _check(orc, sd, par, c, n, "random")


def test_tree_select_shapes_and_ties(orc):
    sd = require_gpu()
    rng = np.random.default_rng(5)
    M = 256
    chain = np.tile(np.arange(-1, M - 1, dtype=np.int32), (2, 1))
    star = np.full((2, M), -1, dtype=np.int32)
    for par, name in ((chain, "chain"), (star, "star"), (_random_trees(rng, 2, M, 3), "tied")):
        c = rng.choice(np.array([1.0, 0.5, 0.75, 0.25], dtype=np.float32), size=par.shape)
        _check(orc, sd, par, c, 100, name)
        _check(orc, sd, par, np.ones(par.shape, dtype=np.float32), 100, name + "/ones")
        c0 = c.copy()
        c0[:, ::3] = 0.0
        _check(orc, sd, par, c0, M, name + "/zeros")


def test_tree_select_invalid_and_empty(orc):
    sd = require_gpu()
    rng = np.random.default_rng(6)
    par = _random_trees(rng, 3, 20)
    par[1, 7] = 9   # a parent after its child
    c = rng.uniform(0.1, 1.0, (3, 20)).astype(np.float32)
    got = _check(orc, sd, par, c, 5, "one invalid")
    assert (got["sel"][1] == -1).all() and np.isnan(got["score"][1])
    note("tree select M=0")
    out = host(sd.spec_tree_select(torch.zeros((2, 0), dtype=torch.int32, device="cuda"),
                                   torch.zeros((2, 0), dtype=torch.float32, device="cuda"), 3))
    assert (out["sel"] == -1).all() and (out["score"] == 0).all()
