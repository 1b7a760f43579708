"""GPU parity of typical acceptance on candidate trees against the oracle (the
rule is a reading, not on the pages; see include/specverify.h). Bar: accept_len,
path_nodes and out_tokens bit-exact, except trees with a decisive pass test within
1e-6 (relative) of its threshold or a final draw within 1e-6 of a bin edge,
counted."""
import dataclasses

import numpy as np
import pytest

import gen
import oracle
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _check(w, eps, delta, trees=None):
    G.say(f"typical {w.name} B={w.B} N={w.n_nodes} V={w.V} dtype={w.dtype} eps={eps} delta={delta}")
    g = G.run_tree(dataclasses.replace(w, mode="typical"), None, epsilon=eps, delta=delta)
    sl = slice(None) if trees is None else trees
    par = w.parent if np.asarray(w.parent).ndim == 1 else w.parent[sl]
    o = oracle.verify_tree_typical(w.temperature, eps, delta, par, w.cand[sl], w.logits[sl],
                                   w.uniforms[sl], w.V, w.dtype, w.max_depth, G.TIE_EPS)
    G.compare_tree(g, o, trees)
    return g, o


def test_uniform_rows_boundary():
    parent, _ = gen.cartesian_tree([3, 3])
    n, V, B = len(parent), 3000, 2
    logits = gen.round_to(gen.DT_BF16, np.zeros((B, n, V)))
    cand = np.tile(np.arange(n, dtype=np.int32), (B, 1))
    u = gen.uniforms(gen.key(63, 1, 1), B * n).reshape(B, n)
    w = gen.TreeWorkload("uniform", "stochastic", 1.0, B, n, V, gen.DT_BF16, parent, cand, logits, u, 2)
    g, _ = _check(w, 1.0, 0.999)
    assert list(g["accept_len"]) == [2, 2]
    g, _ = _check(w, 1.0, 1.001)
    assert list(g["accept_len"]) == [0, 0]


@pytest.mark.parametrize("dtype", [gen.DT_F32, gen.DT_BF16, gen.DT_F16])
@pytest.mark.parametrize("eps,delta", [(0.3, 0.09), (0.05, 2.0), (1.0, 0.0)])
def test_small_trees(dtype, eps, delta):
    parent, _ = gen.cartesian_tree([4, 3, 2])
    n, B, V = len(parent), 6, 20001
    x = gen.normal_pair(gen.key(64, V, dtype), 1.5, 0, 0.0, B * n * V, dtype, want_b=False)[0].reshape(B, n, V)
    am = gen.argmax_rows(dtype, x, V).reshape(B, n)
    rng = np.random.default_rng(dtype * 7 + 1)
    cand = np.where(rng.random((B, n)) < 0.7, am[:, parent], rng.integers(0, V, (B, n))).astype(np.int32)
    cand[:, 0] = -1
    u = gen.uniforms(gen.key(64, V, 5), B * n).reshape(B, n)
    w = gen.TreeWorkload("small", "stochastic", 0.8, B, n, V, dtype, parent, cand, x, u, 3)
    g, o = _check(w, eps, delta)
    if delta == 0.0:
        assert np.all(g["accept_len"] == 3)


def test_c4_sparse_trees():
    w = gen.c4_medusa_sparse(2, mode="stochastic")
    g, o = _check(w, 0.09, 0.3)
    assert np.all(g["err_flags"] == 0)


def test_c5_full_tree():
    w = gen.c5_medusa_full(0, mode="stochastic")
    g, o = _check(w, 0.09, 0.3)             # every tree of the batch against the oracle


def test_errors():
    parent = np.array([-1, 0, 1], np.int32)
    B, V = 3, 500
    logits = np.random.default_rng(2).normal(size=(B, 3, V)).astype(np.float32)
    logits[1, 1, 7] = np.nan
    cand = np.array([[-1, 1, 2], [-1, 1, 2], [-1, V + 3, 2]], np.int32)
    u = np.full((B, 3), 0.5, np.float32)
    w = gen.TreeWorkload("errs", "stochastic", 1.0, B, 3, V, gen.DT_F32, parent, cand, logits, u, 2)
    g, o = _check(w, 0.5, 0.5)
    assert list(g["err_flags"]) == [0, 2, 1]
