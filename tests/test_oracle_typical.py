"""Pins of the typical-acceptance oracle. The rule is not defined on the pages (the
workload description names it; see oracle.h), so parity with the pages is
unpinned; these tests pin the oracle to the rule as stated, through closed forms:

* uniform rows: the entropy is ln V and p(cand) = 1/V, so the threshold
  min(eps, delta/V) sits exactly at p when delta = 1: delta just below 1 accepts
  the whole tree, just above rejects everything;
* two-token rows: the binary entropy in closed form puts the pass/fail boundary at a
  known delta;
* delta = 0 (or eps = 0): the threshold is 0, every candidate of positive
  probability passes, so the deepest node of the tree is reached;
* the final token: chi-square of its draws against softmax of the last node's row.
"""
import math

import numpy as np
import pytest
from scipy import stats

import gen
import oracle


def _run(logits, parent, cand, T=1.0, eps=1.0, delta=1.0, u=None, max_depth=4):
    logits = np.ascontiguousarray(logits.astype(np.float32))
    B, n, V = logits.shape
    if u is None:
        u = np.full((B, n), 0.5, np.float32)
    return oracle.verify_tree_typical(T, eps, delta, parent, cand, logits, u, V, gen.DT_F32, max_depth)


def test_uniform_rows_boundary_at_delta_one():
    parent, rank = gen.cartesian_tree([3, 3])
    n, V = len(parent), 50
    logits = np.zeros((2, n, V))
    cand = np.tile(np.arange(n, dtype=np.int32) % V, (2, 1))
    below = _run(logits, parent, cand, eps=1.0, delta=0.999)
    above = _run(logits, parent, cand, eps=1.0, delta=1.001)
    assert list(below["accept_len"]) == [2, 2]
    assert list(above["accept_len"]) == [0, 0]
    # eps caps the threshold: with eps below 1/V everything passes again
    capped = _run(logits, parent, cand, eps=0.9 / V, delta=5.0)
    assert list(capped["accept_len"]) == [2, 2]
    # deepest node, lowest index: the first grandchild
    np.testing.assert_array_equal(below["path_nodes"][0, :2], [1, 4])


@pytest.mark.parametrize("a,T", [(1.3, 1.0), (-0.7, 0.5), (2.5, 2.0)])
def test_two_token_rows_binary_entropy(a, T):
    parent = np.array([-1, 0], np.int32)
    logits = np.array([[[a, 0.0], [0.0, 0.0]]])
    cand = np.array([[-1, 0]], np.int32)            # the child's token is token 0 of the root
    p = 1.0 / (1.0 + math.exp(-a / T))
    H = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    d0 = p * math.exp(H)                             # delta at which delta*exp(-H) = p
    assert _run(logits, parent, cand, T=T, eps=1.0, delta=d0 * (1 - 1e-4))["accept_len"][0] == 1
    assert _run(logits, parent, cand, T=T, eps=1.0, delta=d0 * (1 + 1e-4))["accept_len"][0] == 0


def test_zero_threshold_reaches_the_deepest_node():
    rng = np.random.default_rng(4)
    parent = np.array([-1, 0, 0, 1, 1, 3, 2, 6, 7], np.int32)     # depths 0 1 1 2 2 3 2 3 4
    n, V = len(parent), 300
    logits = rng.normal(0, 3, size=(3, n, V))
    cand = rng.integers(0, V, size=(3, n)).astype(np.int32)
    for eps, delta in ((1.0, 0.0), (0.0, 1.0)):
        r = _run(logits, parent, cand, eps=eps, delta=delta, max_depth=4)
        assert list(r["accept_len"]) == [4, 4, 4]
        np.testing.assert_array_equal(r["path_nodes"][0], [2, 6, 7, 8])


def test_final_token_is_drawn_from_the_last_node():
    parent = np.array([-1, 0], np.int32)
    V = 5
    x = np.array([0.2, -1.0, 1.5, 0.3, 0.0])
    logits = np.zeros((1, 2, V))
    logits[0, 1] = x
    cand = np.array([[-1, 3]], np.int32)
    n = 20000
    u = gen.uniforms(gen.key(91, 1, 1), n).astype(np.float32)
    ys = np.empty(n, np.int64)
    for t in range(0, n, 2000):
        rows = np.repeat(logits, 2000, axis=0)
        uu = np.stack([np.full(2000, 0.5, np.float32), u[t:t + 2000]], axis=1)
        r = oracle.verify_tree_typical(1.0, 1.0, 0.0, parent, np.repeat(cand, 2000, axis=0),
                                       np.ascontiguousarray(rows.astype(np.float32)), uu, V, gen.DT_F32, 1)
        assert np.all(r["accept_len"] == 1)
        ys[t:t + 2000] = r["out_tokens"][:, 1]
    pr = np.exp(x) / np.exp(x).sum()
    assert stats.chisquare(np.bincount(ys, minlength=V), pr * n).pvalue > 1e-3


def test_errors():
    parent = np.array([-1, 0, 5], np.int32)
    logits = np.zeros((1, 3, 10))
    cand = np.array([[-1, 1, 2]], np.int32)
    assert _run(logits, parent, cand)["err_flags"][0] == 4
    logits2 = np.zeros((1, 2, 10))
    logits2[0, 1, 3] = np.nan
    r = _run(logits2, np.array([-1, 0], np.int32), np.array([[-1, 1]], np.int32))
    assert r["err_flags"][0] == 2 and r["accept_len"][0] == -1
