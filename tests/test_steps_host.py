"""CPU checks of the steps around verification: the greedy sparse-tree builder
(host code in the library) against the oracle, bit for bit, and argument
validation of the new entry points (no device work is started)."""
import ctypes

import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import oracle


@pytest.mark.parametrize("K,S,budget,seed", [(4, 8, 64, 0), (4, 8, 4680, 1), (3, 5, 40, 2), (1, 10, 3, 3),
                                             (5, 4, 300, 4), (4, 8, 0, 5)])
def test_tree_build_greedy_matches_oracle(K, S, budget, seed):
    rng = np.random.default_rng(seed)
    acc = rng.uniform(0.0, 1.0, size=(K, S))
    acc[0, 0] = 1.0
    g = sv.tree_build_greedy(acc, budget)
    o = oracle.tree_build_greedy(acc, budget)
    for key in ("parent", "depth", "rank"):
        np.testing.assert_array_equal(g[key], o[key])
    assert g["expected_len"] == o["expected_len"]


def test_tree_build_greedy_ties():
    # equal accuracies everywhere: ties decided by depth, parent, rank alike
    acc = np.full((3, 4), 0.5)
    for budget in (1, 5, 9, 30):
        g = sv.tree_build_greedy(acc, budget)
        o = oracle.tree_build_greedy(acc, budget)
        for key in ("parent", "depth", "rank"):
            np.testing.assert_array_equal(g[key], o[key])


def test_tree_build_greedy_validation():
    L = sv.lib()
    acc = np.full((2, 2), 0.5)
    out = np.empty(8, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.spec_tree_build_greedy(0, 2, p(acc), 3, p(out), None, None, None) == -1
    bad = acc.copy()
    bad[1, 1] = 1.5
    assert L.spec_tree_build_greedy(2, 2, p(bad), 3, p(out), None, None, None) == -1
    assert L.spec_tree_build_greedy(2, 2, p(acc), sv.SV_MAX_TREE_NODES, p(out), None, None, None) == -5


D = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_commit_validation():
    L = sv.lib()
    assert L.spec_commit_linear(-1, 1, D, D, D, D, D, 8, D, D, D, None) == 1
    assert L.spec_commit_linear(2, 32, D, D, D, D, D, 8, D, D, D, None) == 5
    assert L.spec_commit_linear(2, 1, None, D, D, D, D, 8, D, D, D, None) == 1
    assert L.spec_commit_linear(2, 1, D, D, None, D, D, 8, D, D, D, None) == 1   # shifted needs drafts
    assert L.spec_commit_linear(2, 1, D, D, D, D, None, 8, D, D, D, None) == 1   # capacity without history
    assert L.spec_commit_linear(0, 1, None, None, None, None, None, 0, None, None, None, None) == 0


def test_sample_validation():
    L = sv.lib()
    need = L.spec_sample_workspace(4, 1000, 1)
    assert need > 0
    assert L.spec_sample(1, 1.0, 4, 1000, 7, D, D, D, None, D, need, None) == 2
    assert L.spec_sample(1, 0.0, 4, 1000, 1, D, D, D, None, D, need, None) == 1
    assert L.spec_sample(1, 1.0, 4, 1000, 1, D, None, D, None, D, need, None) == 1
    assert L.spec_sample(0, 1.0, 4, 1000, 1, D, None, None, None, D, need, None) == 1
    assert L.spec_sample(1, 1.0, 4, 1000, 1, D, D, D, None, D, need - 1, None) == 3
    assert L.spec_sample(1, 1.0, 4, 3_000_000, 1, D, D, D, None, D, need, None) == 5


def test_tree_mask_validation():
    L = sv.lib()
    assert L.spec_tree_mask(1, 0, D, 0, D, None, None) == 1
    assert L.spec_tree_mask(1, sv.SV_MAX_TREE_NODES + 1, D, 0, D, None, None) == 5
    assert L.spec_tree_mask(1, 5, None, 0, D, None, None) == 1
    assert L.spec_tree_mask(0, 5, None, 0, None, None, None) == 0
