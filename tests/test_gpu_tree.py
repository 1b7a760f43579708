"""GPU parity of candidate-tree verification against the oracle.

Bar: accept_len, path_nodes and out_tokens bit-exact (greedy: always;
stochastic: except trees with an accepted node whose uniform lies within 1e-6
of one of its bin edges, counted)."""
import numpy as np
import pytest

import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _check(w, trees=None, max_depth=None):
    G.say(f"{w.name} {w.mode} B={w.B} N={w.n_nodes} V={w.V} dtype={w.dtype}")
    g = G.run_tree(w, max_depth)
    o = G.oracle_tree(w, trees, max_depth)
    near, n_eval = G.compare_tree(g, o, trees)
    return g, o, near, n_eval


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_c4_sparse_tree_full_size(seed):
    w = gen.c4_medusa_sparse(seed)          # B=16, 64 nodes + root, V=32000, fp16, greedy
    g, o, _, _ = _check(w)
    assert np.all(g["err_flags"] == 0)


@pytest.mark.parametrize("seed", [4, 5])
def test_c4_sparse_tree_stochastic(seed):
    w = gen.c4_medusa_sparse(seed, mode="stochastic")
    _check(w)


def test_c5_full_tree_greedy():
    w = gen.c5_medusa_full(0)               # B=4, 4680 nodes + root, V=32000, fp16
    g, o, _, _ = _check(w)
    assert w.n_nodes == 4681


def test_c5_full_tree_stochastic():
    w = gen.c5_medusa_full(1, mode="stochastic")
    _check(w)                               # every tree of the batch against the oracle


@pytest.mark.parametrize("dtype", [gen.DT_F32, gen.DT_BF16, gen.DT_F16])
@pytest.mark.parametrize("V", [12345, 20000, 7])
@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_small_trees_ragged(dtype, V, mode):
    parent, rank = gen.cartesian_tree([3, 2, 2])
    n = len(parent)
    B = 6
    logits_d = gen.normal_pair(gen.key(60, V, 1), 2.0, 0, 0.0, B * n * V, dtype, want_b=False)[0]
    logits = logits_d.reshape(B, n, V)
    am = gen.argmax_rows(dtype, logits, V).reshape(B, n)
    rng = np.random.default_rng(V + dtype)
    cand = np.where(rng.random((B, n)) < 0.6, am[:, parent], rng.integers(0, V, (B, n))).astype(np.int32)
    cand[:, 0] = -1
    u = gen.uniforms(gen.key(60, V, 4), B * n).reshape(B, n)
    w = gen.TreeWorkload("small", mode, 0.9, B, n, V, dtype, parent, cand, logits, u, 3)
    _check(w)


def test_chain_tree_equals_linear_greedy():
    lw = gen.linear_draft_target(61, 0, 16, 4, 9000, gen.DT_BF16, 2.0, 0.3, "greedy", 1.0, "chain")
    parent = np.arange(-1, 4, dtype=np.int32)
    cand = np.concatenate([np.full((16, 1), -1, np.int32), lw.draft_tokens], axis=1)
    w = gen.TreeWorkload("chain", "greedy", 1.0, 16, 5, lw.V, lw.dtype, parent, cand, lw.target,
                         np.zeros((16, 5), np.float32), 4)
    g, o, _, _ = _check(w)
    lin = G.run_linear(lw)
    np.testing.assert_array_equal(g["accept_len"], lin["accept_len"])
    np.testing.assert_array_equal(g["out_tokens"], lin["out_tokens"])


def test_per_tree_parents_and_errors():
    B, V = 5, 4000
    n = 6
    rng = np.random.default_rng(8)
    logits = gen.round_to(gen.DT_F16, rng.normal(0, 2, size=(B, n, V)))
    am = np.argmax(gen.decode(gen.DT_F16, logits), axis=2)
    parent = np.tile(np.array([-1, 0, 0, 1, 3, 4], np.int32), (B, 1))
    cand = np.zeros((B, n), np.int32)
    for b in range(B):
        for i in range(1, n):
            cand[b, i] = am[b, parent[b, i]]
    parent[1, 4] = 4          # not an earlier node
    parent[2, 0] = 3          # the root must have parent -1
    cand[3, 2] = V + 1        # candidate out of range
    w = gen.TreeWorkload("errs", "greedy", 1.0, B, n, V, gen.DT_F16, parent, cand, logits,
                         np.zeros((B, n), np.float32), 4)
    g, o, _, _ = _check(w)
    assert list(g["err_flags"]) == [0, 4, 4, 1, 0]
    assert g["accept_len"][0] == 4 and g["accept_len"][4] == 4
    # a bound below the tree's depth is an error for every tree
    g2, o2, _, _ = _check(w, max_depth=3)
    assert np.all(g2["err_flags"] & 4)


def test_root_only_tree():
    B, V = 3, 1000
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(B, 1, V)).astype(np.float32)
    for mode in ("greedy", "stochastic"):
        w = gen.TreeWorkload("root", mode, 1.0, B, 1, V, gen.DT_F32, np.array([-1], np.int32),
                             np.full((B, 1), -1, np.int32), logits,
                             gen.uniforms(gen.key(1, 1, 1), B).reshape(B, 1), 0)
        g, o, _, _ = _check(w)
        assert np.all(g["accept_len"] == 0)


@pytest.mark.parametrize("shape", [[2, 2, 2, 2], [3, 3, 3, 3, 3, 3]])
def test_stochastic_tree_deep_acceptance(shape):
    # Rows with one dominant token (all but about 1e-5 of the mass at T = 1) make the
    # drawn tokens predictable, so candidates equal to the parent's dominant
    # token are accepted level after level, and where siblings share a
    # candidate, several nodes of one level are. The small batch (248 rows)
    # draws every node while streaming; the large one (8744 rows) draws in the
    # walk, at every accepted node.
    parent, rank = gen.cartesian_tree(shape)
    n = len(parent)
    B, V = 8, 3000
    rng = np.random.default_rng(77)
    dom = rng.integers(0, V, size=(B, n))
    x = rng.normal(0.0, 1.0, size=(B, n, V))
    x[np.arange(B)[:, None], np.arange(n)[None, :], dom] += 20.0
    logits = gen.round_to(gen.DT_BF16, x)
    cand = np.empty((B, n), np.int32)
    cand[:, 0] = -1
    for b in range(B):
        for i in range(1, n):
            if b < 4 or rank[i] == 1:        # trees 0-3: siblings share the candidate
                cand[b, i] = dom[b, parent[i]]
            else:
                cand[b, i] = (dom[b, parent[i]] + 1 + rng.integers(0, V - 1)) % V
    u = gen.uniforms(gen.key(62, V, 4), B * n).reshape(B, n)
    w = gen.TreeWorkload("dominant", "stochastic", 1.0, B, n, V, gen.DT_BF16, parent, cand, logits, u,
                         len(shape))
    g, o, _, _ = _check(w)
    assert np.all(g["err_flags"] == 0)
    assert g["accept_len"].mean() >= 2.0
    # trees 0-3 accept more nodes than their path holds: several draws per level
    assert np.sum(o["n_eval"][:4]) > np.sum(o["accept_len"][:4] + 1) + 4


@pytest.mark.parametrize("n", [256, 257])
@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_random_trees_at_the_wave_walk_bound(n, mode):
    # Trees of at most 256 nodes whose tokens are known while streaming are walked
    # by one wave of the streaming launch (four nodes per lane); a 257-node tree
    # goes to the walk launch. Random recursive trees (each parent uniform among
    # the earlier nodes) with one dominant token per row, so that long paths are
    # accepted; then a depth bound one below the deepest node is an error for
    # every tree on both paths.
    rng = np.random.default_rng(n * 3 + (mode == "stochastic"))
    parent = np.array([-1] + [rng.integers(0, i) for i in range(1, n)], np.int32)
    depth = np.zeros(n, np.int64)
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    B, V = 6, 2000
    dom = rng.integers(0, V, size=(B, n))
    x = rng.normal(0.0, 1.0, size=(B, n, V))
    x[np.arange(B)[:, None], np.arange(n)[None, :], dom] += 20.0
    logits = gen.round_to(gen.DT_BF16, x)
    cand = np.where(rng.random((B, n)) < 0.7, dom[:, parent], rng.integers(0, V, (B, n))).astype(np.int32)
    cand[:, 0] = -1
    u = gen.uniforms(gen.key(64, n, 5), B * n).reshape(B, n)
    w = gen.TreeWorkload("wavewalk", mode, 1.0, B, n, V, gen.DT_BF16, parent, cand, logits, u,
                         int(depth.max()))
    g, o, _, _ = _check(w)
    assert np.all(g["err_flags"] == 0)
    assert g["accept_len"].max() >= 3
    g2, _, _, _ = _check(w, max_depth=int(depth.max()) - 1)
    assert np.all(g2["err_flags"] & 4)


@pytest.mark.parametrize("mode", ["greedy", "stochastic", "typical"])
def test_row_waves_large_batch_ragged_rows(mode):
    # More than 4096 rows in a batch: one wave streams each row, two chunks in
    # flight. bf16 rows of V = 20001 have five chunks (an odd count, the last one
    # ragged). Two random recursive trees of 2100 nodes, dominant tokens so that
    # paths several levels deep are accepted.
    import dataclasses
    import oracle
    rng = np.random.default_rng(21)
    n, B, V = 2100, 2, 20001
    parent = np.array([-1] + [rng.integers(0, i) for i in range(1, n)], np.int32)
    depth = np.zeros(n, np.int64)
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    dom = rng.integers(0, V, size=(B, n))
    x = rng.normal(0.0, 1.0, size=(B, n, V)).astype(np.float32)
    x[np.arange(B)[:, None], np.arange(n)[None, :], dom] += 20.0
    logits = gen.round_to(gen.DT_BF16, x)
    cand = np.where(rng.random((B, n)) < 0.8, dom[:, parent], rng.integers(0, V, (B, n))).astype(np.int32)
    cand[:, 0] = -1
    u = gen.uniforms(gen.key(65, n, 1), B * n).reshape(B, n)
    w = gen.TreeWorkload("rowwaves", "greedy" if mode == "greedy" else "stochastic", 1.0, B, n, V, gen.DT_BF16,
                         parent, cand, logits, u, int(depth.max()))
    if mode != "typical":
        g, o, _, _ = _check(w)
    else:
        G.say(f"typical rowwaves B={B} N={n} V={V}")
        g = G.run_tree(dataclasses.replace(w, mode="typical"), None, epsilon=0.09, delta=0.3)
        o = oracle.verify_tree_typical(1.0, 0.09, 0.3, parent, cand, logits, u, V, gen.DT_BF16, w.max_depth,
                                       G.TIE_EPS)
        G.compare_tree(g, o)
    assert np.all(g["err_flags"] == 0)
    assert g["accept_len"].max() >= 2
