"""Pins of the oracle's tree verification and of the expected-length formula.

Pages: "Speculative-Decoding, LLM推理的加速 / Medusa 方法阅读"
  * section 三: every node's logits come from one tree-masked forward; the LLM's
    own sampler (greedy or sampling) picks a token from the root's logits, a
    level-1 candidate holding it is followed, and so on level by level until a
    path ends or no child matches;
  * section 四: E[L] = sum over the nodes of the tree of the product of the
    per-level accuracies along the node's path, under independence.
"Accelerating Sonar through speculation", section "EAGLE": the longest
suitable candidate sequence is kept and one more target token appended.
"""
import itertools

import numpy as np
import pytest

import gen
import oracle
from tests import _np_ref as R

F16, F32 = R.DT_F16, R.DT_F32


def _read_golden(name):
    vals = {}
    for line in open(f"tests/golden/{name}"):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        vals[k] = float(v)
    return vals


def _brute_expected_len(parent, rank, acc):
    """Enumerate every per-level outcome (which rank is right, or none) with its
    probability and take the deepest prefix-closed match: no formula involved."""
    parent, rank = list(parent), list(rank)
    K, S = acc.shape
    depth = gen.tree_depths(np.asarray(parent, np.int32))
    children = {}
    for i in range(1, len(parent)):
        children.setdefault(parent[i], {})[rank[i]] = i
    E = 0.0
    for outcome in itertools.product(range(S + 1), repeat=K):   # 0 = no rank right
        p = 1.0
        for j, o in enumerate(outcome):
            p *= (1.0 - acc[j].sum()) if o == 0 else acc[j, o - 1]
        node, L = 0, 0
        for o in outcome:
            nxt = children.get(node, {}).get(o) if o else None
            if nxt is None:
                break
            node, L = nxt, L + 1
        E += p * L
    return E


def _random_prefix_closed_tree(rng, K, S, n_extra):
    parent, rank, depth = [-1], [0], [0]
    slots = {(0, r) for r in range(1, S + 1)}
    for _ in range(n_extra):
        if not slots:
            break
        p, r = sorted(slots)[int(rng.integers(len(slots)))]
        slots.discard((p, r))
        parent.append(p)
        rank.append(r)
        depth.append(depth[p] + 1)
        i = len(parent) - 1
        if depth[i] < K:
            slots |= {(i, rr) for rr in range(1, S + 1)}
    return np.asarray(parent, np.int32), np.asarray(rank, np.int32)


def test_expected_len_formula_matches_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(200):
        K, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        parent, rank = _random_prefix_closed_tree(rng, K, S, int(rng.integers(1, 12)))
        acc = rng.dirichlet(np.ones(S + 1), size=K)[:, :S]
        f = oracle.expected_accept_len(parent, rank, acc)
        assert abs(f - _brute_expected_len(parent, rank, acc)) < 1e-12, trial


def test_expected_len_of_full_tree_matches_golden():
    golden = _read_golden("medusa_expected_len_c5.txt")["expected_len"]
    parent, rank = gen.cartesian_tree([8, 8, 8, 8])
    acc = np.zeros((4, 8))
    acc[:, 0] = [0.8 ** k for k in range(1, 5)]
    assert abs(oracle.expected_accept_len(parent, rank, acc) - golden) < 1e-10


@pytest.mark.parametrize("mut", [oracle.MUT_NONE, oracle.MUT_TREE_NO_ANCESTOR])
def test_greedy_walk_mean_length_matches_formula(mut):
    # Full-tree candidate law (rank-1 right with prob 0.8^k) on a narrower
    # Cartesian tree: only the rank-1 chain can match, so the mean accepted
    # length must approach the same 1.6815181824.
    golden = _read_golden("medusa_expected_len_c5.txt")["expected_len"]
    w = gen.c5_medusa_full(seed=11, mode="greedy", B=6000, V=16, s_list=(2, 2, 2, 2))
    with oracle.mutation(mut):
        res = oracle.verify_tree("greedy", 1.0, w.parent, w.cand, w.logits, None, w.V, w.dtype,
                                 w.max_depth)
    assert np.all(res["err_flags"] == 0)
    L = res["accept_len"].astype(np.float64)
    se = L.std() / np.sqrt(len(L))
    ok = abs(L.mean() - golden) < 4.5 * se
    assert ok if mut == oracle.MUT_NONE else not ok


def test_chain_tree_equals_linear_greedy():
    rng = np.random.default_rng(21)
    B, k, V = 200, 4, 24
    t = (np.round(rng.normal(0, 2, size=(B, k + 1, V)) * 2) / 2).astype(np.float32)
    am = np.argmax(t, axis=2)
    x = np.where(rng.random((B, k)) < 0.7, am[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    lin = oracle.verify_linear("greedy", 1.0, t, None, x, None, V, F32)
    parent = np.arange(-1, k, dtype=np.int32)
    cand = np.concatenate([np.full((B, 1), -1, np.int32), x], axis=1)
    tr = oracle.verify_tree("greedy", 1.0, parent, cand, t, None, V, F32, k)
    np.testing.assert_array_equal(tr["accept_len"], lin["accept_len"])
    np.testing.assert_array_equal(tr["out_tokens"], lin["out_tokens"])


def test_star_tree():
    rng = np.random.default_rng(5)
    B, n, V = 300, 6, 20
    logits = rng.normal(0, 2, size=(B, n + 1, V)).astype(np.float32)
    parent = np.array([-1] + [0] * n, np.int32)
    cand = np.concatenate([np.full((B, 1), -1), rng.integers(0, V, (B, n))], axis=1).astype(np.int32)
    res = oracle.verify_tree("greedy", 1.0, parent, cand, logits, None, V, F32, 1)
    root_am = np.argmax(logits[:, 0], axis=1)
    hit = np.array([root_am[b] in cand[b, 1:] for b in range(B)])
    np.testing.assert_array_equal(res["accept_len"], hit.astype(np.int32))
    for b in range(B):
        if hit[b]:
            node = res["path_nodes"][b, 0]
            assert cand[b, node] == root_am[b] and node == 1 + list(cand[b, 1:]).index(root_am[b])
            assert res["out_tokens"][b, 1] == np.argmax(logits[b, node])
        else:
            assert res["out_tokens"][b, 0] == root_am[b]


def test_stochastic_root_token_follows_root_distribution():
    rng = np.random.default_rng(17)
    n_trials, V, T = 40000, 5, 0.8
    parent = np.array([-1, 0, 0, 1], np.int32)
    row = rng.normal(0, 1.2, size=(4, V)).astype(np.float32)
    logits = np.ascontiguousarray(np.broadcast_to(row, (n_trials, 4, V)))
    cand = np.tile(np.array([-1, 0, 3, 1], np.int32), (n_trials, 1))
    u = (rng.integers(0, 1 << 24, size=(n_trials, 4)) * 2.0 ** -24).astype(np.float32)
    res = oracle.verify_tree("stochastic", T, parent, cand, logits, u, V, F32, 2)
    p_root = R.softmax(row[0].astype(np.float64), T)
    assert R.chi2_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), p_root) > 1e-4


def test_stochastic_expected_len_given_logits():
    # distinct siblings: E[L | logits] = sum over nodes of the product, along the
    # node's path, of the parent's probability of the child's token
    rng = np.random.default_rng(23)
    n_trials, V, T = 50000, 6, 1.0
    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 4], np.int32)
    n = len(parent)
    row = rng.normal(0, 1.0, size=(n, V)).astype(np.float32)
    cand1 = np.array([-1, 0, 1, 2, 3, 0, 5, 2], np.int32)
    probs = np.array([R.softmax(r.astype(np.float64), T) for r in row])
    path_p = np.ones(n)
    for i in range(1, n):
        path_p[i] = path_p[parent[i]] * probs[parent[i], cand1[i]]
    want = path_p[1:].sum()
    logits = np.ascontiguousarray(np.broadcast_to(row, (n_trials, n, V)))
    cand = np.tile(cand1, (n_trials, 1))
    u = (rng.integers(0, 1 << 24, size=(n_trials, n)) * 2.0 ** -24).astype(np.float32)
    res = oracle.verify_tree("stochastic", T, parent, cand, logits, u, V, F32, 3)
    L = res["accept_len"].astype(np.float64)
    assert abs(L.mean() - want) < 5 * L.std() / np.sqrt(n_trials)


def test_tree_data_errors():
    V = 10
    logits = np.zeros((4, 4, V), np.float32)
    logits[:, :, 3] = 1.0
    good_parent = np.array([[-1, 0, 0, 1]] * 4, np.int32)
    parent = good_parent.copy()
    parent[1, 2] = 2          # not an earlier node
    parent[2, 0] = 0          # root must have no parent
    cand = np.array([[-1, 3, 4, 3]] * 4, np.int32)
    cand[3, 1] = V            # out of range
    res = oracle.verify_tree("greedy", 1.0, parent, cand, logits, None, V, F32, 2)
    assert list(res["err_flags"]) == [0, 4, 4, 1]
    assert res["accept_len"][0] == 2 and list(res["accept_len"][1:]) == [-1, -1, -1]
    assert list(res["path_nodes"][0]) == [1, 3]
    shallow = oracle.verify_tree("greedy", 1.0, good_parent, cand, logits, None, V, F32, 1)
    assert np.all(shallow["err_flags"][:3] & 4)


def test_root_only_tree():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(3, 1, 7)).astype(np.float32)
    res = oracle.verify_tree("greedy", 1.0, np.array([-1], np.int32), np.full((3, 1), -1, np.int32),
                             logits, None, 7, F32, 0)
    assert np.all(res["accept_len"] == 0)
    np.testing.assert_array_equal(res["out_tokens"][:, 0], np.argmax(logits[:, 0], axis=1))
