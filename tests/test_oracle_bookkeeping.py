"""Pins of the oracle's parity bookkeeping: which draws count as evaluated
(n_eval) and which are near ties (near_tie), the two numbers that decide what a
GPU result may differ in and how the exception rate is counted.

The rule being pinned: a stochastic draw is evaluated when the result depends
on it, and it is a near tie when its uniform lies within tie_eps = 1e-6 of its
threshold -- the acceptance ratio min(1, p_t/p_d) for an accept test, either
edge of the selected bin for an inverse-CDF draw. A near tie that can change the
accepted length sets bit 1; one that can change only the final token sets bit 2.
The accept test is that of the Leviathan et al. method cited on the Sonar page
("Accelerating Sonar through speculation", sections "Spekulatives Decoding" and
"Ziel-Entwurf"); the tree walk is the Medusa page's (section 三).

Every expected value here comes from numpy arithmetic in the test (softmax,
cumulative sums, an independent acceptance walk), never from the oracle's own
intermediate values, and each pin fails under a planted mistake.
"""
import numpy as np
import pytest

import oracle
from tests import _np_ref as R

F32 = R.DT_F32
EPS = oracle.TIE_EPS
NEAR, FAR = 0.5e-6, 2e-6


def _f32(v):
    return np.float32(v)


# ------------------------------------------------------------------ linear
def _linear_k2(u0, u1=0.999, u2=0.5):
    """k = 2, V = 2, T = 1. Position 0: x_0 = 0 with q_0 = p_t0(0)/p_d0(0) < 1.
    Position 1: x_1 = 0 with a small q_1 (u_1 = 0.999 rejects it). Returns the
    oracle's result and q_0, q_1 from numpy."""
    t = np.array([[[0.0, 1.0], [0.0, 2.5], [0.3, -0.2]]], np.float32)
    d = np.array([[[1.0, 0.0], [2.0, -1.0]]], np.float32)
    x = np.array([[0, 0]], np.int32)
    u = np.array([[u0, u1, u2]], np.float32)
    q = [R.softmax(t[0, i].astype(np.float64), 1.0)[0] / R.softmax(d[0, i].astype(np.float64), 1.0)[0]
         for i in range(2)]
    res = oracle.verify_linear("stochastic", 1.0, t, d, x, u, 2, F32)
    return res, q


@pytest.mark.parametrize("delta,near", [(-NEAR, True), (NEAR, True), (-FAR, False), (FAR, False)])
def test_linear_accept_tie_flagged_within_eps(delta, near):
    _, q = _linear_k2(0.5)
    assert q[0] < 1 and q[1] < 0.5
    res, _ = _linear_k2(_f32(q[0] + delta))
    L = res["accept_len"][0]
    assert L == (1 if delta < 0 else 0)     # below the ratio accepts
    assert bool(res["near_tie"][0] & oracle.NT_DECISION) == near
    assert not res["near_tie"][0] & oracle.NT_FINAL   # u_2 = 0.5 is mid-bin
    assert res["n_eval"][0] == min(L + 1, 2) + 1


def test_linear_tie_in_a_draw_not_evaluated_is_not_flagged():
    # position 0 rejects (u_0 far above q_0): the accept test of position 1 is
    # never evaluated, so u_1 sitting on its ratio is no near tie
    _, q = _linear_k2(0.5)
    res, _ = _linear_k2(0.999, u1=_f32(q[1]))
    assert res["accept_len"][0] == 0
    assert res["near_tie"][0] == 0
    assert res["n_eval"][0] == 2        # the test of position 0 and the final draw
    # the same u_1 after an accepted position 0 is evaluated and flagged
    res, _ = _linear_k2(_f32(q[0] - 0.05), u1=_f32(q[1]))
    assert res["accept_len"][0] in (1, 2)
    assert res["near_tie"][0] & oracle.NT_DECISION
    assert res["n_eval"][0] == 3


def test_planted_accept_tie_off_fails_the_pin():
    _, q = _linear_k2(0.5)
    with oracle.mutation(oracle.MUT_ACCEPT_TIE_OFF):
        res, _ = _linear_k2(_f32(q[0] + NEAR))
    assert not res["near_tie"][0] & oracle.NT_DECISION


def _identity_final(u_last, V=4):
    """k = 2 with draft rows equal to target rows: every draft is accepted and the
    final token is drawn from target row 2 with u_last. Returns result and the
    numpy cumulative distribution of that row."""
    t = np.array([[[0.1, 0.5, -0.3, 0.9], [0.0, 0.2, 0.4, -1.0], [0.7, -0.1, 0.35, 0.2]]], np.float32)
    d = np.ascontiguousarray(t[:, :2])
    x = np.array([[1, 2]], np.int32)
    u = np.array([[0.3, 0.6, u_last]], np.float32)
    c = np.cumsum(R.softmax(t[0, 2].astype(np.float64), 1.0))
    return oracle.verify_linear("stochastic", 1.0, t, d, x, u, V, F32), c


@pytest.mark.parametrize("edge", [0, 1, 2])
@pytest.mark.parametrize("delta,near", [(-NEAR, True), (NEAR, True), (-FAR, False), (FAR, False)])
def test_linear_final_draw_tie_at_both_bin_edges(edge, delta, near):
    _, c = _identity_final(0.5)
    res, _ = _identity_final(_f32(c[edge] + delta))
    assert res["accept_len"][0] == 2
    y = res["out_tokens"][0, 2]
    assert y == (edge if delta < 0 else edge + 1)   # below the edge: the lower bin
    assert bool(res["near_tie"][0] & oracle.NT_FINAL) == near
    assert not res["near_tie"][0] & oracle.NT_DECISION
    assert res["n_eval"][0] == 3


def test_planted_one_edge_check_fails_the_pin():
    # u just below an edge selects the lower bin, whose upper edge is the close one
    _, c = _identity_final(0.5)
    with oracle.mutation(oracle.MUT_NEAR_LO_ONLY):
        res, _ = _identity_final(_f32(c[1] - NEAR))
    assert not res["near_tie"][0] & oracle.NT_FINAL


def _random_linear(seed, B=400, k=4, V=40):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 1.5, size=(B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.normal(0, 1.0, size=(B, k, V))).astype(np.float32)
    x = rng.integers(0, V, size=(B, k)).astype(np.int32)
    x[::37, 0] = V          # a few token errors: nothing is evaluated there
    u = (rng.integers(0, 1 << 24, size=(B, k + 1)) * 2.0 ** -24).astype(np.float32)
    return t, d, x, u, V


def test_linear_n_eval_counts_the_draws_the_result_depends_on():
    t, d, x, u, V = _random_linear(3)
    k = x.shape[1]
    res = oracle.verify_linear("stochastic", 0.8, t, d, x, u, V, F32)
    L, err = res["accept_len"], res["err_flags"]
    ok = err == 0
    assert (~ok).any() and (L[ok] < k).any() and (L[ok] == k).any()
    want = np.where(ok, np.minimum(L + 1, k) + 1, 0)
    np.testing.assert_array_equal(res["n_eval"], want)
    assert np.all(res["near_tie"][~ok] == 0)
    g = oracle.verify_linear("greedy", 1.0, t, None, x, None, V, F32)
    assert np.all(g["n_eval"] == 0) and np.all(g["near_tie"] == 0)


def test_planted_overcount_fails_the_n_eval_pin():
    t, d, x, u, V = _random_linear(3)
    k = x.shape[1]
    with oracle.mutation(oracle.MUT_NEVAL_ALL):
        res = oracle.verify_linear("stochastic", 0.8, t, d, x, u, V, F32)
    ok = res["err_flags"] == 0
    want = np.where(ok, np.minimum(res["accept_len"] + 1, k) + 1, 0)
    assert np.any(res["n_eval"] != want)


def test_near_tie_rate_is_small_on_random_inputs():
    # with uniforms on a 2^-24 grid, about 2e-6 of accept tests and 4e-6 of draws
    # fall within 1e-6 of a threshold; on 400 sequences the flags stay rare
    t, d, x, u, V = _random_linear(5)
    res = oracle.verify_linear("stochastic", 0.8, t, d, x, u, V, F32)
    assert np.count_nonzero(res["near_tie"]) <= 2


# ------------------------------------------------------------------ trees
def _tree_case(u, cand, V=4):
    """Root 0 with children 1 and 2; node 1 has child 3. One logits row per node."""
    parent = np.array([-1, 0, 0, 1], np.int32)
    lg = np.array([[[0.2, 0.9, -0.4, 0.1], [0.5, 0.1, 0.3, -0.2], [0.0, 0.0, 0.4, 0.4],
                    [0.3, -0.6, 0.8, 0.05]]], np.float32)
    cdf = [np.cumsum(R.softmax(lg[0, n].astype(np.float64), 1.0)) for n in range(4)]
    res = oracle.verify_tree("stochastic", 1.0, parent, np.asarray([cand], np.int32), lg,
                             np.asarray([u], np.float32), V, F32, 3)
    return res, cdf


def test_tree_tie_at_a_node_with_children_changes_the_path():
    _, cdf = _tree_case([0.5, 0.5, 0.5, 0.5], [0, 1, 3, 0])
    # root draw just above its first edge picks token 1 = candidate of node 1;
    # node 1's draw mid-bin picks token 0 = candidate of node 3 (a leaf)
    u1 = 0.5 * cdf[1][0]
    for delta, near in ((NEAR, True), (FAR, False)):
        res, _ = _tree_case([_f32(cdf[0][0] + delta), _f32(u1), 0.5, 0.5], [0, 1, 3, 0])
        assert res["accept_len"][0] == 2 and list(res["path_nodes"][0, :2]) == [1, 3]
        assert bool(res["near_tie"][0] & oracle.NT_DECISION) == near
        assert res["n_eval"][0] == 3     # root, node 1, node 3 accepted


def test_tree_tie_at_the_final_leaf_is_final_only():
    _, cdf = _tree_case([0.5, 0.5, 0.5, 0.5], [0, 1, 3, 0])
    u1 = 0.5 * cdf[1][0]
    for delta, near in ((-NEAR, True), (NEAR, True), (FAR, False)):
        res, _ = _tree_case([_f32(0.5 * (cdf[0][0] + cdf[0][1])), _f32(u1), 0.5,
                             _f32(cdf[3][1] + delta)], [0, 1, 3, 0])
        assert res["accept_len"][0] == 2
        assert res["near_tie"][0] == (oracle.NT_FINAL if near else 0)


def _accepted_count(parent, cand, node_token):
    acc = np.zeros(len(parent), bool)
    acc[0] = True
    for i in range(1, len(parent)):
        acc[i] = acc[parent[i]] and cand[i] == node_token[parent[i]]
    return int(acc.sum())


def test_tree_n_eval_is_the_count_of_accepted_nodes():
    rng = np.random.default_rng(17)
    B, V = 60, 6
    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 4, 4, 7, 3], np.int32)
    n = len(parent)
    lg = rng.normal(0, 2, size=(B, n, V)).astype(np.float32)
    cand = rng.integers(0, V, size=(B, n)).astype(np.int32)
    # make many candidates match the likely token, so paths are often deep
    for b in range(B):
        for i in range(1, n):
            if rng.random() < 0.6:
                cand[b, i] = int(np.argmax(lg[b, parent[i]]))
    u = (rng.integers(0, 1 << 24, size=(B, n)) * 2.0 ** -24).astype(np.float32)
    res = oracle.verify_tree("stochastic", 1.0, parent, cand, lg, u, V, F32, 4)
    want = [_accepted_count(parent, cand[b], res["node_token"][b]) for b in range(B)]
    np.testing.assert_array_equal(res["n_eval"], want)
    assert max(want) >= 3
    with oracle.mutation(oracle.MUT_NEVAL_ALL):
        bad = oracle.verify_tree("stochastic", 1.0, parent, cand, lg, u, V, F32, 4)
    assert np.any(bad["n_eval"] != want)
    g = oracle.verify_tree("greedy", 1.0, parent, cand, lg, None, V, F32, 4)
    assert np.all(g["n_eval"] == 0) and np.all(g["near_tie"] == 0)


# ------------------------------------------------------------------ sampler, typical
@pytest.mark.parametrize("delta,near", [(-NEAR, True), (NEAR, True), (-FAR, False), (FAR, False)])
def test_sample_tie_at_bin_edges(delta, near):
    x = np.array([[0.4, -0.2, 1.1, 0.3, 0.0]], np.float32)
    c = np.cumsum(R.softmax(x[0].astype(np.float64), 0.9))
    for edge in range(4):
        res = oracle.sample("stochastic", 0.9, x, [_f32(c[edge] + delta)], 5, F32)
        assert res["tokens"][0] == (edge if delta < 0 else edge + 1)
        assert res["near_tie"][0] == (oracle.NT_FINAL if near else 0)


def test_planted_one_edge_check_fails_the_sample_pin():
    x = np.array([[0.4, -0.2, 1.1, 0.3, 0.0]], np.float32)
    c = np.cumsum(R.softmax(x[0].astype(np.float64), 0.9))
    with oracle.mutation(oracle.MUT_NEAR_LO_ONLY):
        res = oracle.sample("stochastic", 0.9, x, [_f32(c[2] - NEAR)], 5, F32)
    assert res["near_tie"][0] == 0


def _typical_uniform(delta_factor, u_last=0.3, V=4):
    """Uniform rows: p = 1/V, H = ln V, so with epsilon = 1 the threshold is
    delta/V and a candidate passes iff delta < 1; the pass test sits delta - 1 away
    (relative) from its threshold. Chain root - 1 - 2."""
    parent = np.array([-1, 0, 1], np.int32)
    lg = np.zeros((1, 3, V), np.float32)
    cand = np.array([[0, 2, 1]], np.int32)
    u = np.array([[0.3, 0.5, u_last]], np.float32)
    return oracle.verify_tree_typical(1.0, 1.0, delta_factor, parent, cand, lg, u, V, F32, 2)


@pytest.mark.parametrize("rel,near", [(-NEAR, True), (NEAR, True), (-FAR, False), (FAR, False)])
def test_typical_pass_test_tie_is_relative_to_the_threshold(rel, near):
    res = _typical_uniform(1.0 + rel)
    assert res["accept_len"][0] == (2 if rel < 0 else 0)
    assert bool(res["near_tie"][0] & oracle.NT_DECISION) == near
    # decisive tests: the children of accepted nodes (1 or 2 of them), plus the draw
    assert res["n_eval"][0] == (3 if rel < 0 else 2)


def test_typical_final_draw_tie():
    # uniform final row of 4 tokens: bin edges at 1/4, 1/2, 3/4
    for delta, near in ((-NEAR, True), (NEAR, True), (FAR, False)):
        res = _typical_uniform(0.5, u_last=_f32(0.5 + delta))
        assert res["accept_len"][0] == 2
        assert res["out_tokens"][0, 2] == (1 if delta < 0 else 2)
        assert res["near_tie"][0] == (oracle.NT_FINAL if near else 0)
    with oracle.mutation(oracle.MUT_ACCEPT_TIE_OFF):
        assert not _typical_uniform(1.0 + NEAR)["near_tie"][0] & oracle.NT_DECISION
