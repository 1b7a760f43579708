"""Pins of the oracle's steps around verification: commit, sampler, tree mask and
greedy tree construction. Each is checked against what the pages and the
mathematics fix, not against a retyped copy of itself:

* commit (Sonar page, "MTP-Zeitplan für ein einzelnes Token" and "Inferenz mit
  spekulativem Decoding"): speculative greedy decoding of a Markov-chain "model"
  (verify, then commit, round after round) must produce exactly the tokens of
  plain greedy decoding of the target, whatever the draft; the shifted buffer is
  the verification input shifted one place left with the target token inserted;
* sampler: chi-square of its draws against softmax(x / T); greedy = first argmax;
* tree mask (Medusa page, section 三): a chain gives the causal (lower-triangular)
  mask; a star gives the identity plus the root column; the K = 4, top-8 Cartesian
  tree has sum over nodes of (depth + 1) ones; the relation is transitive and
  antisymmetric;
* greedy tree (Medusa page, section 四): with a budget of all 4680 nodes it is the
  full Cartesian tree; on small cases its expected length is the maximum over
  every tree of that size (brute force); its reported expected length equals the
  page's formula evaluated on it.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import gen
import oracle


# ------------------------------------------------------------------ commit
def _greedy_chain(table, t0, n):
    out = [t0]
    for _ in range(n):
        out.append(int(np.argmax(table[out[-1]])))
    return out


def _spec_decode(target_tab, draft_tab, t0, k, n_tokens, B=1):
    """Speculative greedy decoding with the oracle's verify + commit; a Markov
    chain: the logits after token t are row t of the table."""
    V = target_tab.shape[0]
    cap = n_tokens + k + 2
    hist = np.full((B, cap), -1, np.int32)
    hist[:, 0] = t0
    ln = np.ones(B, np.int32)
    rounds = 0
    while ln.min() < n_tokens + 1:
        assert rounds < 4 * n_tokens, "no progress"
        last = hist[np.arange(B), ln - 1]
        drafts = np.empty((B, k), np.int32)
        cur = last.copy()
        for i in range(k):
            cur = np.argmax(draft_tab[cur], axis=1).astype(np.int32)
            drafts[:, i] = cur
        inputs = np.concatenate([last[:, None], drafts], axis=1)          # [B][k+1]
        tgt = np.ascontiguousarray(target_tab[inputs].astype(np.float32))  # [B][k+1][V]
        o = oracle.verify_linear("greedy", 1.0, tgt, None, drafts, None, V, gen.DT_F32)
        ln, hist, c = oracle.commit_linear(o["accept_len"], o["out_tokens"], drafts, ln, hist)
        assert np.all(c["err_flags"] == 0)
        # the draft's next inputs: the verification inputs shifted one left, the
        # target's token inserted where the drafts stop being accepted
        for b in range(B):
            L = o["accept_len"][b]
            exp = np.concatenate([inputs[b, 1:], [o["out_tokens"][b, L]]])
            exp[L] = o["out_tokens"][b, L]
            np.testing.assert_array_equal(c["shifted"][b], exp)
            assert c["next_token"][b] == o["out_tokens"][b, L]
        rounds += 1
    return hist, ln, rounds


@pytest.mark.parametrize("k", [1, 3, 5])
def test_commit_speculative_greedy_equals_plain_greedy(k):
    rng = np.random.default_rng(100 + k)
    V = 40
    target = rng.normal(0, 2, size=(V, V))
    draft = target + rng.normal(0, 1.5, size=(V, V))     # often right, sometimes wrong
    n = 60
    hist, ln, rounds = _spec_decode(target, draft, 3, k, n, B=4)
    plain = _greedy_chain(target, 3, n)
    for b in range(4):
        np.testing.assert_array_equal(hist[b, :n + 1], plain)
    assert rounds < n      # drafts were accepted, several tokens per round


def test_commit_negative_control():
    rng = np.random.default_rng(7)
    V = 40
    target = rng.normal(0, 2, size=(V, V))
    draft = target + rng.normal(0, 1.5, size=(V, V))
    with oracle.mutation(oracle.MUT_COMMIT_REJECTED_DRAFT):
        try:
            hist, _, _ = _spec_decode(target, draft, 3, 3, 30)
            same = np.array_equal(hist[0, :31], _greedy_chain(target, 3, 30))
        except AssertionError:
            same = False
    assert not same


def test_commit_errors_leave_sequence_unchanged():
    acc = np.array([2, -1, 3, 0], np.int32)
    out = np.array([[5, 6, 7, -1], [-1, -1, -1, -1], [1, 2, 3, 4], [9, -1, -1, -1]], np.int32)
    drafts = np.array([[5, 6, 8], [1, 1, 1], [1, 2, 3], [4, 4, 4]], np.int32)
    ln0 = np.array([2, 2, 5, 2], np.int32)
    hist0 = np.zeros((4, 8), np.int32)
    ln, hist, c = oracle.commit_linear(acc, out, drafts, ln0, hist0)
    assert list(c["err_flags"]) == [0, 32, 16, 0]                   # unverified, capacity
    assert list(ln) == [5, 2, 5, 3]
    np.testing.assert_array_equal(hist[0, 2:5], [5, 6, 7])
    np.testing.assert_array_equal(hist[1], hist0[1])
    np.testing.assert_array_equal(hist[2], hist0[2])
    assert hist[3, 2] == 9
    np.testing.assert_array_equal(c["shifted"][1], [-1] * 4)
    np.testing.assert_array_equal(c["shifted"][3], [9, 4, 4, 9])    # L = 0: y first, y last
    assert list(c["next_token"]) == [7, -1, -1, 9]


# ------------------------------------------------------------------ sampler
@pytest.mark.parametrize("T", [0.5, 2.0])
def test_sample_chi_square(T):
    x = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4], np.float32)
    n = 20000
    u = gen.uniforms(gen.key(90, int(T * 10), 1), n).astype(np.float32)
    rows = np.tile(x, (n, 1))
    o = oracle.sample("stochastic", T, rows, u, 6, gen.DT_F32)
    p = np.exp(x.astype(np.float64) / T)
    p /= p.sum()
    counts = np.bincount(o["tokens"], minlength=6)
    chi = stats.chisquare(counts, p * n)
    assert chi.pvalue > 1e-3
    # and the wrong temperature is rejected
    q = np.exp(x.astype(np.float64) / (T * 2))
    q /= q.sum()
    assert stats.chisquare(counts, q * n).pvalue < 1e-6


def test_sample_greedy_and_errors():
    rows = np.array([[1.0, 3.0, 3.0, 2.0], [-np.inf] * 4, [0.0, np.nan, 5.0, 5.0]], np.float32)
    o = oracle.sample("greedy", 1.0, rows, None, 4, gen.DT_F32)
    assert list(o["tokens"]) == [1, -1, 2]
    assert list(o["err_flags"]) == [0, 2, 0]


# ------------------------------------------------------------------ tree mask
def test_mask_chain_is_causal():
    n = 40
    parent = np.arange(-1, n - 1, dtype=np.int32)
    np.testing.assert_array_equal(oracle.tree_mask(parent), np.tril(np.ones((n, n), np.uint8)))


def test_mask_star():
    n = 9
    parent = np.array([-1] + [0] * (n - 1), np.int32)
    m = oracle.tree_mask(parent)
    exp = np.eye(n, dtype=np.uint8)
    exp[:, 0] = 1
    np.testing.assert_array_equal(m, exp)


def test_mask_cartesian_counts_and_relation():
    parent, _ = gen.cartesian_tree([8, 8, 8, 8])
    m = oracle.tree_mask(parent).astype(np.int64)
    assert m.shape == (4681, 4681)
    # ones per row = depth + 1; in all sum_d 8^d (d + 1)
    assert m.sum() == sum(8 ** d * (d + 1) for d in range(5)) == 22737
    depth = np.zeros(len(parent), np.int64)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    np.testing.assert_array_equal(m.sum(axis=1), depth + 1)


def test_mask_relation_on_random_trees():
    rng = np.random.default_rng(3)
    for n in (2, 17, 120):
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)
        m = oracle.tree_mask(parent).astype(bool)
        assert np.all(np.diag(m))
        assert not np.any(m & m.T & ~np.eye(n, dtype=bool))          # antisymmetric
        mm = (m.astype(np.int64) @ m.astype(np.int64)) > 0
        np.testing.assert_array_equal(mm, m)                           # transitive
        # exactly the nodes met walking up the parents
        for i in range(n):
            j, seen = i, set()
            while j >= 0:
                seen.add(j)
                j = parent[j]
            assert set(np.nonzero(m[i])[0]) == seen


def test_mask_invalid():
    assert oracle.tree_mask(np.array([0, 0], np.int32)) is None
    assert oracle.tree_mask(np.array([-1, 1], np.int32)) is None


# ------------------------------------------------------------------ greedy tree
def test_greedy_full_budget_is_cartesian():
    rng = np.random.default_rng(11)
    acc = rng.uniform(0.01, 0.99, size=(4, 8))
    r = oracle.tree_build_greedy(acc, 4680)
    parent, rank = gen.cartesian_tree([8, 8, 8, 8])
    # same shape: breadth-first, children in rank order
    np.testing.assert_array_equal(r["parent"], parent)
    np.testing.assert_array_equal(r["rank"], rank)
    assert abs(r["expected_len"] - oracle.expected_accept_len(parent, rank, acc)) < 1e-12
    # more budget than nodes: the full tree and no more
    assert len(oracle.tree_build_greedy(acc, 5000)["parent"]) == 4681


def _prefix_closed_best(K, S, acc, size):
    parent, rank = gen.cartesian_tree([S] * K)
    n = len(parent)
    best = -1.0
    for sub in itertools.combinations(range(1, n), size):
        keep = set(sub) | {0}
        if any(parent[i] not in keep for i in sub):
            continue
        idx = sorted(keep)
        remap = {o: i for i, o in enumerate(idx)}
        par = np.array([-1] + [remap[parent[o]] for o in idx[1:]], np.int32)
        rk = np.array([0] + [rank[o] for o in idx[1:]], np.int32)
        best = max(best, oracle.expected_accept_len(par, rk, acc))
    return best


@pytest.mark.parametrize("K,S,size", [(3, 2, 4), (3, 2, 7), (2, 3, 5), (3, 3, 5)])
def test_greedy_is_optimal_on_small_trees(K, S, size):
    rng = np.random.default_rng(K * 10 + S + size)
    acc = rng.uniform(0.05, 0.95, size=(K, S))
    r = oracle.tree_build_greedy(acc, size)
    assert len(r["parent"]) == size + 1
    E = oracle.expected_accept_len(r["parent"], r["rank"], acc)
    assert abs(E - r["expected_len"]) < 1e-12
    assert abs(E - _prefix_closed_best(K, S, acc, size)) < 1e-12
    # a tree: parents come first, depth grows by one
    assert r["parent"][0] == -1 and np.all(r["parent"][1:] < np.arange(1, size + 1))
    np.testing.assert_array_equal(r["depth"][1:], r["depth"][r["parent"][1:]] + 1)


def test_greedy_medusa_accuracies():
    # a head-k accuracy table falling with depth and rank, 64 nodes: every node's
    # contribution is at least that of every node left out whose parent is in
    K, S = 4, 8
    acc = np.array([[0.8 ** k / (1 + r) for r in range(S)] for k in range(1, K + 1)])
    r = oracle.tree_build_greedy(acc, 64)
    par, rk, dep = r["parent"], r["rank"], r["depth"]
    val = np.ones(len(par))
    for i in range(1, len(par)):
        val[i] = val[par[i]] * acc[dep[i] - 1, rk[i] - 1]
    worst_in = val[1:].min()
    for i in range(len(par)):
        if dep[i] == K:
            continue
        have = set(rk[j] for j in range(len(par)) if par[j] == i)
        for rr in range(1, S + 1):
            if rr not in have:
                assert val[i] * acc[dep[i], rr - 1] <= worst_in
