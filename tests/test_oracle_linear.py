"""Pins of the oracle's linear verification.

What the pages fix ("Accelerating Sonar through speculation"):
  * section "Spekulatives Decoding": the longest acceptable prefix is kept and a
    draft of n tokens yields up to n+1 tokens;
  * section "Ziel-Entwurf": acceptance compares the full draft and target
    distributions, and the target logits after the accepted prefix are sampled
    for one more token; the rule itself is the cited Leviathan et al. method.

Pins used here, none of which retypes the oracle's arithmetic:
  * identity: equal draft and target rows accept every draft plus one token;
  * losslessness (the cited method's theorem): the first emitted token follows
    the target row 0, and given acceptance the second follows target row 1 --
    chi-square on tiny vocabularies, with planted mistakes that must fail;
  * acceptance probability = sum_v min(p_t(v), p_d(v)) (same theorem);
  * greedy decisions against numpy's argmax.
"""
import numpy as np
import pytest

import oracle
from tests import _np_ref as R

F32 = R.DT_F32


def _u24(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) * 2.0 ** -24).astype(np.float32)


def _sample_rows(rng, probs, n):
    """n draws from each row of probs -> [n][rows]"""
    out = np.empty((n, probs.shape[0]), np.int32)
    for i, p in enumerate(probs):
        out[:, i] = rng.choice(len(p), size=n, p=p)
    return out


def _case(seed, V, k, T, n, spread=1.5):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, spread, size=(k + 1, V)).astype(np.float32)
    d = (t[:k] + rng.normal(0, 1.0, size=(k, V))).astype(np.float32)
    pt = np.array([R.softmax(r.astype(np.float64), T) for r in t])
    pd = np.array([R.softmax(r.astype(np.float64), T) for r in d])
    x = _sample_rows(rng, pd, n)
    u = _u24(rng, (n, k + 1))
    target = np.ascontiguousarray(np.broadcast_to(t, (n, k + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(d, (n, k, V)))
    return t, d, pt, pd, x, u, target, draft


CASES = [(2, 1, 1.0), (3, 2, 1.0), (4, 4, 0.7), (8, 2, 1.0), (8, 4, 0.7), (5, 1, 2.0)]


@pytest.mark.parametrize("V,k,T", CASES)
def test_lossless_first_and_second_token(V, k, T):
    n = 60000
    t, d, pt, pd, x, u, target, draft = _case(100 + V * 10 + k, V, k, T, n)
    res = oracle.verify_linear("stochastic", T, target, draft, x, u, V, F32)
    assert np.all(res["err_flags"] == 0)
    out, L = res["out_tokens"], res["accept_len"]
    assert np.all((L >= 0) & (L <= k))
    # first emitted token ~ target row 0
    assert R.chi2_pvalue(np.bincount(out[:, 0], minlength=V), pt[0]) > 1e-4
    # given the first draft was accepted, the second emitted token ~ target row 1
    sel = L >= 1
    if k >= 1 and sel.sum() > 500:
        assert R.chi2_pvalue(np.bincount(out[sel, 1], minlength=V), pt[1]) > 1e-4
    # accepted tokens are the drafts, then exactly one more token, then padding
    for b in range(0, n, 997):
        l = L[b]
        assert list(out[b, :l]) == list(x[b, :l])
        assert 0 <= out[b, l] < V
        assert all(out[b, l + 1:] == -1)


@pytest.mark.parametrize("V,k,T", CASES[:4])
def test_acceptance_probability_is_overlap(V, k, T):
    n = 60000
    t, d, pt, pd, x, u, target, draft = _case(200 + V * 10 + k, V, k, T, n)
    res = oracle.verify_linear("stochastic", T, target, draft, x, u, V, F32)
    freq = np.mean(res["accept_len"] >= 1)
    alpha = np.minimum(pt[0], pd[0]).sum()
    se = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(freq - alpha) < 5 * se + 1e-12


@pytest.mark.parametrize("mut", [oracle.MUT_RESIDUAL_AS_TARGET, oracle.MUT_SWAPPED_RATIO])
def test_planted_acceptance_mistakes_fail_losslessness(mut):
    V, k, T, n = 4, 1, 1.0, 60000
    t, d, pt, pd, x, u, target, draft = _case(31, V, k, T, n, spread=2.0)
    with oracle.mutation(mut):
        res = oracle.verify_linear("stochastic", T, target, draft, x, u, V, F32)
    assert R.chi2_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), pt[0]) < 1e-6


@pytest.mark.parametrize("k", [1, 3, 4])
def test_identity_accepts_everything_plus_one(k):
    rng = np.random.default_rng(40 + k)
    B, V, T = 300, 50, 0.8
    t = rng.normal(0, 2, size=(B, k + 1, V)).astype(np.float32)
    d = np.ascontiguousarray(t[:, :k])
    pd = np.array([[R.softmax(r.astype(np.float64), T) for r in tb] for tb in d])
    x = np.array([[rng.choice(V, p=p) for p in pb] for pb in pd], np.int32)
    u = _u24(rng, (B, k + 1))
    res = oracle.verify_linear("stochastic", T, t, d, x, u, V, F32)
    assert np.all(res["accept_len"] == k)
    np.testing.assert_array_equal(res["out_tokens"][:, :k], x)
    np.testing.assert_array_equal(res["p_target"], res["p_draft"])
    for b in range(B):
        c = np.cumsum(R.softmax(t[b, k].astype(np.float64), T))
        assert res["out_tokens"][b, k] == np.searchsorted(c, u[b, k] * c[-1], side="right")
    # greedy identity: draft tokens are the argmax of the (equal) rows
    xg = np.argmax(d, axis=2).astype(np.int32)
    g = oracle.verify_linear("greedy", 1.0, t, None, xg, None, V, F32)
    assert np.all(g["accept_len"] == k)
    np.testing.assert_array_equal(g["out_tokens"][:, k], np.argmax(t[:, k], axis=1))


def test_planted_missing_bonus_fails_identity():
    rng = np.random.default_rng(2)
    t = rng.normal(0, 2, size=(20, 3, 30)).astype(np.float32)
    x = np.argmax(t[:, :2], axis=2).astype(np.int32)
    u = _u24(rng, (20, 3))
    with oracle.mutation(oracle.MUT_NO_BONUS):
        res = oracle.verify_linear("stochastic", 1.0, t, np.ascontiguousarray(t[:, :2]), x, u, 30, F32)
    assert np.any(res["out_tokens"][:, 2] == -1)


def test_greedy_against_numpy_argmax():
    rng = np.random.default_rng(8)
    B, k, V = 400, 4, 40
    t = np.round(rng.normal(0, 2, size=(B, k + 1, V)) * 2) / 2   # frequent ties
    t = t.astype(np.float32)
    am = np.argmax(t, axis=2)
    # drafts agree with the target argmax for a random-length prefix
    x = am[:, :k].copy()
    cut = rng.integers(0, k + 1, size=B)
    for b in range(B):
        if cut[b] < k:
            x[b, cut[b]] = (am[b, cut[b]] + 1) % V
    res = oracle.verify_linear("greedy", 1.0, t, None, x.astype(np.int32), None, V, F32)
    np.testing.assert_array_equal(res["accept_len"], cut)
    for b in range(B):
        L = cut[b]
        assert list(res["out_tokens"][b, :L]) == list(x[b, :L])
        assert res["out_tokens"][b, L] == am[b, L]


def test_no_draft_is_plain_sampling():
    # k = 0: nothing to verify; the one emitted token is a draw from target row 0
    rng = np.random.default_rng(12)
    n, V, T = 40000, 6, 0.9
    t = rng.normal(0, 1.5, size=(1, 1, V)).astype(np.float32)
    target = np.ascontiguousarray(np.broadcast_to(t, (n, 1, V)))
    u = _u24(rng, (n, 1))
    res = oracle.verify_linear("stochastic", T, target, None, np.zeros((n, 0), np.int32), u, V, F32)
    assert np.all(res["accept_len"] == 0)
    assert R.chi2_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V),
                         R.softmax(t[0, 0].astype(np.float64), T)) > 1e-4
    g = oracle.verify_linear("greedy", 1.0, target[:5], None, np.zeros((5, 0), np.int32), None, V, F32)
    assert np.all(g["out_tokens"][:, 0] == np.argmax(t[0, 0]))


def test_data_errors_are_flagged():
    rng = np.random.default_rng(1)
    B, k, V = 4, 2, 16
    t = rng.normal(0, 1, size=(B, k + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, size=(B, k, V)).astype(np.float32)
    x = rng.integers(0, V, size=(B, k)).astype(np.int32)
    x[0, 1] = V          # token out of range
    t[1, 2, 3] = np.nan  # non-finite target row
    d[2, 0, :] = -np.inf  # draft row without usable logits
    u = _u24(rng, (B, k + 1))
    res = oracle.verify_linear("stochastic", 1.0, t, d, x, u, V, F32)
    assert list(res["err_flags"]) == [1, 2, 2, 0]
    assert list(res["accept_len"][:3]) == [-1, -1, -1]
    assert np.all(res["out_tokens"][:3] == -1)
    assert np.all(np.isnan(res["p_target"][:3]))
    assert res["accept_len"][3] >= 0
    g = oracle.verify_linear("greedy", 1.0, t, None, x, None, V, F32)
    # greedy ignores NaN entries and never reads the draft rows
    assert list(g["err_flags"]) == [1, 0, 0, 0]


# ------------------------------------------------------------------ exact laws
def _acc_prob(pt, pd, x):
    """min(1, p_t(x) / p_d(x)): the probability that draft token x is accepted."""
    return min(1.0, pt[x] / pd[x])


def _residual(pt, pd):
    r = np.maximum(pt - pd, 0.0)
    return r / r.sum()


def _exact_outcomes_v2_k2(pt, pd):
    """The law of (L, emitted tokens) for V = 2, k = 2, by enumerating the draft
    draws and accept events: draft x_i ~ p_d,i, accepted w.p. min(1, p_t,i/p_d,i);
    on the first reject at L the token comes from the normalised residual
    max(0, p_t,L - p_d,L) (a point mass when V = 2); with both accepted it comes
    from p_t,2."""
    law = {}
    r0, r1 = _residual(pt[0], pd[0]), _residual(pt[1], pd[1])
    for x0 in range(2):
        a0 = _acc_prob(pt[0], pd[0], x0)
        for y in range(2):
            law[(0, y)] = law.get((0, y), 0.0) + pd[0][x0] * (1 - a0) * r0[y]
        for x1 in range(2):
            a1 = _acc_prob(pt[1], pd[1], x1)
            for y in range(2):
                law[(1, x0, y)] = law.get((1, x0, y), 0.0) + pd[0][x0] * a0 * pd[1][x1] * (1 - a1) * r1[y]
                law[(2, x0, x1, y)] = pd[0][x0] * a0 * pd[1][x1] * a1 * pt[2][y]
    return law


def _v2_k2_case(n, seed=77):
    rng = np.random.default_rng(seed)
    t = np.array([[0.3, -0.4], [1.2, 0.1], [-0.5, 0.6]], np.float32)
    d = np.array([[-0.2, 0.5], [0.4, 0.9]], np.float32)
    pt = [R.softmax(r.astype(np.float64), 1.0) for r in t]
    pd = [R.softmax(r.astype(np.float64), 1.0) for r in d]
    x = np.stack([(rng.random(n) >= pd[i][0]).astype(np.int32) for i in range(2)], axis=1)
    u = _u24(rng, (n, 3))
    target = np.ascontiguousarray(np.broadcast_to(t, (n, 3, 2)))
    draft = np.ascontiguousarray(np.broadcast_to(d, (n, 2, 2)))
    return pt, pd, x, u, target, draft


def _outcome_counts(res, law):
    keys = sorted(law)
    idx = {k_: i for i, k_ in enumerate(keys)}
    counts = np.zeros(len(keys) + 1)
    for L, out in zip(res["accept_len"], res["out_tokens"]):
        key = (int(L), *[int(v) for v in out[:L + 1]])
        counts[idx.get(key, len(keys))] += 1
    return counts, np.array([law[k_] for k_ in keys] + [0.0])


def test_exact_outcome_law_v2_k2():
    n = 200000
    pt, pd, x, u, target, draft = _v2_k2_case(n)
    law = _exact_outcomes_v2_k2(pt, pd)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    res = oracle.verify_linear("stochastic", 1.0, target, draft, x, u, 2, F32)
    counts, probs = _outcome_counts(res, law)
    assert counts[-1] == 0, "an outcome outside the law"
    assert R.chi2_pvalue(counts[:-1], probs[:-1]) > 1e-4


@pytest.mark.parametrize("mut", [oracle.MUT_RESIDUAL_AS_TARGET, oracle.MUT_SWAPPED_RATIO, oracle.MUT_NO_BONUS])
def test_planted_mistakes_fail_the_exact_law(mut):
    n = 200000
    pt, pd, x, u, target, draft = _v2_k2_case(n)
    law = _exact_outcomes_v2_k2(pt, pd)
    with oracle.mutation(mut):
        res = oracle.verify_linear("stochastic", 1.0, target, draft, x, u, 2, F32)
    counts, probs = _outcome_counts(res, law)
    assert counts[-1] > 0 or R.chi2_pvalue(counts[:-1], probs[:-1]) < 1e-6


def _fixed_draft_case(n, seed=91):
    """Fixed logits and fixed draft tokens, fresh uniforms per trial: the accept
    events are independent with P(accept_i) = min(1, q_i)."""
    rng = np.random.default_rng(seed)
    V, k, T = 6, 4, 0.8
    t = rng.normal(0, 1.2, size=(k + 1, V)).astype(np.float32)
    d = (t[:k] + rng.normal(0, 1.0, size=(k, V))).astype(np.float32)
    # per position, the token whose ratio is closest to a spread of targets, so
    # that the accept probabilities differ (one of them is 1)
    ratios = [R.softmax(t[i].astype(np.float64), T) / R.softmax(d[i].astype(np.float64), T) for i in range(k)]
    x = np.array([int(np.argmin(np.abs(r - want))) for r, want in zip(ratios, (0.8, 0.5, 1.6, 0.3))], np.int32)
    q = np.array([ratios[i][x[i]] for i in range(k)])
    u = _u24(rng, (n, k + 1))
    target = np.ascontiguousarray(np.broadcast_to(t, (n, k + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(d, (n, k, V)))
    xs = np.ascontiguousarray(np.broadcast_to(x, (n, k)))
    return V, k, T, q, target, draft, xs, u


def _check_accept_length_law(res, q, n, k):
    L = res["accept_len"]
    a = np.minimum(1.0, q)
    for m in range(1, k + 1):
        p = float(np.prod(a[:m]))
        freq = float(np.mean(L >= m))
        se = np.sqrt(max(p * (1 - p), 1e-12) / n)
        if abs(freq - p) > 4 * se + 1e-12:
            return False
    mean = sum(float(np.prod(a[:m])) for m in range(1, k + 1))
    se = np.std(L) / np.sqrt(n)
    return abs(float(np.mean(L)) - mean) <= 4 * se + 1e-12


def test_accept_length_law():
    # P(L >= m) = prod_{i<m} min(1, q_i) for every m <= k, and E[L] = the sum of
    # those products
    n = 200000
    V, k, T, q, target, draft, xs, u = _fixed_draft_case(n)
    assert np.any(q < 0.9) and np.any(q > 0.2) and np.any(q > 1)
    res = oracle.verify_linear("stochastic", T, target, draft, xs, u, V, F32)
    assert _check_accept_length_law(res, q, n, k)


def test_planted_swapped_ratio_fails_the_accept_length_law():
    n = 200000
    V, k, T, q, target, draft, xs, u = _fixed_draft_case(n)
    with oracle.mutation(oracle.MUT_SWAPPED_RATIO):
        res = oracle.verify_linear("stochastic", T, target, draft, xs, u, V, F32)
    assert not _check_accept_length_law(res, q, n, k)
