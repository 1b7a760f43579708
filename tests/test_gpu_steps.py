"""GPU parity of the steps around verification against the oracle: commit
(bit-exact, and end to end: speculative greedy decoding through the GPU verify and
commit entry points equals plain greedy decoding), the sampler (bit-exact except
draws within 1e-6 of a bin edge, counted), and the tree mask (bit-exact)."""
import dataclasses

import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
import oracle
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _cpu(t):
    return t.cpu().numpy()


# ------------------------------------------------------------------ commit
@pytest.mark.parametrize("k", [0, 1, 4, 31])
def test_commit_matches_oracle(k):
    import torch
    rng = np.random.default_rng(200 + k)
    B, cap = 300, 64
    acc = rng.integers(0, k + 1, size=B).astype(np.int32)
    acc[::17] = -1                                     # failed verifications
    out = rng.integers(0, 1000, size=(B, k + 1)).astype(np.int32)
    drafts = rng.integers(0, 1000, size=(B, k)).astype(np.int32)
    ln = rng.integers(0, cap, size=B).astype(np.int32)
    ln[5::11] = cap                                     # full histories: no room left
    hist = rng.integers(0, 1000, size=(B, cap)).astype(np.int32)
    G.say(f"commit k={k} B={B}")
    d_ln, d_hist = G.to_dev(ln), G.to_dev(hist)
    r = sv.commit_linear(G.to_dev(acc), G.to_dev(out), G.to_dev(drafts) if k else None, d_ln, d_hist)
    torch.cuda.synchronize()
    o_ln, o_hist, o = oracle.commit_linear(acc, out, drafts if k else None, ln, hist)
    np.testing.assert_array_equal(_cpu(r["err_flags"]), o["err_flags"])
    np.testing.assert_array_equal(_cpu(d_ln), o_ln)
    np.testing.assert_array_equal(_cpu(d_hist), o_hist)
    np.testing.assert_array_equal(_cpu(r["shifted"]), o["shifted"])
    np.testing.assert_array_equal(_cpu(r["next_token"]), o["next_token"])
    assert np.any(o["err_flags"] == 16) and np.any(o["err_flags"] == 32) and np.any(o["err_flags"] == 0)


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_speculative_decoding_on_device(mode):
    """Rounds of draft (host, from a table) -> GPU verify -> GPU commit on a
    Markov-chain model. Greedy: the history equals plain greedy decoding of the
    target. Stochastic: it equals the oracle's verify + commit run on the same
    uniforms, round for round."""
    import torch
    rng = np.random.default_rng(31)
    V, k, B, n = 64, 4, 8, 48
    target = rng.normal(0, 2, size=(V, V))
    draft = target + rng.normal(0, 1.0, size=(V, V))
    cap = n + k + 2
    hist = np.full((B, cap), -1, np.int32)
    hist[:, 0] = np.arange(B) % V
    d_hist, d_ln = G.to_dev(hist), G.to_dev(np.ones(B, np.int32))
    o_hist, o_ln = hist.copy(), np.ones(B, np.int32)
    G.say(f"speculative decoding {mode} V={V} k={k} B={B}")
    for rnd in range(3 * n):
        ln = _cpu(d_ln)
        if ln.min() >= n + 1:
            break
        h = _cpu(d_hist)
        last = h[np.arange(B), ln - 1]
        drafts = np.empty((B, k), np.int32)
        cur = last.copy()
        for i in range(k):
            cur = np.argmax(draft[cur], axis=1).astype(np.int32)
            drafts[:, i] = cur
        inputs = np.concatenate([last[:, None], drafts], axis=1)
        tgt = np.ascontiguousarray(target[inputs].astype(np.float32))
        drf = np.ascontiguousarray(draft[inputs[:, :k]].astype(np.float32))
        u = gen.uniforms(gen.key(95, rnd, 1), B * (k + 1)).reshape(B, k + 1).astype(np.float32)
        g = sv.verify_linear(G.to_dev(tgt), G.to_dev(drf), G.to_dev(drafts), G.to_dev(u), mode=mode,
                             temperature=1.0)
        sv.commit_linear(g["accept_len"], g["out_tokens"], G.to_dev(drafts), d_ln, d_hist)
        torch.cuda.synchronize()
        if mode == "stochastic":
            o = oracle.verify_linear(mode, 1.0, tgt, drf, drafts, u, V, gen.DT_F32)
            assert not np.any(o["near_tie"]), "a draw at a bin edge: choose another seed"
            o_ln, o_hist, _ = oracle.commit_linear(o["accept_len"], o["out_tokens"], drafts, o_ln, o_hist)
            np.testing.assert_array_equal(_cpu(d_hist), o_hist)
    ln = _cpu(d_ln)
    assert ln.min() >= n + 1
    h = _cpu(d_hist)
    if mode == "greedy":
        for b in range(B):
            chain = [int(h[b, 0])]
            for _ in range(n):
                chain.append(int(np.argmax(target[chain[-1]])))
            np.testing.assert_array_equal(h[b, :n + 1], chain)


# ------------------------------------------------------------------ sampler
def _sample_check(x, V, dtype, mode, T, u):
    import torch
    g = sv.sample(G.to_dev(x, dtype), G.to_dev(u) if mode == "stochastic" else None, mode=mode,
                  temperature=T)
    torch.cuda.synchronize()
    o = oracle.sample(mode, T, x, u, V, dtype)
    gt = _cpu(g["tokens"])
    np.testing.assert_array_equal(_cpu(g["err_flags"]), o["err_flags"])
    differ = gt != o["tokens"]
    bad = differ & (o["near_tie"] == 0)
    assert not bad.any(), (np.nonzero(bad)[0][:5], gt[bad][:5], o["tokens"][bad][:5])
    if mode == "greedy":
        assert not differ.any()
    G._record(differ, o["near_tie"], np.full(len(gt), 1 if mode == "stochastic" else 0))
    return gt, o


def test_sampler_draft_rows_c2():
    # the draft rows of the draft-target workload: 32 sequences x 4 positions,
    # V = 128256 bf16, T = 0.7
    w = gen.c2_linear(0)
    x = np.ascontiguousarray(w.draft.reshape(-1, w.V))
    u = gen.uniforms(gen.key(96, 0, 1), x.shape[0]).astype(np.float32)
    G.say(f"sampler rows={x.shape[0]} V={w.V} bf16 T=0.7")
    _sample_check(x, w.V, w.dtype, "stochastic", 0.7, u)
    _sample_check(x, w.V, w.dtype, "greedy", 1.0, u)


@pytest.mark.parametrize("dtype", [gen.DT_F32, gen.DT_BF16, gen.DT_F16])
@pytest.mark.parametrize("V", [7, 1000, 20001, 65536])
def test_sampler_ragged(dtype, V):
    rows = 37
    x = gen.normal_pair(gen.key(97, V, dtype), 2.5, 0, 0.0, rows * V, dtype, want_b=False)[0].reshape(rows, V)
    u = gen.uniforms(gen.key(97, V, 9), rows).astype(np.float32)
    G.say(f"sampler ragged V={V} dtype={dtype}")
    for mode, T in (("stochastic", 0.8), ("greedy", 1.0)):
        _sample_check(x, V, dtype, mode, T, u)


def test_sampler_error_rows():
    V = 3000
    x = np.random.default_rng(5).normal(size=(4, V)).astype(np.float32)
    x[1] = -np.inf
    x[2, 17] = np.nan
    x[3, 5] = np.inf
    u = np.full(4, 0.5, np.float32)
    for mode in ("greedy", "stochastic"):
        gt, o = _sample_check(x, V, gen.DT_F32, mode, 1.0, u)
        assert gt[1] == -1


# ------------------------------------------------------------------ tree mask
def _unpack(mask, n):
    w = mask.view(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(*w.shape[:-1], -1)[..., :n].astype(np.uint8)


def test_tree_mask_cartesian():
    import torch
    parent, _ = gen.cartesian_tree([8, 8, 8, 8])
    G.say("tree mask cartesian 4681")
    r = sv.tree_mask(G.to_dev(parent))
    torch.cuda.synchronize()
    m = _unpack(_cpu(r["mask"])[0], len(parent))
    np.testing.assert_array_equal(m, oracle.tree_mask(parent))
    assert _cpu(r["err_flags"])[0] == 0


def test_tree_mask_per_tree_and_errors():
    import torch
    rng = np.random.default_rng(9)
    T, n = 6, 300
    par = np.stack([np.array([-1] + [int(rng.integers(max(0, i - 5), i)) for i in range(1, n)], np.int32)
                    for _ in range(T)])
    par[2] = np.arange(-1, n - 1)                # a chain: the causal mask
    par[4, 100] = 150                            # not an earlier node
    par[5, 0] = 0                                # root without parent -1
    G.say("tree mask per-tree")
    r = sv.tree_mask(G.to_dev(par))
    torch.cuda.synchronize()
    ef = _cpu(r["err_flags"])
    assert list(ef) == [0, 0, 0, 0, 4, 4]
    m = _unpack(_cpu(r["mask"]), n)
    for t in range(4):
        np.testing.assert_array_equal(m[t], oracle.tree_mask(par[t]))
    np.testing.assert_array_equal(m[2], np.tril(np.ones((n, n), np.uint8)))


def test_tree_mask_deep_chain_max_nodes():
    import torch
    n = sv.SV_MAX_TREE_NODES
    parent = np.arange(-1, n - 1, dtype=np.int32)
    G.say(f"tree mask chain n={n}")
    r = sv.tree_mask(G.to_dev(parent))
    torch.cuda.synchronize()
    w = _cpu(r["mask"])[0].view(np.uint32)
    # row i: bits 0..i set; check every row's word count and sampled rows in full
    W = (n + 31) // 32
    full = np.uint32(0xFFFFFFFF)
    for i in list(range(0, 70)) + list(range(n - 70, n)) + list(range(4000, 4100)):
        nw = i // 32
        assert np.all(w[i, :nw] == full)
        assert w[i, nw] == np.uint32((1 << (i % 32 + 1)) - 1 if i % 32 < 31 else 0xFFFFFFFF)
        assert np.all(w[i, nw + 1:W] == 0)
    assert _cpu(r["err_flags"])[0] == 0


# ------------------------------------------------------------------ verify + commit in one launch
@pytest.mark.parametrize("case", ["c2", "c3_stochastic", "small_k0", "small_greedy", "full_histories"])
def test_fused_commit_equals_verify_then_commit(case):
    import torch
    if case == "c2":
        w = gen.c2_linear(1)
    elif case == "c3_stochastic":
        w = gen.c3_mtp(1, "stochastic")     # 8192 (sequence, chunk) pairs: two chunks per residual wave
    elif case == "small_k0":
        w = gen.linear_draft_target(65, 0, 40, 0, 5000, gen.DT_F16, 2.0, 0.5, "stochastic", 0.9, "k0")
    else:
        w = gen.linear_draft_target(66, 0, 64, 3, 7001, gen.DT_BF16, 2.0, 0.5,
                                    "greedy" if case == "small_greedy" else "stochastic", 1.0, case)
    B, k = w.B, w.k
    rng = np.random.default_rng(7)
    cap = 40
    ln = rng.integers(0, cap - k - 1, size=B).astype(np.int32)
    if case == "full_histories":
        ln[::3] = cap                           # no room left: capacity errors
    hist = rng.integers(0, 1000, size=(B, cap)).astype(np.int32)
    G.say(f"fused commit {case} B={B} k={k}")
    t, d = G.to_dev(w.target, w.dtype), (G.to_dev(w.draft, w.dtype) if k else None)
    x = G.to_dev(w.draft_tokens.astype(np.int32)) if k else None
    u = G.to_dev(w.uniforms.astype(np.float32))
    # two launches
    l1, h1 = G.to_dev(ln), G.to_dev(hist)
    g = sv.verify_linear(t, d, x, u, mode=w.mode, temperature=w.temperature)
    c = sv.commit_linear(g["accept_len"], g["out_tokens"], x, l1, h1)
    # one launch
    l2, h2 = G.to_dev(ln), G.to_dev(hist)
    f = sv.verify_linear(t, d, x, u, mode=w.mode, temperature=w.temperature, seq_len=l2, history=h2)
    torch.cuda.synchronize()
    for key in ("accept_len", "out_tokens"):
        np.testing.assert_array_equal(_cpu(f[key]), _cpu(g[key]))
    np.testing.assert_array_equal(_cpu(l2), _cpu(l1))
    np.testing.assert_array_equal(_cpu(h2), _cpu(h1))
    np.testing.assert_array_equal(_cpu(f["shifted"]), _cpu(c["shifted"]))
    np.testing.assert_array_equal(_cpu(f["next_token"]), _cpu(c["next_token"]))
    # err_flags: the verification's bits, plus SV_ERR_CAPACITY where the commit found no room
    exp = _cpu(g["err_flags"]) | np.where(_cpu(c["err_flags"]) == sv.SV_ERR_CAPACITY, sv.SV_ERR_CAPACITY, 0)
    np.testing.assert_array_equal(_cpu(f["err_flags"]), exp)
    if case == "full_histories":
        assert np.any(_cpu(f["err_flags"]) == sv.SV_ERR_CAPACITY)


def test_one_workspace_serves_every_entry_point():
    """Every entry point leaves its workspace all zeros, so one workspace serves them
    all in any order (linear, linear + commit, trees greedy / eager / lazy / typical,
    sampler, row statistics)."""
    import torch
    L = sv.lib()
    wl = gen.c2_linear(11, B=6)
    ws_shape = [3, 3, 3, 3, 3, 3]                      # 1093 nodes x 4 trees: lazy draws
    parent, _ = gen.cartesian_tree(ws_shape)
    n, Bt, Vt = len(parent), 4, 3000
    x = gen.normal_pair(gen.key(67, 1, 1), 2.0, 0, 0.0, Bt * n * Vt, gen.DT_F16, want_b=False)[0].reshape(Bt, n, Vt)
    cand = np.random.default_rng(3).integers(0, Vt, size=(Bt, n)).astype(np.int32)
    ut = gen.uniforms(gen.key(67, 1, 2), Bt * n).reshape(Bt, n)
    tl = gen.TreeWorkload("ws-lazy", "stochastic", 1.0, Bt, n, Vt, gen.DT_F16, parent, cand, x, ut, 6)
    te = gen.c4_medusa_sparse(3, mode="stochastic", B=4)      # eager draws
    need = max(L.spec_verify_linear_workspace(wl.B, wl.k, wl.V, wl.dtype, sv.SV_STOCHASTIC),
               L.spec_verify_tree_workspace(Bt, n, Vt, gen.DT_F16, sv.SV_STOCHASTIC),
               L.spec_verify_tree_workspace(te.B, te.n_nodes, te.V, te.dtype, sv.SV_STOCHASTIC),
               L.spec_sample_workspace(wl.B * wl.k, wl.V, wl.dtype),
               L.spec_row_stats_workspace(wl.B * wl.k, wl.V, wl.dtype))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    t, d = G.to_dev(wl.target, wl.dtype), G.to_dev(wl.draft, wl.dtype)
    xd, u = G.to_dev(wl.draft_tokens.astype(np.int32)), G.to_dev(wl.uniforms.astype(np.float32))
    rows = G.to_dev(np.ascontiguousarray(wl.draft.reshape(-1, wl.V)), wl.dtype)
    ur = G.to_dev(gen.uniforms(gen.key(67, 2, 1), wl.B * wl.k).astype(np.float32))
    ln = G.to_dev(np.zeros(wl.B, np.int32))
    hist = G.to_dev(np.zeros((wl.B, 64), np.int32))
    calls = [
        ("linear", lambda: sv.verify_linear(t, d, xd, u, mode="stochastic", temperature=0.7, workspace=ws)),
        ("tree lazy", lambda: G.run_tree(tl, None, workspace=ws)),
        ("linear+commit", lambda: sv.verify_linear(t, d, xd, u, mode="stochastic", temperature=0.7,
                                                   seq_len=ln, history=hist, workspace=ws)),
        ("tree eager", lambda: G.run_tree(te, None, workspace=ws)),
        ("tree typical", lambda: G.run_tree(dataclasses.replace(tl, mode="typical"), None, epsilon=0.1,
                                            delta=0.3, workspace=ws)),
        ("sampler", lambda: sv.sample(rows, ur, mode="stochastic", temperature=0.7, workspace=ws)),
        ("tree greedy", lambda: G.run_tree(dataclasses.replace(te, mode="greedy"), None, workspace=ws)),
        ("row stats", lambda: sv.row_stats(rows, 0.7, workspace=ws)),
        ("linear again", lambda: sv.verify_linear(t, d, xd, u, mode="stochastic", temperature=0.7, workspace=ws)),
    ]
    for name, f in calls:
        G.say(f"shared workspace: {name}")
        f()
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, name
