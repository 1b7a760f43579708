"""GPU parity on random shapes: linear verification over random batch sizes, draft
lengths, vocabulary sizes (below, at and past chunk boundaries), dtypes, modes and
temperatures; tree verification over random recursive trees (across the
256-node bound of the in-stream walk and the 4096-row bound of row waves) in
greedy, stochastic and typical modes; the sampler over random row counts and
vocabulary sizes; and tree masks of random trees up to 4681 nodes. Seeded; every
case against the oracle, to the bar of the other parity tests."""
import dataclasses

import numpy as np
import pytest

import gen
import oracle
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_random_linear_shapes():
    rng = np.random.default_rng(7)
    for c in range(60):
        mode = "stochastic" if rng.random() < 0.75 else "greedy"
        dtype = int(rng.choice([gen.DT_F32, gen.DT_BF16, gen.DT_F16]))
        k = int(rng.choice([0, 1, 1, 2, 3, 4, 5, 7, 9]))
        V = int(rng.choice([1, 7, 100, 4095, 4096, 4097, 8193, 20000, 32000, 50001, 70000]))
        bmax = max(1, min(600, int(20e6 // ((2 * k + 1) * V))))
        B = int(rng.integers(1, bmax + 1))
        T = float(rng.choice([0.5, 0.7, 1.0, 1.5]))
        sig_n = float(rng.choice([0.05, 0.3, 1.0, 3.0]))
        seed = int(rng.integers(0, 1 << 30))
        G.say(f"random linear {c}: mode={mode} dtype={dtype} B={B} k={k} V={V} T={T} sig_n={sig_n}")
        w = gen.linear_draft_target(300 + c, seed, B, k, V, dtype, 3.0, sig_n, mode, T, f"rand{c}")
        G.compare_linear(G.run_linear(w), G.oracle_linear(w), mode == "stochastic")


def test_random_trees():
    rng = np.random.default_rng(3)
    for c in range(40):
        mode = str(rng.choice(["greedy", "stochastic", "typical"]))
        dtype = int(rng.choice([gen.DT_F32, gen.DT_BF16, gen.DT_F16]))
        n = int(rng.choice([1, 2, 17, 65, 200, 256, 257, 600, 1500, 3000]))
        V = int(rng.choice([5, 100, 3000, 8193, 20001]))
        B = int(rng.integers(1, max(1, min(24, int(30e6 // (n * V)))) + 1))
        T = float(rng.choice([0.7, 1.0]))
        # parents mostly among the few nodes just before (deep trees), else anywhere earlier
        parent = np.array([-1] + [int(rng.integers(max(0, i - 1 - int(rng.integers(0, 8))), i))
                                  if rng.random() < 0.7 else int(rng.integers(0, i)) for i in range(1, n)],
                          np.int32)
        depth = np.zeros(n, np.int64)
        for i in range(1, n):
            depth[i] = depth[parent[i]] + 1
        md = int(depth.max()) + int(rng.integers(0, 2))
        dom = rng.integers(0, V, size=(B, n))
        x = rng.normal(0.0, 1.0, size=(B, n, V)).astype(np.float32)
        boost = float(rng.choice([0.0, 3.0, 20.0]))   # weight of one dominant token per row
        x[np.arange(B)[:, None], np.arange(n)[None, :], dom] += boost
        logits = gen.round_to(dtype, x)
        cand = np.where(rng.random((B, n)) < 0.7, dom[:, parent], rng.integers(0, V, (B, n))).astype(np.int32)
        cand[:, 0] = -1
        u = gen.uniforms(gen.key(400 + c, n, 1), B * n).reshape(B, n)
        G.say(f"random tree {c}: mode={mode} dtype={dtype} B={B} n={n} V={V} T={T} boost={boost} md={md}")
        w = gen.TreeWorkload(f"rand{c}", "greedy" if mode == "greedy" else "stochastic", T, B, n, V, dtype,
                             parent, cand, logits, u, md)
        if mode == "typical":
            eps, delta = float(rng.choice([0.09, 0.3])), float(rng.choice([0.3, 0.09]))
            g = G.run_tree(dataclasses.replace(w, mode="typical"), None, epsilon=eps, delta=delta)
            o = oracle.verify_tree_typical(T, eps, delta, parent, cand, logits, u, V, dtype, md, G.TIE_EPS)
        else:
            g = G.run_tree(w, None)
            o = G.oracle_tree(w)
        G.compare_tree(g, o)


def test_random_sampler_and_tree_mask_shapes():
    import torch
    import acceptance_row_softmax_amd as sv
    rng = np.random.default_rng(11)
    for c in range(30):
        mode = "stochastic" if rng.random() < 0.7 else "greedy"
        dtype = int(rng.choice([gen.DT_F32, gen.DT_BF16, gen.DT_F16]))
        V = int(rng.choice([1, 9, 4095, 4096, 4097, 20001, 70000]))
        rows = int(rng.integers(1, max(1, min(600, int(20e6 // V))) + 1))
        T = float(rng.choice([0.6, 1.0, 1.7]))
        G.say(f"random sampler {c}: mode={mode} dtype={dtype} rows={rows} V={V} T={T}")
        x = gen.normal_pair(gen.key(98, V, c), 2.5, 0, 0.0, rows * V, dtype, want_b=False)[0].reshape(rows, V)
        u = gen.uniforms(gen.key(98, V, 100 + c), rows).astype(np.float32)
        g = sv.sample(G.to_dev(x, dtype), G.to_dev(u) if mode == "stochastic" else None, mode=mode, temperature=T)
        torch.cuda.synchronize()
        o = oracle.sample(mode, T, x, u, V, dtype)
        gt = g["tokens"].cpu().numpy()
        np.testing.assert_array_equal(g["err_flags"].cpu().numpy(), o["err_flags"])
        differ = gt != o["tokens"]
        assert not (differ & (o["near_tie"] == 0)).any()
        if mode == "greedy":
            assert not differ.any()
        G._record(differ, o["near_tie"], np.full(rows, 1 if mode == "stochastic" else 0))
    for c in range(30):
        n = int(rng.choice([1, 2, 31, 32, 33, 64, 65, 300, 2000, 4681]))
        trees = int(rng.integers(1, 6))
        par = np.stack([np.array([-1] + [int(rng.integers(max(0, i - 1 - int(rng.integers(0, 6))), i))
                                         if rng.random() < 0.6 else int(rng.integers(0, i)) for i in range(1, n)],
                                 np.int32) for _ in range(trees)])
        G.say(f"random tree mask {c}: trees={trees} n={n}")
        r = sv.tree_mask(G.to_dev(par))
        torch.cuda.synchronize()
        assert not r["err_flags"].cpu().numpy().any()
        w = r["mask"].cpu().numpy().view(np.uint32)
        bits = ((w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(trees, n, -1)[..., :n]
        for t in range(trees):
            np.testing.assert_array_equal(bits[t].astype(np.uint8), oracle.tree_mask(par[t]))
