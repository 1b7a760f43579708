"""GPU parity on random shapes: linear verification over random batch sizes, draft
lengths, vocabulary sizes (below, at and past chunk boundaries), dtypes, modes and
temperatures, and tree verification over random recursive trees (across the
256-node bound of the in-stream walk and the 4096-row bound of row waves) in
greedy, stochastic and typical modes. Seeded; every case against the oracle, to
the bar of the other parity tests."""
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
