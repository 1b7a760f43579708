"""Repeat-run byte identity: the same inputs give the same bytes in every output
(accepted lengths, tokens, path nodes, probabilities, error flags), for each
configuration and mode, with calls of another shape in between (the workspace is
shared and every record is tagged per call, so nothing of an earlier call may
leak into a later one)."""
import dataclasses

import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _same(a: dict, b: dict, what: str):
    assert a.keys() == b.keys(), what
    for key in a:
        if a[key] is None:
            assert b[key] is None, (what, key)
            continue
        x, y = np.ascontiguousarray(a[key]), np.ascontiguousarray(b[key])
        assert x.shape == y.shape and x.dtype == y.dtype, (what, key)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (what, key)


@pytest.mark.parametrize("cfg,mode", [("c1", "greedy"), ("c1", "stochastic"), ("c2", "greedy"),
                                      ("c3", "greedy"), ("c3", "stochastic")])
def test_linear_repeat(cfg, mode):
    w = {"c1": gen.c1_tiny, "c2": gen.c2_linear, "c3": gen.c3_mtp}[cfg](11, mode)
    other = gen.c2_linear(12, "stochastic", B=5)
    G.say(f"repeat: {cfg} {mode} B={w.B} k={w.k} V={w.V}")
    a = G.run_linear(w)
    G.run_linear(other)
    b = G.run_linear(w)
    _same(a, b, f"{cfg} {mode}")


@pytest.mark.parametrize("mode", ["greedy", "stochastic", "typical"])
def test_c4_repeat(mode):
    w = gen.c4_medusa_sparse(6, mode="greedy" if mode == "greedy" else "stochastic")
    kw = {"epsilon": 0.09, "delta": 0.3} if mode == "typical" else {}
    if mode == "typical":
        w = dataclasses.replace(w, mode="typical")
    other = gen.c4_medusa_sparse(7, mode="stochastic", B=3)
    G.say(f"repeat: c4 {mode}")
    a = G.run_tree(w, None, **kw)
    G.run_tree(other)
    b = G.run_tree(w, None, **kw)
    _same(a, b, f"c4 {mode}")


def test_c5_repeat_every_mode():
    base = gen.c5_medusa_full(2, mode="stochastic")
    for mode in ("greedy", "stochastic", "typical"):
        w = dataclasses.replace(base, mode=mode)
        kw = {"epsilon": 0.09, "delta": 0.3} if mode == "typical" else {}
        G.say(f"repeat: c5 {mode}")
        a = G.run_tree(w, None, **kw)
        b = G.run_tree(w, None, **kw)
        _same(a, b, f"c5 {mode}")


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_sampler_repeat(mode):
    import torch
    w = gen.c2_linear(13)
    rows = G.to_dev(w.draft.reshape(-1, w.V), w.dtype)
    u = G.to_dev(w.uniforms.reshape(-1)[: rows.shape[0]].astype(np.float32)) if mode == "stochastic" else None
    G.say(f"repeat: sampler {mode} rows={rows.shape[0]}")

    def run():
        r = sv.sample(rows, u, mode=mode, temperature=w.temperature)
        torch.cuda.synchronize()
        return {k_: v.cpu().numpy() for k_, v in r.items()}
    a = run()
    G.run_linear(gen.c2_linear(14, B=3))
    b = run()
    _same(a, b, f"sampler {mode}")
