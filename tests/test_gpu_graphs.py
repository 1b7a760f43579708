"""Calls captured in a HIP graph and replayed: every replay must give the eager
call's outputs byte for byte. A replay reuses the captured call's tag, so this
checks that each call leaves its workspace as it found it (records cleared by
their last reader, counters by the wave that completes them). Between replays the
program does eager work of its own (another call, on another workspace) and
synchronises."""
import dataclasses

import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _host(d):
    return {k_: np.ascontiguousarray(v.cpu().numpy()) for k_, v in d.items() if v is not None}


def _same(a, b, what):
    assert a.keys() == b.keys(), what
    for k_ in a:
        assert a[k_].shape == b[k_].shape, (what, k_)
        assert np.array_equal(a[k_].view(np.uint8), b[k_].view(np.uint8)), (what, k_)


def _linear_case(w):
    import torch
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype) if (w.mode == "stochastic" and w.k > 0) else None
    x = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))
    L = sv.lib()
    need = L.spec_verify_linear_workspace(w.B, w.k, w.V, w.dtype,
                                          sv.SV_STOCHASTIC if w.mode == "stochastic" else sv.SV_GREEDY)

    def make():
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        dev = torch.device("cuda")
        out = {"accept_len": torch.empty(w.B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((w.B, w.k + 1), dtype=torch.int32, device=dev),
               "err_flags": torch.empty(w.B, dtype=torch.int32, device=dev)}
        if w.mode == "stochastic":
            out["p_target"] = torch.empty((w.B, w.k), dtype=torch.float32, device=dev)
            out["p_draft"] = torch.empty((w.B, w.k), dtype=torch.float32, device=dev)

        def run():
            return sv.verify_linear(t, d, x, u, mode=w.mode, temperature=w.temperature, workspace=ws, out=out)
        return run
    return make


def _static_case(w):
    import torch
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype)
    x = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))

    def make():
        dev = torch.device("cuda")
        out = {"accept_len": torch.empty(w.B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((w.B, w.k + 1), dtype=torch.int32, device=dev),
               "err_flags": torch.empty(w.B, dtype=torch.int32, device=dev),
               "p_target": torch.empty((w.B, w.k), dtype=torch.float32, device=dev),
               "p_draft": torch.empty((w.B, w.k), dtype=torch.float32, device=dev)}

        def run():
            return sv.verify_linear_static(t, d, x, u, mode=w.mode, temperature=w.temperature, out=out)
        return run
    return make


def _tree_case(w, **kw):
    import torch
    par = G.to_dev(np.asarray(w.parent, np.int32))
    cand = G.to_dev(w.cand.astype(np.int32))
    lg = G.to_dev(w.logits, w.dtype)
    u = G.to_dev(w.uniforms.astype(np.float32))
    L = sv.lib()
    need = L.spec_verify_tree_workspace(w.B, w.n_nodes, w.V, w.dtype,
                                        sv.SV_GREEDY if w.mode == "greedy" else sv.SV_STOCHASTIC)

    def make():
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

        def run():
            return sv.verify_tree(par, cand, lg, u, w.max_depth, mode=w.mode, temperature=w.temperature,
                                  workspace=ws, **kw)
        return run
    return make


def _sample_case(mode):
    import torch
    w = gen.c2_linear(45)
    rows = G.to_dev(w.draft.reshape(-1, w.V), w.dtype)
    u = G.to_dev(w.uniforms.reshape(-1)[: rows.shape[0]].astype(np.float32)) if mode == "stochastic" else None
    L = sv.lib()
    need = L.spec_sample_workspace(rows.shape[0], w.V, w.dtype)

    def make():
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

        def run():
            return sv.sample(rows, u, mode=mode, temperature=w.temperature, workspace=ws)
        return run
    return make


def _cases():
    c4 = gen.c4_medusa_sparse(46, mode="stochastic")
    return {
        "c2_stochastic": lambda: _linear_case(gen.c2_linear(41)),
        "c3_stochastic_no_hold": lambda: _linear_case(gen.c3_mtp(42, "stochastic", B=128)),
        "c3_greedy": lambda: _linear_case(gen.c3_mtp(43, "greedy", B=64)),
        "c2_static": lambda: _static_case(gen.c2_linear(44, B=8)),
        "c4_greedy": lambda: _tree_case(dataclasses.replace(c4, mode="greedy")),
        "c4_stochastic": lambda: _tree_case(c4),
        "c4_typical": lambda: _tree_case(dataclasses.replace(c4, mode="typical"), epsilon=0.09, delta=0.3),
        "sample_stochastic": lambda: _sample_case("stochastic"),
    }


@pytest.mark.parametrize("case", list(_cases().keys()))
def test_graph_replays_match_eager(case):
    import torch
    make = _cases()[case]()
    G.say(f"graph replays: {case}")
    eager_run = make()
    ref = _host(eager_run())
    torch.cuda.synchronize()
    # other eager work between the replays, on its own workspace
    other = _linear_case(gen.c2_linear(47, B=3))()
    run = make()
    run()   # one eager call of the captured instance first (its buffers, the library's setup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        _same(_host(outs), ref, f"{case} replay {r}")
        other()
        torch.cuda.synchronize()
    # and eager again after the replays, on the captured instance's workspace
    _same(_host(run()), ref, f"{case} eager after replays")
