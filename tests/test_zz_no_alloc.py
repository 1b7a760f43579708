"""The entry point that allocates nothing (spec_verify_linear_static), through the
C ABI: its results equal those of spec_verify_linear with a caller workspace,
bit for bit, on two calls in a row, the second on a smaller batch; shapes beyond
its scratch array are refused on the host."""
import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
from tests import _gpu as G


def _inputs(w):
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype) if w.mode == "stochastic" else None
    tok = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))
    return t, d, tok, u


def _both(w):
    import torch
    t, d, tok, u = _inputs(w)
    ref = sv.verify_linear(t, d, tok, u, mode=w.mode, temperature=w.temperature)
    got = sv.verify_linear_static(t, d, tok, u, mode=w.mode, temperature=w.temperature)
    torch.cuda.synchronize()
    for key, v in ref.items():
        if v is None:
            continue
        a, b = v.cpu().numpy(), got[key].cpu().numpy()
        assert np.array_equal(a, b, equal_nan=True), key
    return {k_: (v.cpu().numpy() if v is not None else None) for k_, v in got.items()}


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_static_matches_workspace_entry_point(mode):
    w1 = gen.c2_linear(11, mode=mode, B=16)
    w2 = gen.c2_linear(12, mode=mode, B=5)
    G.say(f"static workspace: {mode}, B=16 then B=5")
    g1 = _both(w1)
    g2 = _both(w2)
    # and both against the oracle, to the usual bar
    G.compare_linear(g1, G.oracle_linear(w1), mode == "stochastic")
    G.compare_linear(g2, G.oracle_linear(w2), mode == "stochastic")


@pytest.mark.gpu
def test_static_c3_shape():
    w = gen.c3_mtp(3, "stochastic", B=64)
    G.say("static workspace: c3 law, B=64")
    G.compare_linear(_both(w), G.oracle_linear(w), True)


def test_static_rejects_shapes_beyond_its_array():
    import ctypes
    L = sv.lib()
    dummy = ctypes.c_void_p(0x1000)    # never dereferenced: the call is refused first
    B, k, V = 4096, 4, 1 << 20
    assert L.spec_verify_linear_workspace(B, k, V, sv.SV_BF16, sv.SV_STOCHASTIC) > sv.SV_MAX_STATIC_WORKSPACE
    st = L.spec_verify_linear_static(sv.SV_STOCHASTIC, 1.0, B, k, V, sv.SV_BF16, dummy, dummy, dummy, dummy,
                                     dummy, dummy, None, None, None, None)
    assert st == 5     # SV_ELIMIT
    assert L.spec_verify_linear_static(sv.SV_STOCHASTIC, 1.0, 2, 2, 100, 7, dummy, dummy, dummy, dummy,
                                       dummy, dummy, None, None, None, None) == 2   # SV_EDTYPE
