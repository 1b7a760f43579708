"""The give-up path of the bounded waits between waves, forced from the host: with
the wait limit at zero (spec_set_wait_limit) every wait gives up after its second
unsuccessful poll, and every kernel still ends. A sequence whose outputs were
written either carries SV_ERR_INTERNAL with accept_len -1 and -1 tokens, or, if none
of its waits gave up, the oracle's result; a wait that gave up may also leave a
sequence unwritten. After the limit is restored and the workspace cleared, the same
call matches the oracle again."""
import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu

SENTINEL = -7
ERR_INTERNAL = 8


def _call(w, ws):
    import torch
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype) if (w.mode == "stochastic" and w.k > 0) else None
    x = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))
    dev = torch.device("cuda")
    out = {"accept_len": torch.full((w.B,), SENTINEL, dtype=torch.int32, device=dev),
           "out_tokens": torch.full((w.B, w.k + 1), SENTINEL, dtype=torch.int32, device=dev),
           "err_flags": torch.full((w.B,), SENTINEL, dtype=torch.int32, device=dev)}
    if w.mode == "stochastic":
        out["p_target"] = torch.zeros((w.B, w.k), dtype=torch.float32, device=dev)
        out["p_draft"] = torch.zeros((w.B, w.k), dtype=torch.float32, device=dev)
    res = sv.verify_linear(t, d, x, u, mode=w.mode, temperature=w.temperature, workspace=ws, out=out)
    torch.cuda.synchronize()
    return {k_: (v.cpu().numpy() if v is not None else None) for k_, v in res.items()}


@pytest.mark.parametrize("case", ["c2_hold", "c3_no_hold", "c3_greedy"])
def test_waits_give_up_and_recover(case):
    import torch
    w = {"c2_hold": lambda: gen.c2_linear(31),
         "c3_no_hold": lambda: gen.c3_mtp(32, "stochastic", B=128),
         "c3_greedy": lambda: gen.c3_mtp(33, "greedy", B=256)}[case]()
    L = sv.lib()
    need = L.spec_verify_linear_workspace(w.B, w.k, w.V, w.dtype,
                                          sv.SV_STOCHASTIC if w.mode == "stochastic" else sv.SV_GREEDY)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o = G.oracle_linear(w)
    G.say(f"give-up: {case} B={w.B} k={w.k} V={w.V} {w.mode}, wait limit 0")
    torch.cuda.synchronize()
    try:
        sv.set_wait_limit(0.0)
        g = _call(w, ws)
    finally:
        torch.cuda.synchronize()
        sv.set_wait_limit(0.25)
    ef, acc, tok = g["err_flags"], g["accept_len"], g["out_tokens"]
    written = ef != SENTINEL
    gave_up = written & ((ef & ERR_INTERNAL) != 0)
    assert np.all(acc[gave_up] == -1) and np.all(tok[gave_up] == -1)
    clean = written & (ef == 0)
    near = o["near_tie"] != 0
    same = (acc == o["accept_len"]) & np.all(tok == o["out_tokens"], axis=1)
    assert np.all(same[clean & ~near]), np.nonzero(clean & ~near & ~same)[0][:5]
    # unwritten sequences keep the sentinel everywhere
    assert np.all(acc[~written] == SENTINEL)
    if w.mode == "stochastic":
        # pair combines start before their rows have streamed: with no waiting
        # allowed some of their waits give up
        assert gave_up.any() or (~written).any()
    G.say(f"give-up: {case}: {int(gave_up.sum())} gave up, {int(clean.sum())} clean, {int((~written).sum())} unwritten")
    # restored limit, cleared workspace: the oracle's result again
    assert L.spec_workspace_clear(ws.data_ptr(), need, None) == 0
    torch.cuda.synchronize()
    g2 = _call(w, ws)
    G.compare_linear(g2, o, w.mode == "stochastic")
    assert np.all(g2["err_flags"] == 0)
