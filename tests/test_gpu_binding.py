"""The Python binding on the GPU: calls on a stream that is not the current one,
and shape checks that reject a mis-shaped tensor before anything is launched."""
import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_call_on_a_side_stream_matches_the_oracle():
    import torch
    w = gen.c2_linear(5, B=6)
    G.say("side stream: c2 law, B=6")
    side = torch.cuda.Stream()        # default priority
    t = G.to_dev(w.target, w.dtype)
    d = G.to_dev(w.draft, w.dtype)
    tok = G.to_dev(w.draft_tokens.astype(np.int32))
    u = G.to_dev(w.uniforms.astype(np.float32))
    side.wait_stream(torch.cuda.current_stream())     # inputs were copied on the current stream
    res = sv.verify_linear(t, d, tok, u, mode="stochastic", temperature=w.temperature, stream=side)
    side.synchronize()
    g = {k_: (v.cpu().numpy() if v is not None else None) for k_, v in res.items()}
    G.compare_linear(g, G.oracle_linear(w), True)
    # a second call with a larger shape grows the side stream's workspace on that stream
    w2 = gen.c2_linear(6, B=12)
    t2, d2 = G.to_dev(w2.target, w2.dtype), G.to_dev(w2.draft, w2.dtype)
    tok2, u2 = G.to_dev(w2.draft_tokens.astype(np.int32)), G.to_dev(w2.uniforms.astype(np.float32))
    side.wait_stream(torch.cuda.current_stream())
    res2 = sv.verify_linear(t2, d2, tok2, u2, mode="stochastic", temperature=w2.temperature, stream=side)
    side.synchronize()
    g2 = {k_: (v.cpu().numpy() if v is not None else None) for k_, v in res2.items()}
    G.compare_linear(g2, G.oracle_linear(w2), True)


def test_misshaped_tensors_are_rejected_before_launch():
    import torch
    dev = torch.device("cuda")
    i32 = torch.int32
    B, k, V = 4, 2, 300
    acc = torch.zeros(B, dtype=i32, device=dev)
    out = torch.zeros((B, k + 1), dtype=i32, device=dev)
    drafts = torch.zeros((B, k), dtype=i32, device=dev)
    ln = torch.zeros(B, dtype=i32, device=dev)
    hist = torch.zeros((B, 16), dtype=i32, device=dev)
    G.say("binding checks: commit_linear")
    with pytest.raises(ValueError):
        sv.commit_linear(acc, out, drafts, torch.zeros(B + 1, dtype=i32, device=dev), hist)
    with pytest.raises(ValueError):
        sv.commit_linear(acc, out, drafts, ln, torch.zeros((B - 1, 16), dtype=i32, device=dev))
    with pytest.raises(ValueError):
        sv.commit_linear(acc, torch.zeros((B + 2, k + 1), dtype=i32, device=dev), drafts, ln, hist)
    with pytest.raises(ValueError):
        sv.commit_linear(acc, out, torch.zeros((B, k + 1), dtype=i32, device=dev), ln, hist)
    with pytest.raises(ValueError):
        sv.commit_linear(acc, out, None, ln, hist)
    G.say("binding checks: verify_linear with commit")
    t = torch.zeros((B, k + 1, V), dtype=torch.bfloat16, device=dev)
    d = torch.zeros((B, k, V), dtype=torch.bfloat16, device=dev)
    u = torch.zeros((B, k + 1), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        sv.verify_linear(t, d, drafts, u, seq_len=torch.zeros(B + 1, dtype=i32, device=dev), history=hist)
    with pytest.raises(ValueError):
        sv.verify_linear(t, d, drafts, u, seq_len=ln, history=torch.zeros((2 * B, 16), dtype=i32, device=dev))
    with pytest.raises(ValueError):
        sv.verify_linear(t, d, drafts, u, out={"accept_len": acc, "out_tokens": out[:, :k]})
    G.say("binding checks: sample")
    x = torch.zeros((B, V), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        sv.sample(x, torch.zeros(B - 1, dtype=torch.float32, device=dev), mode="stochastic")
    with pytest.raises(ValueError):
        sv.sample(x, None, mode="stochastic")
    with pytest.raises(ValueError):
        sv.sample(x, None, mode="argmax")
    torch.cuda.synchronize()
