"""Helpers for GPU parity tests: move generator outputs to the device, run the
library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import acceptance_row_softmax_amd as sv
import gen
import oracle

TIE_EPS = 1e-6
PROB_RTOL = 1e-5

# Running totals over every stochastic parity check in the session: an exception
# is a sequence or tree whose GPU result differs from the oracle's. Each one must
# be excused by a near tie in the oracle's arithmetic (an evaluated uniform within
# TIE_EPS of its threshold): a near tie in a draw that decides the accepted length
# excuses any difference, one in the final draw only a different final token.
# Exceptions must stay under 1e-4 of evaluated draws; the near-tie counts are
# reported beside them.
STATS = {"exceptions": 0, "evaluated": 0, "near_tie_sequences": 0, "near_tie_decision": 0,
         "near_tie_final_only": 0, "sequences": 0}


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: int):
    import torch
    return {gen.DT_F32: torch.float32, gen.DT_BF16: torch.bfloat16, gen.DT_F16: torch.float16}[dtype]


def to_dev(a: np.ndarray, dtype: int | None = None):
    """numpy -> cuda tensor; uint16 storage is reinterpreted as bf16 / fp16."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype is not None and dtype != gen.DT_F32:
        t = torch.from_numpy(a.view(np.int16)).cuda()
        return t.view(torch_dtype(dtype))
    return torch.from_numpy(a).cuda()


def run_linear(w: gen.LinearWorkload, **kw):
    import torch
    t = to_dev(w.target, w.dtype)
    d = to_dev(w.draft, w.dtype) if w.k > 0 else None
    tok = to_dev(w.draft_tokens.astype(np.int32)) if w.k > 0 else None
    u = to_dev(w.uniforms.astype(np.float32))
    res = sv.verify_linear(t, d, tok, u, mode=w.mode, temperature=w.temperature, **kw)
    torch.cuda.synchronize()
    return {k_: (v.cpu().numpy() if v is not None else None) for k_, v in res.items()}


def oracle_linear(w: gen.LinearWorkload, seqs=None):
    sl = slice(None) if seqs is None else seqs
    return oracle.verify_linear(w.mode, w.temperature, w.target[sl],
                                w.draft[sl] if w.mode == "stochastic" else None,
                                w.draft_tokens[sl], w.uniforms[sl], w.V, w.dtype, TIE_EPS)


def _record(differ, near, n_eval):
    near = np.asarray(near)
    STATS["exceptions"] += int(np.sum(differ))
    STATS["evaluated"] += int(np.sum(n_eval))
    STATS["near_tie_sequences"] += int(np.sum(near != 0))
    STATS["near_tie_decision"] += int(np.sum((near & oracle.NT_DECISION) != 0))
    STATS["near_tie_final_only"] += int(np.sum(near == oracle.NT_FINAL))
    STATS["sequences"] += int(len(near))


def _unexcused(diff_len_or_path, diff_final, near):
    """Sequences whose differences no near tie excuses: a different accepted
    length, path or accepted token needs a decision near tie; a different final
    token alone needs any near tie."""
    near = np.asarray(near)
    dec = (near & oracle.NT_DECISION) != 0
    return (diff_len_or_path & ~dec) | (diff_final & (near == 0))


def compare_linear(g, o, stochastic: bool, seqs=None):
    """Asserts parity; returns (exceptions, evaluated draws)."""
    sel = np.arange(len(o["accept_len"])) if seqs is None else np.asarray(seqs)
    acc_g = g["accept_len"][sel]
    out_g = g["out_tokens"][sel]
    np.testing.assert_array_equal(g["err_flags"][sel], o["err_flags"])
    L = o["accept_len"]
    col = np.arange(out_g.shape[1])[None, :]
    at_final = col == np.maximum(L, 0)[:, None]
    tok_diff = out_g != o["out_tokens"]
    diff_path = (acc_g != L) | np.any(tok_diff & ~at_final, axis=1)
    diff_final = np.any(tok_diff & at_final, axis=1)
    differ = diff_path | diff_final
    bad = np.nonzero(_unexcused(diff_path, diff_final, o["near_tie"]))[0]
    assert bad.size == 0, (f"{bad.size} sequences differ, first {bad[:5]}: gpu L={acc_g[bad[:5]]} "
                           f"oracle L={o['accept_len'][bad[:5]]} gpu out={out_g[bad[:3]]} "
                           f"oracle out={o['out_tokens'][bad[:3]]}")
    if not stochastic:
        assert not np.any(differ), "greedy results must match exactly"
    if stochastic:
        ok = o["err_flags"] == 0
        pt_o, pd_o = o["p_target"][ok], o["p_draft"][ok]
        pt_g, pd_g = g["p_target"][sel][ok].astype(np.float64), g["p_draft"][sel][ok].astype(np.float64)
        for name, a, b in (("p_target", pt_g, pt_o), ("p_draft", pd_g, pd_o)):
            rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-300)
            tiny = np.abs(b) < 1e-37          # below fp32's normal range
            assert np.all((rel <= PROB_RTOL) | tiny), (name, float(rel.max()))
        assert np.all(np.isnan(g["p_target"][sel][~ok]))
        _record(differ, o["near_tie"], o["n_eval"])
    return int(np.sum(differ)), int(np.sum(o["n_eval"]))


def run_tree(w: gen.TreeWorkload, max_depth=None, **kw):
    import torch
    md = w.max_depth if max_depth is None else max_depth
    par = to_dev(np.asarray(w.parent, np.int32))
    cand = to_dev(w.cand.astype(np.int32))
    lg = to_dev(w.logits, w.dtype)
    u = to_dev(w.uniforms.astype(np.float32))
    res = sv.verify_tree(par, cand, lg, u, md, mode=w.mode, temperature=w.temperature, **kw)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in res.items()}


def oracle_tree(w: gen.TreeWorkload, trees=None, max_depth=None):
    md = w.max_depth if max_depth is None else max_depth
    sl = slice(None) if trees is None else trees
    par = w.parent if np.asarray(w.parent).ndim == 1 else w.parent[sl]
    return oracle.verify_tree(w.mode, w.temperature, par, w.cand[sl], w.logits[sl],
                              w.uniforms[sl], w.V, w.dtype, md, TIE_EPS)


def compare_tree(g, o, trees=None):
    sel = np.arange(len(o["accept_len"])) if trees is None else np.asarray(trees)
    np.testing.assert_array_equal(g["err_flags"][sel], o["err_flags"])
    L = o["accept_len"]
    diff_path = (g["accept_len"][sel] != L) | np.any(g["path_nodes"][sel] != o["path_nodes"], axis=1)
    out_g = g["out_tokens"][sel]
    col = np.arange(out_g.shape[1])[None, :]
    at_final = col == np.maximum(L, 0)[:, None]
    tok_diff = out_g != o["out_tokens"]
    diff_path |= np.any(tok_diff & ~at_final, axis=1)
    diff_final = np.any(tok_diff & at_final, axis=1)
    differ = diff_path | diff_final
    bad = np.nonzero(_unexcused(diff_path, diff_final, o["near_tie"]))[0]
    assert bad.size == 0, (bad[:5], g["accept_len"][sel][bad[:3]], L[bad[:3]], out_g[bad[:3]],
                           o["out_tokens"][bad[:3]])
    if np.any(o["n_eval"] > 0):
        _record(differ, o["near_tie"], o["n_eval"])
    else:
        assert not np.any(differ), "greedy results must match exactly"
    return int(np.sum(differ)), int(np.sum(o["n_eval"]))
