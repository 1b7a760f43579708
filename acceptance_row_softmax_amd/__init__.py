"""Python binding of libspecverify (speculative-decoding verification on MI355X).

Argument marshalling only: every step of the verification runs in the HIP
kernels of ``libspecverify.so``; PyTorch supplies device buffers and the
current stream. There is no fallback: if the library is missing this module
raises on first use.

Entry points mirror the C ABI in ``include/specverify.h``:

* :func:`verify_linear` -- longest acceptable draft prefix + one target token
  ("Accelerating Sonar through speculation", sections "Spekulatives Decoding"
  and "Ziel-Entwurf").
* :func:`verify_tree` -- candidate-tree walk ("Speculative-Decoding, LLM推理的加速 /
  Medusa 方法阅读", section 三).
* :func:`row_stats` -- per-row max, log-sum-exp and argmax at a temperature.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from . import _build

SV_GREEDY, SV_STOCHASTIC = 0, 1
SV_F32, SV_BF16, SV_F16 = 0, 1, 2
SV_ERR_TOKEN, SV_ERR_ROW, SV_ERR_TREE, SV_ERR_INTERNAL = 1, 2, 4, 8
SV_ERR_CAPACITY, SV_ERR_UNVERIFIED = 16, 32
SV_MAX_K, SV_MAX_TREE_NODES, SV_MAX_ROW_BYTES = 31, 16384, 2097152

LIB_PATH = _build.LIB
_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libspecverify.so not found at {LIB_PATH}; run "
                               "acceptance_row_softmax_amd._build.build() (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, sz, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
        L.spec_verify_status_string.restype = ctypes.c_char_p
        L.spec_verify_status_string.argtypes = [i32]
        L.spec_verify_linear_workspace.restype = sz
        L.spec_verify_linear_workspace.argtypes = [i64, i64, i64, i32, i32]
        L.spec_verify_linear.restype = i32
        L.spec_verify_linear.argtypes = [i32, f32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp]
        L.spec_verify_tree_workspace.restype = sz
        L.spec_verify_tree_workspace.argtypes = [i64, i64, i64, i32, i32]
        L.spec_verify_tree.restype = i32
        L.spec_verify_tree.argtypes = [i32, f32, i64, i64, i64, i32, vp, i64, vp, vp, vp, i64, vp, vp,
                                       vp, vp, vp, sz, vp]
        L.spec_row_stats_workspace.restype = sz
        L.spec_row_stats_workspace.argtypes = [i64, i64, i32]
        L.spec_row_stats.restype = i32
        L.spec_row_stats.argtypes = [i32, f32, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.spec_workspace_clear.restype = i32
        L.spec_workspace_clear.argtypes = [vp, sz, vp]
        L.spec_set_wait_limit.restype = i32
        L.spec_set_wait_limit.argtypes = [ctypes.c_double]
        L.spec_verify_tree_typical.restype = i32
        L.spec_verify_tree_typical.argtypes = [f32, ctypes.c_double, ctypes.c_double, i64, i64, i64, i32, vp,
                                               i64, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]
        L.spec_verify_linear_commit.restype = i32
        L.spec_verify_linear_commit.argtypes = [i32, f32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, i64, vp, vp, vp, sz, vp]
        L.spec_commit_linear.restype = i32
        L.spec_commit_linear.argtypes = [i64, i64, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
        L.spec_sample_workspace.restype = sz
        L.spec_sample_workspace.argtypes = [i64, i64, i32]
        L.spec_sample.restype = i32
        L.spec_sample.argtypes = [i32, f32, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp]
        L.spec_tree_mask.restype = i32
        L.spec_tree_mask.argtypes = [i64, i64, vp, i64, vp, vp, vp]
        L.spec_verify_linear_static.restype = i32
        L.spec_verify_linear_static.argtypes = [i32, f32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp]
        L.spec_tree_build_greedy.restype = i64
        L.spec_tree_build_greedy.argtypes = [i64, i64, vp, i64, vp, vp, vp, vp]
        L.spec_read_probe.restype = i32
        L.spec_read_probe.argtypes = [vp, sz, vp, sz, vp, sz, vp]
        _lib = L
    return _lib


EXPORTED = ("spec_verify_linear_workspace", "spec_verify_linear", "spec_verify_tree_workspace",
            "spec_verify_tree", "spec_row_stats_workspace", "spec_row_stats",
            "spec_workspace_clear", "spec_verify_status_string", "spec_commit_linear",
            "spec_sample_workspace", "spec_sample", "spec_tree_mask", "spec_tree_build_greedy",
            "spec_verify_tree_typical", "spec_verify_linear_commit", "spec_verify_linear_static",
            "spec_set_wait_limit", "spec_read_probe")
SV_MAX_STATIC_WORKSPACE = 8 * 1024 * 1024


def status_string(status: int) -> str:
    return lib().spec_verify_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise SpecVerifyError(status, where)


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def sv_dtype(t) -> int:
    torch = _torch()
    m = {torch.float32: SV_F32, torch.bfloat16: SV_BF16, torch.float16: SV_F16}
    if t.dtype not in m:
        raise TypeError(f"logits dtype {t.dtype} not supported (float32, bfloat16, float16)")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _need(t, name, dtype=None, device=None):
    torch = _torch()
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _torch_stream(stream=None):
    """The torch stream a call runs on: `stream`, else the current stream."""
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


def _stream(stream=None):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


class Workspace:
    """One zero-filled device workspace per (device, stream), grown on demand.
    Every call that completes leaves it all zeros, so it serves every entry point
    and shape; calls on one stream never overlap, calls on two streams get two.
    A buffer is allocated and zero-filled on the stream of the calls that use it,
    so the fill is ordered before them and the allocator reuses a replaced buffer
    only after that stream has passed it."""

    def __init__(self):
        self._bufs = {}

    def get(self, device, stream, nbytes: int):
        torch = _torch()
        k = (str(device), stream.cuda_stream)
        buf = self._bufs.get(k)
        if buf is None or buf.numel() < nbytes:
            with torch.cuda.stream(stream):
                buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._bufs[k] = buf
        return buf


_WS = Workspace()


def _check_out(out, shapes, dev):
    """Preallocated outputs: each present tensor must be contiguous, on `dev` and of
    its shape (int32, or float32 for the probabilities)."""
    torch = _torch()
    for name, shape in shapes.items():
        t = out.get(name)
        if t is None:
            continue
        want = torch.float32 if name in ("p_target", "p_draft") else torch.int32
        _need(t, name, want, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"out[{name!r}] must have shape {shape}, got {tuple(t.shape)}")
    for name in ("accept_len", "out_tokens"):
        if out.get(name) is None:
            raise ValueError(f"out must hold {name!r}")


def verify_linear(target, draft, draft_tokens, uniforms, mode: str = "stochastic",
                  temperature: float = 1.0, *, with_probs: bool = True, err_flags: bool = True,
                  seq_len=None, history=None, shifted: bool = True, workspace=None, stream=None, out=None):
    """Verify B linear drafts of k tokens.

    target [B][k+1][V], draft [B][k][V] (same dtype; draft unused in greedy mode),
    draft_tokens [B][k] int32, uniforms [B][k+1] float32 (stochastic only).
    Returns a dict of device tensors: accept_len [B], out_tokens [B][k+1],
    p_target / p_draft [B][k] (stochastic, if with_probs), err_flags [B].
    ``out`` may hold preallocated tensors of those names and shapes.
    With ``seq_len`` [B] int32 (and optionally ``history`` [B][capacity] int32) the
    same launch also commits the result in place (spec_verify_linear_commit) and
    the dict gains "shifted" [B][k+1] (if ``shifted``) and "next_token" [B].
    """
    torch = _torch()
    stoch = mode == "stochastic"
    if mode not in ("stochastic", "greedy"):
        raise ValueError("mode must be 'greedy' or 'stochastic'")
    _need(target, "target")
    dev = target.device
    if target.dim() != 3:
        raise ValueError("target must be [B][k+1][V]")
    B, k1, V = target.shape
    k = k1 - 1
    dt = sv_dtype(target)
    if stoch and k > 0:
        _need(draft, "draft", target.dtype, dev)
        if tuple(draft.shape) != (B, k, V):
            raise ValueError("draft must be [B][k][V]")
    else:
        draft = None
    if k > 0:
        _need(draft_tokens, "draft_tokens", torch.int32, dev)
        if tuple(draft_tokens.shape) != (B, k):
            raise ValueError("draft_tokens must be [B][k]")
    else:
        draft_tokens = None
    if stoch:
        _need(uniforms, "uniforms", torch.float32, dev)
        if tuple(uniforms.shape) != (B, k + 1):
            raise ValueError("uniforms must be [B][k+1]")
    else:
        uniforms = None
    ts = _torch_stream(stream)
    if seq_len is not None:
        _need(seq_len, "seq_len", torch.int32, dev)
        if tuple(seq_len.shape) != (B,):
            raise ValueError("seq_len must be [B]")
        cap = 0
        if history is not None:
            _need(history, "history", torch.int32, dev)
            if history.dim() != 2 or history.shape[0] != B:
                raise ValueError("history must be [B][capacity]")
            cap = history.shape[-1]
    if out is None:
        with torch.cuda.stream(ts):
            out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
                   "out_tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                   "err_flags": torch.empty(B, dtype=torch.int32, device=dev) if err_flags else None}
            if stoch and with_probs:
                out["p_target"] = torch.empty((B, k), dtype=torch.float32, device=dev)
                out["p_draft"] = torch.empty((B, k), dtype=torch.float32, device=dev)
    else:
        _check_out(out, {"accept_len": (B,), "out_tokens": (B, k + 1), "err_flags": (B,), "p_target": (B, k),
                         "p_draft": (B, k), "shifted": (B, k + 1), "next_token": (B,)}, dev)
    L = lib()
    mcode = SV_STOCHASTIC if stoch else SV_GREEDY
    nbytes = L.spec_verify_linear_workspace(B, k, V, dt, mcode)
    s = ctypes.c_void_p(ts.cuda_stream)
    ws = workspace if workspace is not None else _WS.get(dev, ts, nbytes)
    if seq_len is not None:
        with torch.cuda.stream(ts):
            if shifted and "shifted" not in out:
                out["shifted"] = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
            if "next_token" not in out:
                out["next_token"] = torch.empty(B, dtype=torch.int32, device=dev)
        st = L.spec_verify_linear_commit(
            mcode, float(temperature), B, k, V, dt, _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
            _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("p_target")), _ptr(out.get("p_draft")),
            _ptr(out.get("err_flags")), _ptr(seq_len), _ptr(history), cap, _ptr(out.get("shifted")),
            _ptr(out["next_token"]), _ptr(ws), ws.numel(), s)
        _check(st, "spec_verify_linear_commit")
        return out
    st = L.spec_verify_linear(mcode, float(temperature), B, k, V, dt, _ptr(target), _ptr(draft), _ptr(draft_tokens),
            _ptr(uniforms), _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("p_target")),
            _ptr(out.get("p_draft")), _ptr(out.get("err_flags")), _ptr(ws), ws.numel(), s)
    _check(st, "spec_verify_linear")
    return out


def verify_linear_static(target, draft, draft_tokens, uniforms, mode: str = "stochastic",
                         temperature: float = 1.0, *, with_probs: bool = True, stream=None, out=None):
    """verify_linear through spec_verify_linear_static: the library's own per-GPU
    scratch array instead of a workspace (no device allocation by the library; the
    outputs are allocated here unless ``out`` holds them). Calls that overlap on one
    GPU race."""
    torch = _torch()
    stoch = mode == "stochastic"
    if mode not in ("stochastic", "greedy"):
        raise ValueError("mode must be 'greedy' or 'stochastic'")
    _need(target, "target")
    dev = target.device
    if target.dim() != 3:
        raise ValueError("target must be [B][k+1][V]")
    B, k1, V = target.shape
    k = k1 - 1
    dt = sv_dtype(target)
    if stoch and k > 0:
        _need(draft, "draft", target.dtype, dev)
        if tuple(draft.shape) != (B, k, V):
            raise ValueError("draft must be [B][k][V]")
    else:
        draft = None
    if k > 0:
        _need(draft_tokens, "draft_tokens", torch.int32, dev)
        if tuple(draft_tokens.shape) != (B, k):
            raise ValueError("draft_tokens must be [B][k]")
    else:
        draft_tokens = None
    if stoch:
        _need(uniforms, "uniforms", torch.float32, dev)
        if tuple(uniforms.shape) != (B, k + 1):
            raise ValueError("uniforms must be [B][k+1]")
    else:
        uniforms = None
    ts = _torch_stream(stream)
    if out is None:
        with torch.cuda.stream(ts):
            out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
                   "out_tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                   "err_flags": torch.empty(B, dtype=torch.int32, device=dev)}
            if stoch and with_probs:
                out["p_target"] = torch.empty((B, k), dtype=torch.float32, device=dev)
                out["p_draft"] = torch.empty((B, k), dtype=torch.float32, device=dev)
    else:
        _check_out(out, {"accept_len": (B,), "out_tokens": (B, k + 1), "err_flags": (B,), "p_target": (B, k),
                         "p_draft": (B, k)}, dev)
    st = lib().spec_verify_linear_static(
        SV_STOCHASTIC if stoch else SV_GREEDY, float(temperature), B, k, V, dt, _ptr(target), _ptr(draft),
        _ptr(draft_tokens), _ptr(uniforms), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out.get("p_target")), _ptr(out.get("p_draft")), _ptr(out.get("err_flags")),
        ctypes.c_void_p(ts.cuda_stream))
    _check(st, "spec_verify_linear_static")
    return out


def verify_tree(parent, cand_tokens, logits, uniforms, max_depth: int, mode: str = "greedy",
                temperature: float = 1.0, *, epsilon: float = None, delta: float = None, workspace=None,
                stream=None):
    """Verify B candidate trees of n_nodes (node 0 = root).

    parent [n_nodes] (shared) or [B][n_nodes] int32, cand_tokens [B][n_nodes] int32,
    logits [B][n_nodes][V], uniforms [B][n_nodes] float32 (stochastic and typical).
    mode "greedy", "stochastic" (spec_verify_tree) or "typical" (typical acceptance,
    spec_verify_tree_typical; epsilon and delta required).
    Returns accept_len [B], path_nodes [B][max_depth], out_tokens [B][max_depth+1],
    err_flags [B].
    """
    torch = _torch()
    typical = mode == "typical"
    stoch = mode == "stochastic" or typical
    if mode not in ("stochastic", "greedy", "typical"):
        raise ValueError("mode must be 'greedy', 'stochastic' or 'typical'")
    if typical and (epsilon is None or delta is None):
        raise ValueError("typical acceptance needs epsilon and delta")
    _need(logits, "logits")
    dev = logits.device
    B, N, V = logits.shape
    dt = sv_dtype(logits)
    _need(parent, "parent", torch.int32, dev)
    if parent.dim() == 1:
        if parent.shape[0] != N:
            raise ValueError("parent must have n_nodes entries")
        stride = 0
    else:
        if tuple(parent.shape) != (B, N):
            raise ValueError("parent must be [n_nodes] or [B][n_nodes]")
        stride = N
    _need(cand_tokens, "cand_tokens", torch.int32, dev)
    if tuple(cand_tokens.shape) != (B, N):
        raise ValueError("cand_tokens must be [B][n_nodes]")
    if stoch:
        _need(uniforms, "uniforms", torch.float32, dev)
        if tuple(uniforms.shape) != (B, N):
            raise ValueError("uniforms must be [B][n_nodes]")
    else:
        uniforms = None
    if int(max_depth) < 0:
        raise ValueError("max_depth must be >= 0")
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        path = torch.empty((B, max_depth), dtype=torch.int32, device=dev)
        out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
        ef = torch.empty(B, dtype=torch.int32, device=dev)
    L = lib()
    mcode = SV_STOCHASTIC if stoch else SV_GREEDY
    nbytes = L.spec_verify_tree_workspace(B, N, V, dt, mcode)
    s = ctypes.c_void_p(ts.cuda_stream)
    ws = workspace if workspace is not None else _WS.get(dev, ts, nbytes)
    if typical:
        st = L.spec_verify_tree_typical(float(temperature), float(epsilon), float(delta), B, N, V, dt,
                                        _ptr(parent), stride, _ptr(cand_tokens), _ptr(logits),
                                        _ptr(uniforms), int(max_depth), _ptr(acc),
                                        _ptr(path) if max_depth > 0 else None, _ptr(out), _ptr(ef),
                                        _ptr(ws), ws.numel(), s)
        _check(st, "spec_verify_tree_typical")
        return {"accept_len": acc, "path_nodes": path, "out_tokens": out, "err_flags": ef}
    st = L.spec_verify_tree(mcode, float(temperature), B, N, V, dt, _ptr(parent), stride,
                            _ptr(cand_tokens), _ptr(logits), _ptr(uniforms), int(max_depth),
                            _ptr(acc), _ptr(path) if max_depth > 0 else None, _ptr(out), _ptr(ef),
                            _ptr(ws), ws.numel(), s)
    _check(st, "spec_verify_tree")
    return {"accept_len": acc, "path_nodes": path, "out_tokens": out, "err_flags": ef}


def row_stats(x, temperature: float = 1.0, *, workspace=None, stream=None):
    """Per-row max, log-sum-exp at temperature T, argmax and error bits of x [rows][V]."""
    torch = _torch()
    _need(x, "x")
    dev = x.device
    V = x.shape[-1]
    rows = x.numel() // V
    dt = sv_dtype(x)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        m = torch.empty(rows, dtype=torch.float32, device=dev)
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
        am = torch.empty(rows, dtype=torch.int32, device=dev)
        ef = torch.empty(rows, dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.spec_row_stats_workspace(rows, V, dt)
    s = ctypes.c_void_p(ts.cuda_stream)
    ws = workspace if workspace is not None else _WS.get(dev, ts, nbytes)
    st = L.spec_row_stats(dt, float(temperature), rows, V, _ptr(x), _ptr(m), _ptr(lse), _ptr(am),
                          _ptr(ef), _ptr(ws), ws.numel(), s)
    _check(st, "spec_row_stats")
    return {"max": m, "lse": lse, "argmax": am, "err_flags": ef}


def commit_linear(accept_len, out_tokens, draft_tokens, seq_len, history=None, *, shifted: bool = True,
                  stream=None):
    """Applies a verification's outcome in place (seq_len, history) and returns
    {"shifted", "next_token", "err_flags"} (spec_commit_linear)."""
    torch = _torch()
    i32 = torch.int32
    _need(accept_len, "accept_len", i32)
    dev = accept_len.device
    _need(out_tokens, "out_tokens", i32, dev)
    _need(seq_len, "seq_len", i32, dev)
    if accept_len.dim() != 1:
        raise ValueError("accept_len must be [B]")
    B = accept_len.shape[0]
    if out_tokens.dim() != 2 or out_tokens.shape[0] != B or out_tokens.shape[1] < 1:
        raise ValueError("out_tokens must be [B][k+1]")
    k = out_tokens.shape[-1] - 1
    if tuple(seq_len.shape) != (B,):
        raise ValueError("seq_len must be [B]")
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", i32, dev)
        if tuple(draft_tokens.shape) != (B, k):
            raise ValueError("draft_tokens must be [B][k]")
    elif shifted and k > 0:
        raise ValueError("the shifted row needs draft_tokens [B][k]")
    cap = 0
    if history is not None:
        _need(history, "history", i32, dev)
        if history.dim() != 2 or history.shape[0] != B:
            raise ValueError("history must be [B][capacity]")
        cap = history.shape[-1]
    with torch.cuda.stream(_torch_stream(stream)):
        sh = torch.empty((B, k + 1), dtype=i32, device=dev) if shifted else None
        nxt = torch.empty(B, dtype=i32, device=dev)
        ef = torch.empty(B, dtype=i32, device=dev)
    st = lib().spec_commit_linear(B, k, _ptr(accept_len), _ptr(out_tokens), _ptr(draft_tokens),
                                  _ptr(seq_len), _ptr(history), cap, _ptr(sh), _ptr(nxt), _ptr(ef),
                                  _stream(stream))
    _check(st, "spec_commit_linear")
    return {"shifted": sh, "next_token": nxt, "err_flags": ef}


def sample(logits, uniforms=None, mode: str = "stochastic", temperature: float = 1.0, *, workspace=None,
           stream=None):
    """One token per row of logits [..., V] (spec_sample); returns {"tokens", "err_flags"}."""
    torch = _torch()
    if mode not in ("stochastic", "greedy"):
        raise ValueError("mode must be 'greedy' or 'stochastic'")
    _need(logits, "logits")
    dev = logits.device
    V = logits.shape[-1]
    rows = logits.numel() // V
    m = SV_STOCHASTIC if mode == "stochastic" else SV_GREEDY
    if m == SV_STOCHASTIC:
        if uniforms is None:
            raise ValueError("stochastic sampling needs uniforms")
        _need(uniforms, "uniforms", torch.float32, dev)
        if uniforms.numel() != rows:
            raise ValueError(f"uniforms must hold one value per row ({rows}), got {uniforms.numel()}")
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        tok = torch.empty(rows, dtype=torch.int32, device=dev)
        ef = torch.empty(rows, dtype=torch.int32, device=dev)
    L = lib()
    dt = sv_dtype(logits)
    nbytes = L.spec_sample_workspace(rows, V, dt)
    s = ctypes.c_void_p(ts.cuda_stream)
    ws = workspace if workspace is not None else _WS.get(dev, ts, nbytes)
    st = L.spec_sample(m, float(temperature), rows, V, dt, _ptr(logits),
                       _ptr(uniforms) if m == SV_STOCHASTIC else None, _ptr(tok), _ptr(ef), _ptr(ws),
                       ws.numel(), s)
    _check(st, "spec_sample")
    return {"tokens": tok, "err_flags": ef}


def tree_mask(parent, n_trees: int = 1, *, stream=None):
    """Ancestor-or-self bitmaps [n_trees][n][ceil(n/32)] uint32 (as int32 storage) of
    parent arrays [n] (shared) or [n_trees][n] (spec_tree_mask)."""
    torch = _torch()
    _need(parent, "parent", torch.int32)
    dev = parent.device
    if parent.dim() not in (1, 2):
        raise ValueError("parent must be [n] or [n_trees][n]")
    n = parent.shape[-1]
    stride = 0 if parent.dim() == 1 else n
    if parent.dim() > 1:
        n_trees = parent.shape[0]
    if n_trees < 1 or n < 1:
        raise ValueError("need at least one tree of at least one node")
    W = (n + 31) // 32
    with torch.cuda.stream(_torch_stream(stream)):
        mask = torch.empty((n_trees, n, W), dtype=torch.int32, device=dev)
        ef = torch.empty(n_trees, dtype=torch.int32, device=dev)
    st = lib().spec_tree_mask(n_trees, n, _ptr(parent), stride, _ptr(mask), _ptr(ef), _stream(stream))
    _check(st, "spec_tree_mask")
    return {"mask": mask, "err_flags": ef}


def read_probe_words(*tensors) -> int:
    """Sink words spec_read_probe needs for these tensors (one per 8 KiB chunk)."""
    return sum((t.numel() * t.element_size() + 8191) // 8192 for t in tensors if t is not None)


def read_probe(a, b=None, sink=None, stream=None):
    """spec_read_probe: a plain streaming read of device tensors a and b (b may be
    None), a measurement aid; returns the sink (each chunk's largest 32-bit word)."""
    torch = _torch()
    for t in (a, b):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("read_probe: contiguous device tensors")
    need = read_probe_words(a, b)
    if sink is None:
        with torch.cuda.stream(_torch_stream(stream)):
            sink = torch.empty(max(need, 1), dtype=torch.int32, device=a.device)
    elif sink.dtype != torch.int32 or not sink.is_contiguous() or sink.numel() < need:
        raise ValueError(f"read_probe: sink of at least {need} int32 words")
    nb = lambda t: 0 if t is None else t.numel() * t.element_size()
    st = lib().spec_read_probe(_ptr(a), nb(a), _ptr(b), nb(b), _ptr(sink), sink.numel(), _stream(stream))
    _check(st, "spec_read_probe")
    return sink


def set_wait_limit(seconds: float):
    """spec_set_wait_limit: how long any wait between the waves of a launch may last
    before it gives up with SV_ERR_INTERNAL, on the current device (a test hook;
    default 0.25 s)."""
    _check(lib().spec_set_wait_limit(float(seconds)), "spec_set_wait_limit")


def tree_build_greedy(accuracy, budget: int):
    """Greedy sparse tree from a [K][S] accuracy table (host; spec_tree_build_greedy).
    Returns numpy arrays parent, depth, rank and the expected accepted length."""
    import numpy as np
    acc = np.ascontiguousarray(np.asarray(accuracy, np.float64))
    K, S = acc.shape
    par = np.empty(budget + 1, np.int32)
    dep = np.empty(budget + 1, np.int32)
    rk = np.empty(budget + 1, np.int32)
    E = ctypes.c_double()
    cp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    n = lib().spec_tree_build_greedy(K, S, cp(acc), budget, cp(par), cp(dep), cp(rk), ctypes.byref(E))
    if n < 0:
        raise SpecVerifyError(int(-n), "spec_tree_build_greedy")
    return {"parent": par[:n].copy(), "depth": dep[:n].copy(), "rank": rk[:n].copy(), "expected_len": E.value}

