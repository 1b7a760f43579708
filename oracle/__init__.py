"""ctypes binding of the reference oracle -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The HIP library never calls it, and it
shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

TIE_EPS = 1e-6

MUT_NONE = 0
MUT_RESIDUAL_AS_TARGET = 1
MUT_SWAPPED_RATIO = 2
MUT_NO_BONUS = 3
MUT_INVCDF_GE = 4
MUT_TREE_NO_ANCESTOR = 5
MUT_TEMPERATURE_IGNORED = 6
MUT_LSE_WITHOUT_MAX = 7
MUT_COMMIT_REJECTED_DRAFT = 8
MUT_NEAR_LO_ONLY = 9
MUT_NEVAL_ALL = 10
MUT_ACCEPT_TIE_OFF = 11

# near_tie bits: a near tie that can change the accepted length, one that can
# change only the final token
NT_DECISION = 1
NT_FINAL = 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (plain host C++17, single-threaded)."""
    src = os.path.join(_HERE, "oracle.cpp")
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fno-fast-math", "-shared", "-fPIC",
                               src, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.orc_row_stats.restype = i32
        L.orc_row_stats.argtypes = [i32, dbl, i64, i64, vp, vp, vp, vp, vp]
        L.orc_invcdf.restype = i64
        L.orc_invcdf.argtypes = [vp, i64, dbl, vp, vp]
        L.orc_verify_linear.restype = i32
        L.orc_verify_linear.argtypes = [i32, dbl, i64, i64, i64, i32, vp, vp, vp, vp, dbl,
                                        vp, vp, vp, vp, vp, vp, vp]
        L.orc_verify_tree.restype = i32
        L.orc_verify_tree.argtypes = [i32, dbl, i64, i64, i64, i32, vp, i64, vp, vp, vp, i64, dbl,
                                      vp, vp, vp, vp, vp, vp, vp]
        L.orc_expected_accept_len.restype = dbl
        L.orc_expected_accept_len.argtypes = [i64, vp, vp, i64, vp]
        L.orc_commit_linear.restype = i32
        L.orc_commit_linear.argtypes = [i64, i64, vp, vp, vp, vp, vp, i64, vp, vp, vp]
        L.orc_sample.restype = i32
        L.orc_sample.argtypes = [i32, dbl, i64, i64, i32, vp, vp, dbl, vp, vp, vp]
        L.orc_tree_mask.restype = i32
        L.orc_tree_mask.argtypes = [i64, vp, vp]
        L.orc_tree_build_greedy.restype = i64
        L.orc_tree_build_greedy.argtypes = [i64, i64, vp, i64, vp, vp, vp, vp]
        L.orc_verify_tree_typical.restype = i32
        L.orc_verify_tree_typical.argtypes = [dbl, dbl, dbl, i64, i64, i64, i32, vp, i64, vp, vp, vp, i64,
                                              dbl, vp, vp, vp, vp, vp, vp]
        L.orc_set_mutation.restype = None
        L.orc_set_mutation.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


class mutation:
    """Context manager planting a mistake in the oracle (negative-control tests)."""

    def __init__(self, which: int):
        self.which = which

    def __enter__(self):
        lib().orc_set_mutation(self.which)
        return self

    def __exit__(self, *exc):
        lib().orc_set_mutation(MUT_NONE)


def row_stats(x: np.ndarray, V: int, dtype: int, T: float = 1.0):
    x = np.ascontiguousarray(x)
    rows = x.size // V
    m = np.empty(rows, np.float64)
    lse = np.empty(rows, np.float64)
    am = np.empty(rows, np.int32)
    fl = np.empty(rows, np.int32)
    rc = lib().orc_row_stats(dtype, T, rows, V, _p(x), _p(m), _p(lse), _p(am), _p(fl))
    if rc:
        raise ValueError("orc_row_stats: bad arguments")
    return {"max": m, "lse": lse, "argmax": am, "err": fl}


def invcdf(w, u: float):
    w = np.ascontiguousarray(np.asarray(w, np.float64))
    lo, hi = ctypes.c_double(), ctypes.c_double()
    y = lib().orc_invcdf(_p(w), w.size, float(u), ctypes.byref(lo), ctypes.byref(hi))
    return int(y), lo.value, hi.value


def verify_linear(mode: str, T: float, target, draft, draft_tokens, uniforms, V: int, dtype: int,
                  tie_eps: float = TIE_EPS):
    target = np.ascontiguousarray(target)
    B = target.shape[0]
    k = target.shape[1] - 1
    tok = np.ascontiguousarray(np.asarray(draft_tokens, np.int32).reshape(B, k))
    stoch = mode == "stochastic"
    draft = np.ascontiguousarray(draft) if (draft is not None and stoch) else None
    u = np.ascontiguousarray(np.asarray(uniforms, np.float32)) if stoch else None
    acc = np.empty(B, np.int32)
    out = np.empty((B, k + 1), np.int32)
    pt = np.full((B, k), np.nan)
    pd = np.full((B, k), np.nan)
    err = np.empty(B, np.int32)
    nt = np.empty(B, np.int32)
    ne = np.empty(B, np.int32)
    rc = lib().orc_verify_linear(1 if stoch else 0, T, B, k, V, dtype, _p(target), _p(draft),
                                 _p(tok), _p(u), tie_eps, _p(acc), _p(out), _p(pt), _p(pd),
                                 _p(err), _p(nt), _p(ne))
    if rc:
        raise ValueError("orc_verify_linear: bad arguments")
    return {"accept_len": acc, "out_tokens": out, "p_target": pt, "p_draft": pd,
            "err_flags": err, "near_tie": nt, "n_eval": ne}


def verify_tree(mode: str, T: float, parent, cand, logits, uniforms, V: int, dtype: int,
                max_depth: int, tie_eps: float = TIE_EPS):
    logits = np.ascontiguousarray(logits)
    B, n = logits.shape[0], logits.shape[1]
    parent = np.ascontiguousarray(np.asarray(parent, np.int32))
    stride = 0 if parent.ndim == 1 else n
    cand = np.ascontiguousarray(np.asarray(cand, np.int32).reshape(B, n))
    stoch = mode == "stochastic"
    u = np.ascontiguousarray(np.asarray(uniforms, np.float32)) if stoch else None
    acc = np.empty(B, np.int32)
    path = np.empty((B, max_depth), np.int32)
    out = np.empty((B, max_depth + 1), np.int32)
    err = np.empty(B, np.int32)
    nt = np.empty(B, np.int32)
    ne = np.empty(B, np.int32)
    y = np.empty((B, n), np.int32)
    rc = lib().orc_verify_tree(1 if stoch else 0, T, B, n, V, dtype, _p(parent), stride, _p(cand),
                               _p(logits), _p(u), max_depth, tie_eps, _p(acc), _p(path), _p(out),
                               _p(err), _p(nt), _p(ne), _p(y))
    if rc:
        raise ValueError("orc_verify_tree: bad arguments")
    return {"accept_len": acc, "path_nodes": path, "out_tokens": out, "err_flags": err,
            "near_tie": nt, "n_eval": ne, "node_token": y}


def expected_accept_len(parent, rank, acc_table) -> float:
    parent = np.ascontiguousarray(np.asarray(parent, np.int32))
    rank = np.ascontiguousarray(np.asarray(rank, np.int32))
    acc_table = np.ascontiguousarray(np.asarray(acc_table, np.float64))
    S = acc_table.shape[1]
    return lib().orc_expected_accept_len(parent.size, _p(parent), _p(rank), S, _p(acc_table))


def commit_linear(accept_len, out_tokens, drafts, seq_len, history=None):
    """Returns (seq_len', history', {"shifted", "next_token", "err_flags"}); inputs untouched."""
    acc = np.ascontiguousarray(np.asarray(accept_len, np.int32))
    out = np.ascontiguousarray(np.asarray(out_tokens, np.int32))
    B, k = out.shape[0], out.shape[1] - 1
    dr = np.ascontiguousarray(np.asarray(drafts, np.int32).reshape(B, k)) if drafts is not None else None
    ln = np.array(seq_len, np.int32, copy=True)
    hist = np.array(history, np.int32, copy=True) if history is not None else None
    cap = hist.shape[1] if hist is not None else 0
    sh = np.empty((B, k + 1), np.int32)
    nx = np.empty(B, np.int32)
    ef = np.empty(B, np.int32)
    rc = lib().orc_commit_linear(B, k, _p(acc), _p(out), _p(dr), _p(ln), _p(hist), cap, _p(sh), _p(nx), _p(ef))
    if rc:
        raise ValueError("orc_commit_linear: bad arguments")
    return ln, hist, {"shifted": sh, "next_token": nx, "err_flags": ef}


def sample(mode: str, T: float, x, uniforms, V: int, dtype: int, tie_eps: float = TIE_EPS):
    x = np.ascontiguousarray(x)
    rows = x.size // V
    stoch = mode == "stochastic"
    u = np.ascontiguousarray(np.asarray(uniforms, np.float32).reshape(rows)) if stoch else None
    tok = np.empty(rows, np.int32)
    ef = np.empty(rows, np.int32)
    nt = np.empty(rows, np.int32)
    rc = lib().orc_sample(1 if stoch else 0, T, rows, V, dtype, _p(x), _p(u), tie_eps, _p(tok), _p(ef), _p(nt))
    if rc:
        raise ValueError("orc_sample: bad arguments")
    return {"tokens": tok, "err_flags": ef, "near_tie": nt}


def tree_mask(parent):
    """Dense [n][n] uint8 ancestor-or-self matrix, or None for an invalid parent array."""
    parent = np.ascontiguousarray(np.asarray(parent, np.int32))
    n = parent.size
    dense = np.empty((n, n), np.uint8)
    rc = lib().orc_tree_mask(n, _p(parent), _p(dense))
    return None if rc else dense


def tree_build_greedy(acc, budget: int):
    acc = np.ascontiguousarray(np.asarray(acc, np.float64))
    K, S = acc.shape
    par = np.empty(budget + 1, np.int32)
    dep = np.empty(budget + 1, np.int32)
    rk = np.empty(budget + 1, np.int32)
    E = ctypes.c_double()
    n = lib().orc_tree_build_greedy(K, S, _p(acc), budget, _p(par), _p(dep), _p(rk), ctypes.byref(E))
    if n < 0:
        raise ValueError("orc_tree_build_greedy: bad arguments")
    return {"parent": par[:n].copy(), "depth": dep[:n].copy(), "rank": rk[:n].copy(), "expected_len": E.value}


def verify_tree_typical(T: float, epsilon: float, delta: float, parent, cand, logits, uniforms, V: int,
                        dtype: int, max_depth: int, tie_eps: float = TIE_EPS):
    logits = np.ascontiguousarray(logits)
    B, n = logits.shape[0], logits.shape[1]
    parent = np.ascontiguousarray(np.asarray(parent, np.int32))
    stride = 0 if parent.ndim == 1 else n
    cand = np.ascontiguousarray(np.asarray(cand, np.int32).reshape(B, n))
    u = np.ascontiguousarray(np.asarray(uniforms, np.float32).reshape(B, n))
    acc = np.empty(B, np.int32)
    path = np.empty((B, max_depth), np.int32)
    out = np.empty((B, max_depth + 1), np.int32)
    err = np.empty(B, np.int32)
    nt = np.empty(B, np.int32)
    ne = np.empty(B, np.int32)
    rc = lib().orc_verify_tree_typical(T, epsilon, delta, B, n, V, dtype, _p(parent), stride, _p(cand),
                                       _p(logits), _p(u), max_depth, tie_eps, _p(acc), _p(path), _p(out),
                                       _p(err), _p(nt), _p(ne))
    if rc:
        raise ValueError("orc_verify_tree_typical: bad arguments")
    return {"accept_len": acc, "path_nodes": path, "out_tokens": out, "err_flags": err,
            "near_tie": nt, "n_eval": ne}

