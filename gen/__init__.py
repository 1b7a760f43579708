"""Seeded synthetic inputs for speculative-decoding verification.

This module produces inputs only: logits, draft tokens, uniforms, candidate
trees. It contains none of the verification arithmetic, and both the CPU
oracle and the HIP library consume exactly the bytes it returns.

Workloads follow the shapes and value laws of the five named configurations:

* ``c1_tiny``   linear, B=1,  k=4, V=1000,   fp32, d~N(0,2^2), t=d+N(0,0.5^2)
* ``c2_linear`` linear, B=32, k=4, V=128256, bf16, d~N(0,3^2), t=d+N(0,1^2), T=0.7,
                draft tokens sampled from softmax(d/T)
* ``c3_mtp``    linear, D=256, k=1, V=129280, bf16, t~N(0,3^2) at 2 positions,
                d_0 = t_0 + N(0,0.7^2)
* ``c4_medusa_sparse`` tree, B=16, 64 candidates + root, depth <= 4, V=32000, fp16,
                t~N(0,3^2), candidate = argmax of its parent's row with prob 0.6
* ``c5_medusa_full``  tree, B=4, Cartesian K=4 top-8 (4680 candidates + root),
                V=32000, fp16, t~N(0,3^2), head-k rank-1 accuracy 0.8^k

Draft tokens in greedy modes are the argmax of the draft row (the draft takes
its top token at each step, "Accelerating Sonar through speculation",
section "Ziel-Entwurf"); in stochastic modes they are drawn from
softmax(d/T) with a Gumbel-max draw in ``svgen.cpp``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsvgen.so")
_lib = None

DT_F32, DT_BF16, DT_F16 = 0, 1, 2
DTYPE_NAMES = {DT_F32: "f32", DT_BF16: "bf16", DT_F16: "f16"}
_NP_STORAGE = {DT_F32: np.float32, DT_BF16: np.uint16, DT_F16: np.uint16}

# stream purposes
P_PRIMARY, P_SECOND, P_DRAFT_DRAW, P_UNIFORM, P_SHAPE, P_CAND = 1, 2, 3, 4, 5, 6

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def build(force: bool = True) -> str:
    """Compile libsvgen.so with g++ (host code only)."""
    src = os.path.join(_HERE, "svgen.cpp")
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread",
                               src, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_double, ctypes.c_void_p)
        L.svg_mix64.restype = u64; L.svg_mix64.argtypes = [u64]
        L.svg_stream_at.restype = u64; L.svg_stream_at.argtypes = [u64, u64]
        L.svg_normal_at.restype = dbl; L.svg_normal_at.argtypes = [u64, u64]
        L.svg_key.restype = u64; L.svg_key.argtypes = [u64, u64, u64]
        L.svg_normal_pair.restype = None
        L.svg_normal_pair.argtypes = [u64, dbl, u64, dbl, u64, u64, i32, vp, vp, i32]
        L.svg_uniform24.restype = None; L.svg_uniform24.argtypes = [u64, u64, u64, vp]
        L.svg_gumbel_rows.restype = None
        L.svg_gumbel_rows.argtypes = [u64, i32, i64, i64, vp, dbl, vp, i32]
        L.svg_argmax_rows.restype = None
        L.svg_argmax_rows.argtypes = [i32, i64, i64, vp, vp, i32]
        L.svg_round.restype = None; L.svg_round.argtypes = [i32, i64, vp, vp]
        L.svg_decode.restype = None; L.svg_decode.argtypes = [i32, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- small helpers
def sm_mix(z: int) -> int:
    """SplitMix64 output function (pure Python twin of ``mix64`` in svgen.cpp)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_at(key: int, i: int) -> int:
    return sm_mix((key + (i + 1) * GAMMA) & MASK64)


def key(cfg: int, seed: int, purpose: int) -> int:
    return stream_at(stream_at(stream_at(cfg, 0) ^ seed, 0) ^ purpose, 0)


class Stream:
    """Sequential draws from one counter-based SplitMix64 stream (small draws only)."""

    def __init__(self, k: int):
        self.k, self.i = k, 0

    def next(self) -> int:
        r = stream_at(self.k, self.i)
        self.i += 1
        return r

    def below(self, n: int) -> int:
        """Integer in [0, n) by multiply-shift of the top 32 bits."""
        return ((self.next() >> 32) * n) >> 32

    def unit(self) -> float:
        """Uniform in [0, 1) with 53 bits."""
        return (self.next() >> 11) * (1.0 / 9007199254740992.0)


def empty_logits(dtype: int, shape) -> np.ndarray:
    return np.empty(shape, dtype=_NP_STORAGE[dtype])


def normal_pair(key_a, sig_a, key_b, sig_b, n, dtype, first=0, want_a=True, want_b=True):
    a = empty_logits(dtype, (n,)) if want_a else None
    b = empty_logits(dtype, (n,)) if want_b else None
    lib().svg_normal_pair(key_a, sig_a, key_b, sig_b, first, n, dtype,
                          _ptr(a) if a is not None else None,
                          _ptr(b) if b is not None else None, 0)
    return a, b


def uniforms(k_: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().svg_uniform24(k_, first, n, _ptr(out))
    return out


def gumbel_rows(k_: int, dtype: int, logits: np.ndarray, V: int, T: float) -> np.ndarray:
    rows = logits.size // V
    out = np.empty(rows, dtype=np.int32)
    lib().svg_gumbel_rows(k_, dtype, rows, V, _ptr(np.ascontiguousarray(logits)), T, _ptr(out), 0)
    return out


def argmax_rows(dtype: int, logits: np.ndarray, V: int) -> np.ndarray:
    rows = logits.size // V
    out = np.empty(rows, dtype=np.int32)
    lib().svg_argmax_rows(dtype, rows, V, _ptr(np.ascontiguousarray(logits)), _ptr(out), 0)
    return out


def round_to(dtype: int, x) -> np.ndarray:
    """Round float64 values to the storage dtype (fp32 / bf16 / fp16 bits)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = empty_logits(dtype, x.shape)
    lib().svg_round(dtype, x.size, _ptr(x), _ptr(out))
    return out


def decode(dtype: int, a: np.ndarray) -> np.ndarray:
    """Storage bits -> float64 (exact)."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    lib().svg_decode(dtype, a.size, _ptr(a), _ptr(out))
    return out


# ---------------------------------------------------------------- workloads
@dataclass
class LinearWorkload:
    name: str
    mode: str                   # "greedy" | "stochastic"
    temperature: float
    B: int
    k: int
    V: int
    dtype: int
    target: np.ndarray          # [B][k+1][V] storage dtype
    draft: np.ndarray           # [B][k][V]   storage dtype
    draft_tokens: np.ndarray    # [B][k] int32
    uniforms: np.ndarray        # [B][k+1] float32
    meta: dict = field(default_factory=dict)

    @property
    def elem_bytes(self):
        return 4 if self.dtype == DT_F32 else 2

    def algorithmic_bytes(self):
        rows = self.B * ((2 * self.k + 1) if self.mode == "stochastic" else (self.k + 1))
        return rows * self.V * self.elem_bytes


@dataclass
class TreeWorkload:
    name: str
    mode: str
    temperature: float
    B: int
    n_nodes: int                # candidates + root
    V: int
    dtype: int
    parent: np.ndarray          # [n_nodes] int32 (shared by the batch)
    cand: np.ndarray            # [B][n_nodes] int32, entry 0 unused (-1)
    logits: np.ndarray          # [B][n_nodes][V]
    uniforms: np.ndarray        # [B][n_nodes] float32
    max_depth: int
    meta: dict = field(default_factory=dict)

    @property
    def elem_bytes(self):
        return 4 if self.dtype == DT_F32 else 2

    def algorithmic_bytes(self):
        return self.B * self.n_nodes * self.V * self.elem_bytes


CFG_IDS = {"c1_tiny": 1, "c2_linear": 2, "c3_mtp": 3, "c4_medusa_sparse": 4, "c5_medusa_full": 5}


def linear_draft_target(cfg_id, seed, B, k, V, dtype, sig_d, sig_n, mode, T, name="custom"):
    """Draft-target law: d ~ N(0, sig_d^2), t = d + N(0, sig_n^2) for k+1 rows.

    Target row k (no draft row exists there) is derived from a virtual draft
    row k drawn with the same law and then discarded.
    """
    n = B * (k + 1) * V
    d_full, t = normal_pair(key(cfg_id, seed, P_PRIMARY), sig_d,
                            key(cfg_id, seed, P_SECOND), sig_n, n, dtype)
    d_full = d_full.reshape(B, k + 1, V)
    draft = np.ascontiguousarray(d_full[:, :k, :])
    target = t.reshape(B, k + 1, V)
    tokens = _draft_tokens(cfg_id, seed, draft, B, k, V, dtype, mode, T)
    u = uniforms(key(cfg_id, seed, P_UNIFORM), B * (k + 1)).reshape(B, k + 1)
    return LinearWorkload(name, mode, T, B, k, V, dtype, target, draft, tokens, u,
                          {"cfg_id": cfg_id, "seed": seed})


def linear_mtp(cfg_id, seed, B, V, dtype, sig_t, sig_n, mode, T, name="custom"):
    """MTP law (k=1): t ~ N(0, sig_t^2) at 2 positions, d_0 = t_0 + N(0, sig_n^2)."""
    k = 1
    n = B * 2 * V
    t, d_all = normal_pair(key(cfg_id, seed, P_PRIMARY), sig_t,
                           key(cfg_id, seed, P_SECOND), sig_n, n, dtype)
    target = t.reshape(B, 2, V)
    draft = np.ascontiguousarray(d_all.reshape(B, 2, V)[:, :1, :])
    tokens = _draft_tokens(cfg_id, seed, draft, B, k, V, dtype, mode, T)
    u = uniforms(key(cfg_id, seed, P_UNIFORM), B * 2).reshape(B, 2)
    return LinearWorkload(name, mode, T, B, k, V, dtype, target, draft, tokens, u,
                          {"cfg_id": cfg_id, "seed": seed})


def _draft_tokens(cfg_id, seed, draft, B, k, V, dtype, mode, T):
    if k == 0:
        return np.zeros((B, 0), dtype=np.int32)
    if mode == "greedy":
        return argmax_rows(dtype, draft, V).reshape(B, k)
    return gumbel_rows(key(cfg_id, seed, P_DRAFT_DRAW), dtype, draft, V, T).reshape(B, k)


def c1_tiny(seed: int, mode: str = "stochastic", B: int = 1):
    return linear_draft_target(1, seed, B, 4, 1000, DT_F32, 2.0, 0.5, mode, 1.0, "c1_tiny")


def c2_linear(seed: int, mode: str = "stochastic", B: int = 32):
    return linear_draft_target(2, seed, B, 4, 128256, DT_BF16, 3.0, 1.0, mode, 0.7, "c2_linear")


def c3_mtp(seed: int, mode: str = "stochastic", B: int = 256):
    return linear_mtp(3, seed, B, 129280, DT_BF16, 3.0, 0.7, mode, 1.0, "c3_mtp")


# ---------------------------------------------------------------- trees
def tree_depths(parent: np.ndarray) -> np.ndarray:
    depth = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    return depth


def random_sparse_tree(cfg_id, seed, n_cand=64, max_depth=4):
    """Random tree: n_cand depths uniform in {1..max_depth}, sorted (BFS order),
    redrawn until every level is non-empty; each node's parent is a uniformly
    chosen node one level up (the root for level 1)."""
    st = Stream(key(cfg_id, seed, P_SHAPE))
    while True:
        depths = sorted(1 + st.below(max_depth) for _ in range(n_cand))
        if set(depths) == set(range(1, max_depth + 1)):
            break
    depth = [0] + depths
    by_level = {0: [0]}
    parent = [-1]
    for i in range(1, n_cand + 1):
        ups = by_level[depth[i] - 1]
        parent.append(ups[st.below(len(ups))])
        by_level.setdefault(depth[i], []).append(i)
    return np.asarray(parent, dtype=np.int32)


def cartesian_tree(s_list):
    """Cartesian candidate tree in BFS order: every node at level i-1 has s_i
    children (ranks 1..s_i, contiguous). Returns (parent, rank)."""
    parent, rank = [-1], [0]
    level = [0]
    for s in s_list:
        nxt = []
        for p in level:
            for r in range(1, s + 1):
                parent.append(p)
                rank.append(r)
                nxt.append(len(parent) - 1)
        level = nxt
    return np.asarray(parent, dtype=np.int32), np.asarray(rank, dtype=np.int32)


def tree_logits(cfg_id, seed, B, n_nodes, V, dtype, sig):
    a, _ = normal_pair(key(cfg_id, seed, P_PRIMARY), sig, 0, 0.0, B * n_nodes * V, dtype,
                       want_b=False)
    return a.reshape(B, n_nodes, V)


def c4_medusa_sparse(seed: int, mode: str = "greedy", B: int = 16, V: int = 32000,
                     n_cand: int = 64, p_hit: float = 0.6, T: float = 1.0):
    cfg = 4
    parent = random_sparse_tree(cfg, seed, n_cand, 4)
    n = len(parent)
    logits = tree_logits(cfg, seed, B, n, V, DT_F16, 3.0)
    am = argmax_rows(DT_F16, logits, V).reshape(B, n)
    st = Stream(key(cfg, seed, P_CAND))
    cand = np.full((B, n), -1, dtype=np.int32)
    for b in range(B):
        for i in range(1, n):
            if st.unit() < p_hit:
                cand[b, i] = am[b, parent[i]]
            else:
                cand[b, i] = st.below(V)
    u = uniforms(key(cfg, seed, P_UNIFORM), B * n).reshape(B, n)
    return TreeWorkload("c4_medusa_sparse", mode, T, B, n, V, DT_F16, parent, cand, logits, u,
                        int(tree_depths(parent).max()), {"cfg_id": cfg, "seed": seed})


def c5_medusa_full(seed: int, mode: str = "greedy", B: int = 4, V: int = 32000,
                   s_list=(8, 8, 8, 8), acc_base: float = 0.8, T: float = 1.0):
    """Cartesian top-s tree; at depth k, rank 1 of each node's children is the
    parent's argmax with probability acc_base**k, otherwise a non-argmax token;
    ranks 2..s are distinct non-argmax tokens (siblings are all distinct)."""
    cfg = 5
    parent, rank = cartesian_tree(list(s_list))
    n = len(parent)
    depth = tree_depths(parent)
    logits = tree_logits(cfg, seed, B, n, V, DT_F16, 3.0)
    am = argmax_rows(DT_F16, logits, V).reshape(B, n)
    st = Stream(key(cfg, seed, P_CAND))
    cand = np.full((B, n), -1, dtype=np.int32)
    for b in range(B):
        i = 1
        while i < n:
            p = parent[i]
            s = s_list[depth[i] - 1]
            a = int(am[b, p])
            used = {a}
            for r in range(s):
                j = i + r
                if r == 0 and st.unit() < acc_base ** depth[j]:
                    cand[b, j] = a
                    continue
                while True:
                    t = st.below(V)
                    if t not in used:
                        break
                used.add(t)
                cand[b, j] = t
            i += s
    u = uniforms(key(cfg, seed, P_UNIFORM), B * n).reshape(B, n)
    return TreeWorkload("c5_medusa_full", mode, T, B, n, V, DT_F16, parent, cand, logits, u,
                        int(depth.max()), {"cfg_id": cfg, "seed": seed, "rank": rank})


CONFIGS = {
    "c1_tiny": c1_tiny,
    "c2_linear": c2_linear,
    "c3_mtp": c3_mtp,
    "c4_medusa_sparse": c4_medusa_sparse,
    "c5_medusa_full": c5_medusa_full,
}
