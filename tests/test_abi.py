"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host before anything reaches a GPU (no compute
calls here: every call below returns before the first HIP call)."""
import ctypes
import os
import re

import pytest

import acceptance_row_softmax_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sv.LIB_PATH):
        pytest.fail("libspecverify.so is not built (run __graft_entry__.build())")
    return sv.lib()


def test_header_symbols_are_exported(L):
    names = _declared()
    assert set(names) == set(sv.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_no_oracle_dependency():
    # the product library and binding never load the oracle
    import subprocess
    out = subprocess.run(["ldd", sv.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    src = open(os.path.join(ROOT, "acceptance_row_softmax_amd", "__init__.py")).read()
    assert "import oracle" not in src and "from oracle" not in src


DUMMY = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _lin(L, mode=1, T=1.0, B=2, k=2, V=100, dt=1, tgt=DUMMY, drf=DUMMY, tok=DUMMY, u=DUMMY,
         acc=DUMMY, out=DUMMY, ws=None, wsb=0):
    return L.spec_verify_linear(mode, T, B, k, V, dt, tgt, drf, tok, u, acc, out, None, None, None,
                                ws, wsb, None)


def test_linear_validation(L):
    assert _lin(L, dt=7) == 2                      # SV_EDTYPE
    assert _lin(L, mode=3) == 1                    # SV_EINVAL
    assert _lin(L, T=0.0) == 1
    assert _lin(L, T=float("nan")) == 1
    assert _lin(L, T=-1.0) == 1
    assert _lin(L, B=-1) == 1
    assert _lin(L, V=0) == 1
    assert _lin(L, k=32) == 5                      # SV_ELIMIT (k <= 31)
    assert _lin(L, V=3_000_000) == 5               # more than 256 chunks per row
    # SV_MAX_ROW_BYTES: 2 MiB of logits per row; at the limit validation goes on
    assert _lin(L, V=sv.SV_MAX_ROW_BYTES // 2 + 1) == 5
    assert _lin(L, V=sv.SV_MAX_ROW_BYTES // 2, ws=None) == 3
    assert _lin(L, V=sv.SV_MAX_ROW_BYTES // 4 + 1, dt=0) == 5
    assert _lin(L, V=sv.SV_MAX_ROW_BYTES // 4, dt=0, ws=None) == 3
    assert _lin(L, tgt=None) == 1
    assert _lin(L, tok=None) == 1
    assert _lin(L, u=None) == 1
    assert _lin(L, drf=None) == 1
    assert _lin(L, ws=None) == 3                   # SV_EWORKSPACE
    need = L.spec_verify_linear_workspace(2, 2, 100, 1, 1)
    assert need > 0
    assert _lin(L, ws=ctypes.c_void_p(0x1000), wsb=need - 1) == 3
    assert _lin(L, ws=ctypes.c_void_p(0x1001), wsb=need) == 3   # misaligned
    assert _lin(L, B=0) == 0                       # empty batch: nothing to do
    # greedy needs neither draft logits, uniforms nor a temperature
    assert _lin(L, mode=0, T=0.0, drf=None, u=None, ws=None) == 3


def test_tree_validation(L):
    def call(**kw):
        a = dict(mode=0, T=1.0, B=2, N=5, V=100, dt=2, par=DUMMY, stride=0, cand=DUMMY, lg=DUMMY,
                 u=None, md=2, acc=DUMMY, path=DUMMY, out=DUMMY, ws=None, wsb=0)
        a.update(kw)
        return L.spec_verify_tree(a["mode"], a["T"], a["B"], a["N"], a["V"], a["dt"], a["par"],
                                  a["stride"], a["cand"], a["lg"], a["u"], a["md"], a["acc"],
                                  a["path"], a["out"], None, a["ws"], a["wsb"], None)
    assert call(N=0) == 1
    assert call(N=16385) == 5
    assert call(md=-1) == 1
    assert call(par=None) == 1
    assert call(mode=1) == 1                      # stochastic needs uniforms
    assert call(mode=1, u=DUMMY, T=0.0) == 1
    assert call() == 3
    assert call(B=0) == 0
    assert L.spec_verify_tree_workspace(4, 4681, 32000, 2, 0) > 4 * 4681 * 4 * 16


def test_row_stats_validation(L):
    assert L.spec_row_stats(1, 0.0, 4, 10, DUMMY, None, None, None, None, None, 0, None) == 1
    assert L.spec_row_stats(1, 1.0, 4, 10, None, None, None, None, None, None, 0, None) == 1
    assert L.spec_row_stats(1, 1.0, 0, 10, None, None, None, None, None, None, 0, None) == 0
    assert L.spec_row_stats(1, 1.0, 4, 10, DUMMY, None, None, None, None, None, 0, None) == 3


def test_read_probe_validation(L):
    P = lambda a, ab, b, bb, sink, sw: L.spec_read_probe(a, ab, b, bb, sink, sw, None)
    assert P(None, 0, None, 0, None, 0) == 0                       # nothing to read
    assert P(None, 16, None, 0, DUMMY, 1) == 1                     # null buffer of nonzero size
    assert P(DUMMY, 16, None, 8, DUMMY, 1) == 1
    assert P(ctypes.c_void_p(0x1008), 16, None, 0, DUMMY, 1) == 1  # misaligned
    assert P(DUMMY, 8192, DUMMY, 8193, DUMMY, 2) == 1              # sink: 1 + 2 chunks
    assert P(DUMMY, 8192, DUMMY, 8193, None, 3) == 1


def test_status_strings(L):
    for s in range(6):
        assert len(sv.status_string(s)) > 0
