"""The oracle, the input generator and the library's host code under the address
and undefined-behaviour sanitizers, on the CPU. Two programs are built into a
temporary folder and run:

- tests/sanitize/oracle_gen.cpp with oracle/oracle.cpp and gen/svgen.cpp (g++);
- tests/sanitize/lib_host.cpp with the library sources; hipcc sanitizes only the
  host side of those (the flags follow -Xarch_host), and the program makes no
  call that passes its argument checks, so nothing reaches a GPU.

A sanitizer report or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd[:3]), r.stdout[-2000:], r.stderr[-4000:])
    return r


def _clean(r):
    for bad in ("AddressSanitizer", "runtime error:", "LeakSanitizer", "check failed"):
        assert bad not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_gen")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-pthread", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_gen.cpp"), os.path.join(ROOT, "oracle", "oracle.cpp"),
          os.path.join(ROOT, "gen", "svgen.cpp"), "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    _clean(r)
    assert "all checks passed" in r.stdout


def _hipcc():
    from acceptance_row_softmax_amd import _build
    return _build.hipcc()


def test_library_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang++"
    inc = os.path.join(ROOT, "include")
    objs = []
    for src in ("specverify.hip", "steps.hip"):
        obj = str(tmp_path / (src + ".o"))
        # the sanitizer flags apply to the host side only
        host_san = []
        for f in SAN:
            host_san += ["-Xarch_host", f]
        _run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", *host_san,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, "-c",
              os.path.join(ROOT, "acceptance_row_softmax_amd", "csrc", src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "lib_host.o")
    _run([clang, "-std=c++17", "-O1", "-g", *SAN, "-I", inc, "-c",
          os.path.join(ROOT, "tests", "sanitize", "lib_host.cpp"), "-o", drv])
    exe = str(tmp_path / "lib_host")
    rocm_lib = "/opt/rocm/lib"
    _run([clang, *SAN, drv, *objs, "-L", rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib, "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    _clean(r)
    assert "all checks passed" in r.stdout
