"""CPU-only AddressSanitizer / UndefinedBehaviorSanitizer builds.

Two programs, built here and run on the host (no GPU is touched):

* ``tests/sanitize/oracle_checks.cpp`` with ``oracle/dgo.cpp``, both compiled
  by g++ with ``-fsanitize=address,undefined``: every oracle function on
  ragged shapes, row/column subsets, one and several threads, and its
  argument errors (leak detection on).
* ``tests/sanitize/host_checks.cpp`` with the library's host source
  ``dg_host.hip`` compiled by hipcc with the sanitizers on its host side only
  (``-Xarch_host``; its device part is the static scratch array), the kernel
  table and launchers taken from the built ``libdg.so``: the tile queries over
  a grid of shapes and every entry point with one argument error, all of which
  return before any HIP call, so no kernel is launched.

Either program ends with a non-zero status on any sanitizer report (the
sanitizers are built not to recover) or failed check.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "fp8_block_scaled_scales_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def _env(detect_leaks: bool):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=%d:halt_on_error=1" % int(detect_leaks)
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    rc, out = _run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-pthread"] + SAN_FLAGS +
                   [os.path.join(ROOT, "oracle", "dgo.cpp"), os.path.join(HERE, "oracle_checks.cpp"), "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=_env(True))
    assert rc == 0 and "oracle checks passed" in out, out
    assert "Sanitizer" not in out and "runtime error" not in out, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_host_logic_under_asan_ubsan(tmp_path):
    lib = os.path.join(PKG, "libdg.so")
    if not os.path.exists(lib):
        pytest.skip("libdg.so not built (run __graft_entry__.build())")
    obj = str(tmp_path / "dg_host.o")
    exe = str(tmp_path / "host_checks")
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
                   ["-c", os.path.join(PKG, "csrc", "dg_host.hip"), "-o", obj])
    assert rc == 0, out
    rc, out = _run([CLANG, "-O1", "-g", "-std=c++17"] + SAN_FLAGS +
                   ["-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "host_checks.cpp"), obj,
                    "-L" + PKG, "-l:libdg.so", "-Wl,-rpath," + PKG, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    # the sanitized definitions of the entry points are the program's own
    rc, syms = _run(["nm", exe])
    assert rc == 0 and " T dg_gemm_fp8_ws" in syms and "__asan_report" in syms, syms[-2000:]
    # leaks off: the HIP runtime's own allocations at exit are not this library's
    rc, out = _run([exe], env=_env(False))
    assert rc == 0 and "host checks passed" in out, out
    assert "Sanitizer" not in out and "runtime error" not in out, out
