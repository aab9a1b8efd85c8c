"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

* The C ABI's host code (api.cpp: validation, workspace arithmetic, plans,
  block entries) is built with the sanitizers on the host side only (each
  -fsanitize flag behind -Xarch_host; no device code is instrumented), linked
  with launcher stubs and driven through every entry point with invalid,
  extreme and valid arguments on this machine, which has no GPU.
* The oracle (oracle/qsa_oracle.c) is built with gcc and the same
  sanitizers and driven through all its functions on small seeded inputs.
Any out-of-bounds access, signed overflow or other undefined behaviour aborts
the driver and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "token_indexed_sparse_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "qsa_oracle.c"),
          "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=600)
    assert "oracle driver ok" in r.stdout


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is not installed")
def test_api_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "noalloc.hip"),
                os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "api_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, *common, *san, "-c", src, "-o", obj])
        objs.append(obj)
    # link on the host with ROCm's clang, which carries the host sanitizer runtimes
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    rocm_lib = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib")
    exe = str(tmp_path / "api_driver")
    _run([clang, "-fsanitize=address,undefined", "-o", exe, *objs, "-L" + rocm_lib,
          "-Wl,-rpath," + rocm_lib, "-lamdhip64"])
    r = _run([exe], env=dict(ENV, HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", "")),
             timeout=300)
    assert "api driver ok" in r.stdout
