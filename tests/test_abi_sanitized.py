"""The host code of the C ABI (argument validation, workspace planning) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by tests/abi_host_check.c.

CPU only: the sanitizers instrument host code alone (the kernels are linked from the
regular build), and the driver makes no GPU call that gets past validation on a
machine without a GPU.  Any sanitizer report or failed expectation fails the test.
"""

import os
import shutil
import subprocess

import pytest

from helpers import ROOT, ensure_built

PKG = os.path.join(ROOT, "compressed_sparse_attention_07_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only sanitizer run; a GPU is visible")
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    ensure_built()
    objs = [os.path.join(PKG, "_build", f"{n}.o") for n in ("compress", "indexer", "topk", "mqa", "proj")]
    if not all(os.path.exists(o) for o in objs):
        from compressed_sparse_attention_07_amd import build
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-I" + os.path.join(ROOT, "include"),
          "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o])
    drv_o = str(tmp_path / "driver.o")
    _run([CLANG, "-x", "c", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "abi_host_check.c"), "-o", drv_o])
    exe = str(tmp_path / "abi_host_check")
    _run([CLANG, "-fsanitize=address,undefined", drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "abi host check: ok" in r.stdout, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
