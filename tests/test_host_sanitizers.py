"""The library's host code (argument validation, shape limits, workspace
size arithmetic and carving) built with AddressSanitizer and
UndefinedBehaviorSanitizer, driven by tests/host_sanitize/abi_checks.cpp.

Only the host side is instrumented (each sanitizer flag follows -Xarch_host;
the GPU code is compiled as usual but never launched).  The checker passes
fake, never-dereferenced device addresses to calls that the library rejects
before any HIP call, or that are pure host computations, and refuses to run
where a GPU is visible.  A sanitizer report aborts the checker (recovery is
off), which fails the test with the report in its output.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_decode_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SOURCES = ["gemm_q4k", "gemm_wk", "attn_decode", "kv_append", "small", "prefill", "qkdec"]
SAN = ["address", "undefined"]


def _build(out):
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(name):
        obj = os.path.join(out, name + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", *host_san, '-DQKDEC_BUILD_ID="sanitized"', "-c",
               os.path.join(CSRC, name + ".hip"), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    exe = os.path.join(out, "abi_checks")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=" + ",".join(SAN), "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "host_sanitize", "abi_checks.cpp"), *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_host_code_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = _build(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    if "skipped: a GPU is visible" in out:
        pytest.skip("a GPU is visible: the checker passes fake device addresses")
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert ", 0 failures" in out, out[-4000:]
