"""Build libqkdec.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m quantized_decode_amd.build        # or build() from Python

Objects go to quantized_decode_amd/_build/, the library to
quantized_decode_amd/libqkdec.so.  Every call recompiles.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqkdec.so")
ARCH = os.environ.get("QKDEC_ARCH", "gfx950")

SOURCES = ["gemm_q4k.hip", "gemm_wk.hip", "attn_decode.hip", "kv_append.hip", "small.hip", "prefill.hip", "qkdec.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_id() -> str:
    """Hash of everything the library is built from (its HIP sources and
    headers, the public header and the compiler flags): the build id that
    qkdec_build_id() reports, so measurements can be tied to the code they
    were taken on."""
    h = hashlib.sha256()
    h.update(" ".join(CFLAGS).encode())
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for path in [os.path.join(CSRC, f) for f in files] + [os.path.join(HERE, "..", "include", "qkdec.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _compile(src: str, build_id: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, f'-DQKDEC_BUILD_ID="{build_id}"', "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    bid = source_id()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, bid), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
