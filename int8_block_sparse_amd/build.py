"""Build libsagesla.so (the C-ABI library with the gfx950 HIP kernels) in-tree with hipcc.

    python -m int8_block_sparse_amd.build        # or __graft_entry__.build()
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsagesla.so")
# measurement tooling beside the library: the matrix-core peak probe the benchmark runs (--workload mfma-peak)
PROBE_OUT = os.path.join(PKG, "libsagesla_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "k_quant.hip", "k_select.hip", "k_linear.hip", "k_attn.hip", "k_w8a8.hip", "k_backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the SageSLA library)")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed fp32 (v_pk_*_f32) instructions anywhere
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for out, srcs in ((OUT, SOURCES), (PROBE_OUT, PROBE_SOURCES)):
        tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
               *[o for o, src in zip(objs, SOURCES + PROBE_SOURCES) if src in srcs]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
