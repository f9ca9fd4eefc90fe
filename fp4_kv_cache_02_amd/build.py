"""Build the CSA2 HIP library (libcsa2.so) in-tree for gfx950.

Usage: python -m fp4_kv_cache_02_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["csa2_api.hip", "csa2_codec.hip", "csa2_index.hip", "csa2_attn.hip", "csa2_prefill.hip",
           "csa2_attn_prefill.hip"]
# per-source code generation options
EXTRA = {
    # MFMA results in vector registers: the epilogue reads them with vector
    # instructions, which cannot take accumulation registers as operands
    "csa2_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "csa2_attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}
ARCH = os.environ.get("CSA2_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libcsa2.so next to this file; returns its path."""
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
               # no packed-fp32 instructions (CDNA packed fp32 ops are avoided on purpose)
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # keep private arrays in registers: never move them into spare LDS
               "-mllvm", "-disable-promote-alloca-to-lds",
               "-Wno-unused-result", *EXTRA.get(src, []), os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for src, p in jobs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"[csa2 build] {src} failed:\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    # every symbol must resolve: a kernel whose host stub the compiler left
    # out links fine and only fails when the library is loaded
    r = subprocess.run(["nm", "-u", "-C", tmp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    missing = [ln.strip() for ln in r.stdout.splitlines() if "csa2::" in ln]
    if missing:
        os.remove(tmp)
        raise RuntimeError("libcsa2 has unresolved symbols:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
