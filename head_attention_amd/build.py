"""Build libheadattn.so in-tree with hipcc for gfx950 (MI355X).

Usage: python -m head_attention_amd.build   (or head_attention_amd.build.build())
The library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libheadattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd_f32.hip", "attn_fwd_bf16.hip", "attn_fwd_bf16_pair.hip", "attn_fwd_bf16_short.hip",
           "attn_fwd_bf16_band.hip",
           "attn_decode.hip", "attn_cache.hip", "attn_proj.hip",
           "attn_bwd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are turned off for every device compile.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless.
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errors.append(f"$ {' '.join(cmd)}\n{text}")
        elif verbose and text.strip():
            print(text)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libheadattn.so. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS)
    _run(cmds, verbose)
    tmp = LIB_PATH + ".tmp"
    _run([[HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
