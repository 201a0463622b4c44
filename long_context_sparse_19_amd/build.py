"""Build libindexpool.so in-tree with hipcc for gfx950 only.

    python -m long_context_sparse_19_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libindexpool.so")
STAMPS_LIB = os.path.join(PKG, "libindexpool_stamps.so")
SOURCES = ["compress.hip", "score.hip", "select.hip", "topk.hip", "attn.hip", "attn_step_h32.hip", "attn_pipe.hip", "kda.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (hand-off to the scalar forms)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs where they fit: the attention kernel
    # rescales its O accumulators with VALU ops, which otherwise costs a copy of
    # all of them between register files on every sub-tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, stamps: bool = False) -> str:
    bdir = BUILD + ("_stamps" if stamps else "")
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DIP_PHASE_STAMPS"] if stamps else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, stamps: bool = False) -> str:
    """The library; stamps: the diagnostics library that records the decode step's
    phase stamps (ip_phase_stamps), built beside it as libindexpool_stamps.so."""
    os.makedirs(BUILD + ("_stamps" if stamps else ""), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, stamps), SOURCES))
    lib = STAMPS_LIB if stamps else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, stamps="--stamps" in sys.argv[1:])
    sys.exit(0)
