"""Build libpbs.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m block_sparse_attention_pbs_amd.build [--verbose]

Every HIP source is compiled to an object in parallel under ``_build/`` and linked into
``block_sparse_attention_pbs_amd/libpbs.so``.  Packed-fp32 instruction selection is switched
off for all device code (``-packed-fp32-ops``).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpbs.so")
SOURCES = ["pbs_api.cpp", "pbs_score.hip", "pbs_permute.hip", "pbs_select.hip", "pbs_attn.hip"]
# Per-source extra flags.  The attention kernel keeps its MFMA accumulators in VGPRs: its scores
# feed VALU work directly (no v_accvgpr_read per score), and the whole kernel then fits the
# 168-register budget of three waves per SIMD.
EXTRA_FLAGS = {"pbs_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(debug: bool = False):
    flags = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]
    flags += ["-O0", "-g"] if debug else ["-O3"]
    return flags


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc(), "-x", "hip", *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
