"""Build liblychee_decode.so (gfx950) in-tree with hipcc.

Usage: python -m hybrid_head_sparse_retrieval_amd.build  [--verbose]
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblychee_decode.so")
# (source, object, extra options): the attention kernels compile once per KV group size and
# kind of instance (token sets, block sets, token sets over paged KV)
UNITS = [("ld_api.hip", "ld_api.o", []), ("ld_select.hip", "ld_select.o", []),
         ("ld_window.hip", "ld_window.o", []), ("ld_tsa.hip", "ld_tsa.o", []),
         ("ld_prefill.hip", "ld_prefill.o", [])] + \
        [("ld_attention.hip", f"ld_attention_g{g}.o", [f"-DLD_ATTN_G={g}"]) for g in (1, 2, 4, 8)] + \
        [("ld_attention.hip", f"ld_attention_blk_g{g}.o", [f"-DLD_ATTN_G={g}", "-DLD_ATTN_BLK=1"]) for g in (1, 2, 4, 8)] + \
        [("ld_attention.hip", f"ld_attention_pg_g{g}.o", [f"-DLD_ATTN_G={g}", "-DLD_ATTN_PG=1"]) for g in (1, 2, 4, 8)]
SOURCES = sorted({u[0] for u in UNITS})

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 instructions stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# per-source options: the dense-attention kernel keeps its matrix-core accumulators in
# VGPRs, so the online-softmax rescale works on them in place
EXTRA = {"ld_tsa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "ld_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass does not know the packed-fp32 feature; that notice is harmless
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src, oname, opts in UNITS:
        obj = os.path.join(BUILD, oname)
        cmd = [hipcc, *COMMON, *EXTRA.get(src, []), *opts, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "--save-temps")
        objs.append(obj)
        cmds.append(cmd)
    with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, save_temps="--save-temps" in sys.argv))
