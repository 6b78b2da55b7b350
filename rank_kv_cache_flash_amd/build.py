"""Build libwsvd.so (gfx950) in-tree with hipcc.

    python -m rank_kv_cache_flash_amd.build          # compile + link

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off, and linked into rank_kv_cache_flash_amd/libwsvd.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwsvd.so")

SOURCES = ["abi.hip", "decode.hip", "decode_bf16_r32.hip", "decode_rope.hip", "combine.hip", "append.hip", "append_stream.hip", "w8a8.hip", "factorize.hip", "shared_decode.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# Per-source additions.  The rotary-key decode keeps its MFMA results in
# ordinary VGPRs (gfx950 MFMAs can write them directly), which removes the
# 32 accumulation-register reads per 16-row tile: 113.5 -> 112.5 us on the
# 16 x 32-head, 4096-token r 64 decode.  The append kernel measured slower
# with the same option, so it stays per file.
SOURCE_FLAGS = {
    "decode_rope.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # The bf16 rank-32 split-kernel instances, scheduled for ILP: 5.01 ->
    # 4.87 us on the 1 x 32-head, 1088-token decode (other instances slower).
    "decode_bf16_r32.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), 8)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
