"""Builds the HIP library libgdn.so in-tree for gfx950 with hipcc.

Usage: ``python -m linear_attention_sequence_recompute_amd.build`` (or
``build_library()``). Every call recompiles all sources.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgdn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["gdn_api.hip", "gdn_chunk.hip", "gdn_decode.hip", "gdn_fp8.hip", "gdn_layer.hip", "gdn_kda_chunk.hip", "gdn_probe.hip", "gdn_gate.hip", "gdn_decode_layer.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # keep the compiler from forming packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in arch VGPRs: the scan's state and partial products feed
        # VALU work every step, and accumulator registers would need copies
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build_library(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
