"""Build libgguf_qk.so in-tree with hipcc for gfx950 only.

    python -m gguf_block_quant_dequant_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libgguf_qk.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep every fp32 operation scalar (no v_pk_*_f32).
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the dispatcher places up to 16 leading scalar kernel arguments in SGPRs
    # before the waves start (no argument load on the critical path)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def sources() -> list[str]:
    return [os.path.join(CSRC, "gguf_qk.hip"), os.path.join(CSRC, "gguf_file.cpp")]


def build_library(verbose: bool = False) -> str:
    """Compile the HIP sources into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
