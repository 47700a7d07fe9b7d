"""Build libgguf_qk.so in-tree with hipcc for gfx950 only.

    python -m gguf_block_quant_dequant_amd.build [-v] [--timeline]

Each source is compiled to an object file in parallel (one hipcc process per
translation unit), then the objects are linked into the shared library.
--timeline builds libgguf_qk_timeline.so instead: the same library with
per-wave time stamps recorded by the decode GEMV kernels (GQK_TIMELINE), for
stage timelines; it is never the default library. --sanitize builds
_build/libgguf_qk_asan.so: the host code under AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged), for the CPU tests of the
file reader and of argument validation (load it with the sanitizer runtime
preloaded, see tests/test_host_sanitizers.py).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libgguf_qk.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
TIMELINE_LIB_PATH = os.path.join(PKG_DIR, "libgguf_qk_timeline.so")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
ASAN_LIB_PATH = os.path.join(OBJ_DIR, "libgguf_qk_asan.so")
# host-only sanitizers (each -fsanitize= applies to the host pass only)
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep every fp32 operation scalar (no v_pk_*_f32).
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the dispatcher places up to 16 leading scalar kernel arguments in SGPRs
    # before the waves start (no argument load on the critical path)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


# (source, extra defines, object tag): the lanes-along-K launches are compiled
# once per block type (GGUF ids 12 Q4_K, 2 Q4_0, 14 Q6_K, 8 Q8_0; Q4_K also
# with the fused epilogues) so that the heavy kernel families build in parallel.
UNITS = [
    ("gguf_qk.hip", [], "abi"),
    ("lk.hip", [], "lkplan"),
    ("lk_typed.hip", ["-DGQK_LK_TYPE=12", "-DGQK_LK_EP=0"], "lk_q4k"),
    ("lk_typed.hip", ["-DGQK_LK_TYPE=12", "-DGQK_LK_EP=1"], "lk_q4k_ep"),
    ("lk_typed.hip", ["-DGQK_LK_TYPE=2", "-DGQK_LK_EP=0"], "lk_q4_0"),
    ("lk_typed.hip", ["-DGQK_LK_TYPE=14", "-DGQK_LK_EP=0"], "lk_q6_k"),
    ("lk_typed.hip", ["-DGQK_LK_TYPE=8", "-DGQK_LK_EP=0"], "lk_q8_0"),
    ("gguf_file.cpp", [], "file"),
]


def sources() -> list[str]:
    return sorted({os.path.join(CSRC, f) for f, _, _ in UNITS})


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    return msgs


def build_library(verbose: bool = False, timeline: bool = False, sanitize: bool = False) -> str:
    """Compile the sources and link them into LIB_PATH (or TIMELINE_LIB_PATH,
    ASAN_LIB_PATH); always recompiles."""
    out = TIMELINE_LIB_PATH if timeline else ASAN_LIB_PATH if sanitize else LIB_PATH
    tag = "tl" if timeline else "asan" if sanitize else "rel"
    os.makedirs(OBJ_DIR, exist_ok=True)
    defs = (["-DGQK_TIMELINE=1"] if timeline else []) + (SANITIZE_FLAGS if sanitize else [])
    jobs = []
    for f, extra, name in UNITS:
        src = os.path.join(CSRC, f)
        obj = os.path.join(OBJ_DIR, f"{name}.{tag}.o")
        jobs.append(([HIPCC, *HIP_FLAGS, *defs, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o",
                      obj], obj))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = out + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libasan"] if sanitize else []
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_san, *[o for _, o in jobs], "-o",
                      tmp], verbose))
    msgs = "\n".join(m for m in outs if m)
    if verbose and msgs:
        print(msgs, flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv,
                        sanitize="--sanitize" in sys.argv))
