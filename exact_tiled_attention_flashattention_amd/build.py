"""Build libattn.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m exact_tiled_attention_flashattention_amd.build

Every source is compiled on each call (objects under ``_build/`` at the repo
root) and linked into ``exact_tiled_attention_flashattention_amd/libattn.so``.
Packed fp32 VALU instructions are disabled for all device code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libattn.so")

SOURCES = ["attn_api.cpp", "block_pool.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip",
           "kv_cache.hip", "backward_bf16.hip", "decode_static.cpp"]
ARCH = "gfx950"


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libattn")
    return exe


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wno-unused-result",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", path, "-o", obj] + common_flags()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
