"""Build libattn_mi355x.so (gfx950) in-tree with hipcc.

    python exact_attention_108_amd/build.py

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instruction selection disabled, and linked into one shared library whose only
exported symbols are the extern "C" entry points of include/attn.h.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_prefill_bf16.hip", "attn_prefill_f32.hip", "attn_decode_bf16.hip", "attn_bwd_bf16.hip", "attn_bias.hip",
           "attn_api.cpp"]
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
# Per-source additions.  The dense prefill kernel never forms a NaN (masked
# scores are -inf, their probabilities exactly 0, inputs finite by contract), so
# its device pass may drop the NaN-quieting of max/min.  Host code and the
# decode kernel (which must ignore whatever lies past a sequence's end in the
# paged cache) keep IEEE NaN semantics.
SOURCE_FLAGS = {"attn_prefill_bf16.hip": ["-Xarch_device", "-fno-honor-nans"]}


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return out


def build(lib: str = LIB, extra_flags=()) -> str:
    """Compile and link; ``lib``/``extra_flags`` select another output and
    additional hipcc flags (e.g. -D tuning switches) for side-by-side builds."""
    obj_dir = OBJ if lib == LIB else os.path.join(os.path.dirname(os.path.abspath(lib)), "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra_flags), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())
