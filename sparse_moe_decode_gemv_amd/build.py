"""Build the HIP libraries in-tree for gfx950 (hipcc, no JIT cache).

  libmoe_decode.so   the decode library (C ABI in include/moe.h)
  libmoe_inputs.so   the device filler of the synthetic-input generator
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled: only scalar fp32 arithmetic is emitted.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-ffp-contract=fast"]

DECODE_SOURCES = ["abi.cpp", "moe_t1.hip", "moe_batched.hip"]
LIB_DECODE = os.path.join(HERE, "libmoe_decode.so")
LIB_INPUTS = os.path.join(ROOT, "moe_inputs", "libmoe_inputs.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build failed: {' '.join(cmd)}")
    return out


def _compile(src, obj, extra=()):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    _run([HIPCC, *HIP_FLAGS, *extra, *lang, "-c", src, "-o", obj])


def build(verbose: bool = False) -> None:
    """Compile every HIP source (always, even if a library exists)."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in DECODE_SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        _compile(os.path.join(CSRC, src), obj, ["-I", os.path.join(ROOT, "include")])
        objs.append(obj)
    tmp = LIB_DECODE + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_DECODE)
    src = os.path.join(ROOT, "moe_inputs", "fill.hip")
    obj = os.path.join(bdir, "fill.o")
    _compile(src, obj)
    tmp = LIB_INPUTS + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, "-o", tmp])
    os.replace(tmp, LIB_INPUTS)
    if verbose:
        print("built", LIB_DECODE, LIB_INPUTS)


if __name__ == "__main__":
    build(verbose=True)
