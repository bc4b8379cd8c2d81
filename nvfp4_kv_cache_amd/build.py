"""Builds libnvfp4kv.so for gfx950 in-tree with hipcc.

    python -m nvfp4_kv_cache_amd.build

Flags: -O3, C++17, no fast math (IEEE fp32 division and denormals are part of
the quantizer's bit-exact contract), and packed-fp32 VALU instructions disabled
for device code.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "quantize.hip", "attention.hip", "export.hip"]
# Per-source extra flags.  The attention kernel never produces NaN (its -inf logits
# of masked keys are handled explicitly), so its max reductions may skip the NaN
# canonicalization; the quantizer keeps full IEEE semantics.
EXTRA_FLAGS = {"attention.hip": ["-fno-honor-nans"]}

DEVICE_FLAGS = [
    "--offload-arch=gfx950",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose=False):
    out_tmp = LIB + ".tmp"
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-fno-fast-math", "-Wall",
              "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        _run(common + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", out_tmp] + objs, verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
