"""Build libmqa_decode.so in-tree with hipcc for gfx950.

Run as ``python -m transformer_decode_attention_amd.build`` (or through
``__graft_entry__.build()``). The library is written next to this file so that
it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "mqa_decode.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libmqa_decode.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Werror",
    "-Wno-unused-command-line-argument",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core accumulators in ordinary vector registers. The kernels'
    # online-softmax rescale multiplies the accumulators on the vector ALUs;
    # with accumulators in AGPRs the compiler copied all of them to VGPRs and
    # back on every 32-position step (~130 extra instructions per step).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # that line is expected. Anything else is shown.
    noise = [ln for ln in (res.stderr or "").splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
