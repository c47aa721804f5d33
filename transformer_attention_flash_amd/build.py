"""Ahead-of-time build of libattn.so for gfx950 (hipcc, no JIT, no torch extension).

    python -m transformer_attention_flash_amd.build

compiles every HIP source under csrc/ into ``transformer_attention_flash_amd/libattn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "scatter.hip", "decode.hip", "prefill.hip", "prefill_small.hip", "prefill_lowp.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code on purpose; the
# host pass warns that it does not know the feature, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")
    return path


def build(out: str = LIB, extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra_flags or []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
