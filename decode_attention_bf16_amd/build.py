"""Build the gfx950 shared library libdecode_attn.so in-tree with hipcc, and the
benchmark's HBM read-rate probe libda_read_probe.so beside it.

    python -m decode_attention_bf16_amd.build          # build
    python -m decode_attention_bf16_amd.build --asm    # also keep the AMDGPU assembly in _build/

Flags: -O3 for gfx950 only; packed-fp32 instructions are switched off for the
device code (the kernels are written with scalar/float4 fp32 arithmetic and
must not be turned into v_pk_* forms).
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "decode_attn.hip")
LIB = os.path.join(HERE, "libdecode_attn.so")
PROBE_SRC = os.path.join(HERE, "csrc", "read_probe.hip")
PROBE_LIB = os.path.join(HERE, "libda_read_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(asm: bool = False, verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [SRC, "-o", tmp]
    if asm:
        os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
        # temps (assembly etc.) go to the working directory, _build/
        cmd += ["-save-temps", "-Rpass-analysis=kernel-resource-usage"]
    cwd = os.path.join(ROOT, "_build") if asm else HERE
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, LIB)
    ptmp = PROBE_LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC] + FLAGS + [PROBE_SRC, "-o", ptmp], check=True, cwd=HERE)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, verbose=True))
    sys.exit(0)
