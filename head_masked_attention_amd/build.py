"""Build libbsattn.so in-tree with hipcc for gfx950.

    python -m head_masked_attention_amd.build

The shared library lands next to this file so it travels with the source
tree; nothing is installed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libbsattn.so")
SOURCES = ["bsattn.hip", "select.hip", "attn_mfma.hip", "attn_f32.hip", "attn_fp8.hip", "stage.cpp"]
HEADERS = ["common.h", "internal.h"]
# Per-source extra flags.  The attention kernel's scores come out of MFMA
# accumulators and are never NaN for finite inputs; without NaN semantics
# fmaxf lowers to bare v_max / v_max3 instead of also quieting each input
# first.  (NaN in Q, K or V gives unspecified output.)
EXTRA_FLAGS = {"attn_mfma.hip": ["-fno-honor-nans"], "attn_fp8.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libbsattn needs ROCm's hipcc to build")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # no packed fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbsattn.so; returns its path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(
            ln for ln in out.decode(errors="replace").splitlines()
            if "packed-fp32-ops" not in ln
        )
        if p.returncode != 0:
            failed.append(f"{src}:\n{text}")
        elif verbose and text.strip():
            print(text, flush=True)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
