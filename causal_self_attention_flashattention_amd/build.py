"""Build libattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m causal_self_attention_flashattention_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` at the repository root; the library lands next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_noalloc.hip", "attn_api.cpp"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed-FP32 VALU ops are disabled for all device code.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _compile(src: str, extra: list[str]) -> tuple[subprocess.Popen, str]:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link ``libattn.so``; raises RuntimeError on failure."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    jobs = [_compile(s, extra) for s in SOURCES]
    objs, errors = [], []
    for (proc, obj), src in zip(jobs, SOURCES):
        out, _ = proc.communicate()
        if verbose and out:
            print(out, file=sys.stderr)
        if proc.returncode != 0:
            errors.append(f"{src}:\n{out}")
        objs.append(obj)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
