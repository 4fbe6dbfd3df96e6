"""Build libattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc, and the two
measurement programs under microbench/ (LDS access rates of the kernels' tile layouts, sustained
MFMA rate) into microbench/bin/.

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
MICROBENCH = os.path.join(PKG, "microbench")
MICROBENCH_SOURCES = ["lds_banks.hip", "mfma_rate.hip", "valu_rate.hip"]

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


def build_microbench() -> list[str]:
    """Compile the measurement programs (microbench/*.hip) into microbench/bin/."""
    out_dir = os.path.join(MICROBENCH, "bin")
    os.makedirs(out_dir, exist_ok=True)
    jobs = []
    for src in MICROBENCH_SOURCES:
        exe = os.path.join(out_dir, os.path.splitext(src)[0])
        cmd = [HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-Wno-unused-result",
               os.path.join(MICROBENCH, src), "-o", exe]
        jobs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src, exe))
    errors, exes = [], []
    for proc, src, exe in jobs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            errors.append(f"{src}:\n{out}")
        exes.append(exe)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    return exes


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print("\n".join(build_microbench()))
