"""Build libtreeverify.so in-tree with hipcc for gfx950.

Usage: ``python -m tree_attention_draft_amd.build`` (or ``build()`` from Python).  Every
call recompiles.  Objects go to ``_build/`` at the repository root; the shared library to
``tree_attention_draft_amd/libtreeverify.so``.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libtreeverify.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "tree_meta.cpp", "meta_device.hip", "attn_valu.hip", "attn_mfma.hip",
           "attn_mfma_paged.hip", "merge.hip", "accept.hip", "sample.hip", "budget.cpp",
           "static_scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          # packed fp32 instructions are kept out of every kernel on purpose
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function",
          # the direct-load asm clobbers M0 on purpose (the compiler re-sets it before use)
          "-Wno-inline-asm",
          "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build")
    return h


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, err), src in zip(results, SOURCES):
            warnings = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if warnings:
                print(f"[{src}]\n" + "\n".join(warnings))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
