"""Build the HIP selection library (libdsai.so) in-tree for gfx950.

Usage: python -m sparse_attention_token_index_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsai.so")

SOURCES = ["api.cpp", "score_topk.hip", "score_at.hip", "sort_rows.hip", "pooled.hip", "k_norm.hip",
           "indexer_bwd.hip"]

# Packed-fp32 VALU forms are kept out of the device code: plain fp32 ops only.
# No value the kernels handle is ever NaN (finite inputs; -inf only as padding),
# so NaN-preserving canonicalization (an extra VALU op per ReLU) is dropped.
HIP_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-honor-nans", "-Wall", "-Wno-unused-function",
             # matrix-core results in ordinary VGPRs: the epilogue reads them
             # directly instead of copying each accumulator out of AGPRs
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libdsai.so)")


def build(verbose: bool = False, out: str = LIB) -> str:
    """Compile every source into `out`; always recompiles."""
    cc = hipcc()
    objs = []
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for src, p in procs:
        text = p.communicate()[0].decode(errors="replace")
        # the host pass does not know the packed-fp32 feature name: harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errors.append(f"{src}:\n{text}")
        elif verbose and text.strip():
            print(text)
    if errors:
        raise RuntimeError("HIP build failed:\n" + "\n".join(errors))
    tmp = out + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
