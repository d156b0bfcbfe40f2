"""Build libasv.so (HIP kernels for gfx950 + the host table builder) in-tree.

Run as ``python -m attention_stream_verify_amd.build``; ``__graft_entry__.build``
calls ``build()``. Every call recompiles every source.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libasv.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIP_SOURCES = ["argmax.hip", "conv.hip", "attn.hip", "merge.hip", "draft.hip", "markov.hip", "qk.hip", "upload.hip"]
CXX_SOURCES = ["table.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-ffp-contract=off",
    # packed fp32 arithmetic stays off: the compiler must not form v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libasv.so")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in HIP_SOURCES + CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "c++"]
        flags = HIPCC_FLAGS if src.endswith(".hip") else ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Werror"]
        cmd = [cc, *flags, "-I", INCLUDE, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
