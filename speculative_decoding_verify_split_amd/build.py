"""Build librapid_verify.so for gfx950 with hipcc (in-tree).

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
generation disabled; the host-only validation unit is compiled by the same
driver.  Objects are built in parallel and linked into one shared library
next to this file.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librapid_verify.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["rv_validate.cpp", "attn_prefix.hip", "attn_block.hip", "lse_merge.hip",
           "attn_window.hip", "rapid_accept.hip", "rapid_tree.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + INCLUDE, "-I" + CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The history pass takes row maxima of MFMA scores with fmaxf; allowing the
# compiler to assume no NaN drops the quieting v_max that IEEE mode puts in
# front of every such max (a third of the softmax's VALU work).  The kernels
# compare only against -inf, never against NaN.
PER_SOURCE = {"attn_prefix.hip": ["-fno-honor-nans"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip"] + DEVICE + COMMON + PER_SOURCE.get(src, []) + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++"] + COMMON + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
