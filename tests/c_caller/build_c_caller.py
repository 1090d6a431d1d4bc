"""Builds tests/c_caller/libverify_step_c.so: the plain-C verify step
(verify_step.c), linked against the in-tree librapid_verify.so and the HIP
runtime.  Test infrastructure: only the GPU test that drives the library
from C loads it.  Host code only, compiled with gcc."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "libverify_step_c.so")


def build(rocm="/opt/rocm"):
    libdir = os.path.join(ROOT, "speculative_decoding_verify_split_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "verify_step.c"),
           "-o", OUT, "-L", libdir, "-lrapid_verify", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C caller failed:\n" + res.stderr)
    return OUT


if __name__ == "__main__":
    print(build())
