"""Build step for tests/c/fold_gpu: the C caller of libdetfold that runs on a
GPU (tests/test_c_gpu.py).  gcc, C99, linked to the in-tree libdetfold.so, the
oracle's liboracle.so and the HIP runtime; run by __graft_entry__.build() after
both libraries are built, so that no test compiles anything."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fold_gpu.c")
EXE = os.path.join(HERE, "fold_gpu")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "deterministic_fixed_order_amd"), "-l:libdetfold.so",
           "-L", os.path.join(ROOT, "oracle"), "-l:liboracle.so",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../deterministic_fixed_order_amd:$ORIGIN/../../oracle:"
           + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
