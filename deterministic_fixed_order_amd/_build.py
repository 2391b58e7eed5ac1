"""Build step for ``libdetfold.so`` (hipcc, gfx950 only).

Sources (``csrc/``): fold_kernels.hip (device code and its launches), plan.cpp
(host-only planning and argument checks), detfold.cpp (call sequences and the
C ABI), internal.h (their shared declarations).  exports.map limits the
exported symbols to the C ABI of include/detfold.h.

Flags that fix the fold's bits:
  -ffp-contract=off                 no fused multiply-add anywhere
  -fno-fast-math                    no reassociation of the add chain
  -fno-gpu-flush-denormals-to-zero  binary32 subnormals kept (the gfx9 default, stated)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed FP32 instructions; every add is a
                                    plain v_add_f32
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("fold_kernels.hip", "plan.cpp", "detfold.cpp")]
EXPORTS_MAP = os.path.join(CSRC, "exports.map")
HEADER = os.path.join(ROOT, "include", "detfold.h")
LIB = os.path.join(PKG, "libdetfold.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wl,--version-script=" + EXPORTS_MAP,
    ]


def build_library(out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile the sources into ``out`` (atomically replaced)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + (extra or []) + ["-o", tmp] + SOURCES
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def save_temps(outdir: str) -> None:
    """Keep the gfx950 assembly of the library's sources (for reading our own ISA)."""
    os.makedirs(outdir, exist_ok=True)
    cmd = [hipcc()] + flags() + ["-save-temps=obj", "-o", os.path.join(outdir, "libdetfold.so")] + SOURCES
    subprocess.run(cmd, check=True, cwd=outdir)


if __name__ == "__main__":
    print(build_library())
