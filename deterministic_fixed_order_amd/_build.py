"""Build step for ``libdetfold.so`` (hipcc, gfx950 only).

Sources (``csrc/``): fold_kernels.hip (device code and its launches), plan.cpp
(host-only planning and argument checks), detfold.cpp (call sequences and the
C ABI), internal.h (their shared declarations).  exports.map limits the
exported symbols to the C ABI of include/detfold.h.

fold_kernels.hip is compiled in two passes, so that device-only flags reach
the device compiler only: the device pass writes the gfx950 code object
bundle, and the host pass embeds it (clang's ``-fcuda-include-gpubinary``,
the step the one-command HIP build performs internally).  Both passes share
one compilation-unit id, so host and device agree on the names of any
``__device__`` variable.  plan.cpp and detfold.cpp hold no device code.

Flags that fix the fold's bits:
  -ffp-contract=off                 no fused multiply-add anywhere
  -fno-fast-math                    no reassociation of the add chain
  -fno-gpu-flush-denormals-to-zero  binary32 subnormals kept (the gfx9 default,
                                    stated; device pass)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed FP32 instructions; every add is a
                                    plain v_add_f32 (device pass)

``source_digest()`` is the sha256 of every input of the build (sources,
header, export map and the flags); ``build_library`` writes it beside the
library, and ``is_current()`` compares it, so that a library built from
other sources is rebuilt rather than run.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
KERNELS = os.path.join(CSRC, "fold_kernels.hip")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("plan.cpp", "detfold.cpp")]
SOURCES = [KERNELS] + HOST_SOURCES
INTERNAL_HEADER = os.path.join(CSRC, "internal.h")
EXPORTS_MAP = os.path.join(CSRC, "exports.map")
HEADER = os.path.join(ROOT, "include", "detfold.h")
LIB = os.path.join(PKG, "libdetfold.so")
DIGEST = LIB + ".sha256"
ARCH = "gfx950"
CUID = "detfold_fold_kernels"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def common_flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def device_flags() -> list[str]:
    return ["-fno-gpu-flush-denormals-to-zero",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def link_flags() -> list[str]:
    return ["--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--version-script=" + EXPORTS_MAP]


def source_digest() -> str:
    h = hashlib.sha256()
    for path in SOURCES + [INTERNAL_HEADER, EXPORTS_MAP, HEADER]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read() + b"\0")
    h.update("\0".join(common_flags() + device_flags() + link_flags()).encode())
    return h.hexdigest()


def is_current(lib: str = LIB) -> bool:
    """Whether ``lib`` exists and was built from the sources as they are now."""
    try:
        with open(lib + ".sha256") as f:
            return os.path.exists(lib) and f.read().strip() == source_digest()
    except OSError:
        return False


def _run(cmd: list[str], cwd: str | None = None) -> None:
    subprocess.run(cmd, check=True, cwd=cwd)


def _device_pass(work: str, extra: list[str], temps: bool = False) -> str:
    bundle = os.path.join(work, "fold_kernels.hipfb")
    cmd = [hipcc(), "--cuda-device-only", "-cuid=" + CUID] + common_flags() + device_flags() + extra
    if temps:
        cmd.append("-save-temps=obj")
    _run(cmd + ["-c", KERNELS, "-o", bundle], cwd=work)
    return bundle


def _objects(work: str, extra: list[str]) -> list[str]:
    bundle = _device_pass(work, extra)
    kobj = os.path.join(work, "fold_kernels.o")
    _run([hipcc(), "--cuda-host-only", "-cuid=" + CUID] + common_flags() + extra +
         ["-Xclang", "-fcuda-include-gpubinary", "-Xclang", bundle, "-c", KERNELS, "-o", kobj])
    objs = [kobj]
    for src in HOST_SOURCES:
        obj = os.path.join(work, os.path.splitext(os.path.basename(src))[0] + ".o")
        _run([hipcc()] + common_flags() + extra + ["-c", src, "-o", obj])
        objs.append(obj)
    return objs


def build_library(out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile the sources into ``out`` (atomically replaced) and record the
    source digest beside it (only for the default flags)."""
    extra = extra or []
    work = tempfile.mkdtemp(prefix="detfold_build_")
    try:
        objs = _objects(work, extra)
        tmp = out + ".tmp%d" % os.getpid()
        _run([hipcc()] + link_flags() + ["-o", tmp] + objs)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    digest = out + ".sha256"
    if extra:
        if os.path.exists(digest):
            os.remove(digest)
    else:
        with open(digest, "w") as f:
            f.write(source_digest() + "\n")
    return out


def save_temps(outdir: str) -> None:
    """Keep the gfx950 assembly of the device pass (for reading our own ISA)."""
    os.makedirs(outdir, exist_ok=True)
    _device_pass(outdir, [], temps=True)


if __name__ == "__main__":
    print(build_library())
