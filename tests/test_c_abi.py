"""The C ABI from C: tests/c/abi_smoke.c is compiled as C99 with gcc against
include/detfold.h, linked to libdetfold.so, and run (CPU only; the program
makes no device call)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_caller(tmp_path, detfold_lib):
    lib_dir = os.path.dirname(detfold_lib.LIB_PATH)
    exe = str(tmp_path / "abi_smoke")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_smoke.c"),
                    "-o", exe, "-L", lib_dir, "-l:libdetfold.so", "-Wl,-rpath," + lib_dir,
                    "-Wl,-rpath," + rocm_lib], check=True)
    res = subprocess.run([exe], check=True, capture_output=True, text=True)
    lines = dict(l.split(" ", 1) for l in res.stdout.strip().splitlines())
    assert lines["abi"] == str(detfold_lib.ABI_VERSION)
    assert lines["w0"] == str(detfold_lib.EINVAL)
    assert lines["overlap"] == str(detfold_lib.EOVERLAP)
    assert lines["empty"] == str(detfold_lib.OK)
    assert lines["timed_w0"] == str(detfold_lib.EINVAL)
    assert lines["timed_overlap"] == str(detfold_lib.EOVERLAP)
    assert lines["timed_empty"] == str(detfold_lib.OK)
    assert "overlap" in lines["strerror"]
    assert lines["shards"] == "0 4 3 3"
    assert lines["plan"] == "0 %d 512 32768 128" % detfold_lib.PATH_ROWS
    assert lines["shot_noflags"] == str(detfold_lib.EINVAL)
    assert lines["shot_capacity"] == str(detfold_lib.EINVAL)
    assert lines["shot_rank"] == str(detfold_lib.EINVAL)
    assert lines["shot_empty"] == str(detfold_lib.OK)
    assert lines["shot_words"] == "256 40043 40044"
    assert lines["bcast_noevents"] == str(detfold_lib.EINVAL)
    assert lines["gather_noevents"] == str(detfold_lib.EINVAL)
