"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; the device code is built as usual, the sanitizers apply to the host
side alone).  tests/c/abi_fuzz.c drives every planning and argument-checking
path with extreme widths, lengths, addresses and launch overrides, checks the
invariants of every accepted plan, and never reaches the device."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    from deterministic_fixed_order_amd import _build

    lib = str(tmp_path / "libdetfold_san.so")
    extra = []
    for f in HOST_SAN:
        extra += ["-Xarch_host", f]  # host pass only: no sanitizer in the gfx950 code
    _build.build_library(lib, extra=extra)
    exe = str(tmp_path / "abi_fuzz")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    subprocess.run([clang, "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror"] + HOST_SAN +
                   ["-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_fuzz.c"),
                    "-o", exe, lib, "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-6000:]
    assert "violations 0" in res.stdout, res.stdout[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-6000:]
