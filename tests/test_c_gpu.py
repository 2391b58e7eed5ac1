"""The library from C on a GPU, without Python or torch in the caller:
tests/c/fold_gpu (built by the repository's build step) allocates device
memory with hipMalloc, calls fold_ranks, fold_ranks_scaled, fold_into,
fold_slots, detfold_loopback_round and both two-rank links through
include/detfold.h, and compares every result with the CPU oracle bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "fold_gpu")


def test_c_caller_on_the_device(detfold_lib):
    assert os.path.exists(EXE), "tests/c/fold_gpu is not built; __graft_entry__.build() builds it"
    print("case: tests/c/fold_gpu", flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(res.stdout[-4000:], flush=True)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    lines = res.stdout.splitlines()
    assert lines[-1] == "all ok"
    cases = [l[5:] for l in lines if l.startswith("case ")]
    oks = [l[3:] for l in lines if l.startswith("ok ")]
    assert len(cases) == 15 and not any(l.startswith("FAIL") for l in lines)
    for name in cases:
        if name not in ("pair link all-reduce", "one-shot all-reduce"):
            assert name in oks, name
