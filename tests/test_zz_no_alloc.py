"""The no-allocation round entry (detfold_loopback_round_static, through the
C ABI) against the staged round with a caller stage (detfold_loopback_round),
bit for bit on every arena, and both against the CPU oracle's fold.  Three
calls in a row on one device share the library's static stage: the first at
the stage's full size, then two smaller ones (the second in reversed delivery
order), so a call that read what an earlier call left in the stage would show.
"""
import ctypes

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu

CASES = [  # (W, n, flags): W * ceil(n / W) floats of stage each
    (4, 1 << 22, 0),          # exactly the static stage's capacity
    (8, 1_000_003, 1),        # smaller, reversed delivery, ragged shards
    (16, 77, 0),              # tiny: some owners hold 4 elements, some 5
]


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def test_static_round_equals_the_caller_stage_round(detfold_lib):
    import torch
    df = detfold_lib
    lib = df.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    assert CASES[0][0] * -(-CASES[0][1] // CASES[0][0]) == df.STATIC_STAGE_FLOATS
    for W, n, flags in CASES:
        print("case: static-stage round W=%d n=%d flags=%d" % (W, n, flags), flush=True)
        host = fold_inputs.slots("varied", W, n, 9300 + W, spread=4.0)
        want = oracle.fold_stacked(host)
        a = [torch.from_numpy(host[r]).to(dev) for r in range(W)]
        b = [t.clone() for t in a]
        stage = torch.empty(df.round_stage_elems(n, W), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        rc = lib.detfold_loopback_round_static(_ptrs(a), W, n, flags, stream.cuda_stream)
        assert rc == df.OK, df.strerror(rc)
        rc = lib.detfold_loopback_round(_ptrs(b), W, n, stage.data_ptr(), stage.numel(), flags,
                                        stream.cuda_stream)
        assert rc == df.OK, df.strerror(rc)
        torch.cuda.synchronize()
        for r in range(W):
            got_a, got_b = a[r].cpu().numpy(), b[r].cpu().numpy()
            assert np.array_equal(got_a.view(np.uint32), got_b.view(np.uint32)), "arena %d" % r
            assert np.array_equal(got_a.view(np.uint32), want.view(np.uint32)), "arena %d" % r
        del a, b, stage
        torch.cuda.empty_cache()


def test_static_round_refuses_more_than_its_stage(detfold_lib):
    import torch
    df = detfold_lib
    lib = df.load()
    dev = torch.device("cuda:0")
    n = df.STATIC_STAGE_FLOATS + 1
    a = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    assert lib.detfold_loopback_round_static(_ptrs(a), 2, n, 0, None) == df.ESIZE
    with pytest.raises(df.DetfoldError):
        df.loopback_round_static(a)
    torch.cuda.synchronize()
    for t in a:
        assert not bool(t.any())  # nothing ran
