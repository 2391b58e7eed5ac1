"""The timed fold entry (detfold_fold_ranks_timed, through the C ABI): the
same bits as the oracle, and a kernel duration, recorded by the fold's own
dispatch, that lies inside an event pair recorded around the call."""
import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W,n,off,inv_w", [(8, 1 << 20, 0, None), (16, 100_003, 1, None),
                                           (4, 1_000_001, 2, 0.25), (1, 4099, 3, None),
                                           (33, 70_001, 1, None)])
def test_timed_fold_bits_and_duration(detfold_lib, W, n, off, inv_w):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    print("case: timed fold W=%d n=%d offset=%d scaled=%s" % (W, n, off, inv_w is not None), flush=True)
    host = fold_inputs.slots("varied", W, n, 7100 + W, spread=3.0)
    alloc = torch.empty(W * n + off, dtype=torch.float32, device=dev)
    stacked = alloc[off:].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        df.fold_ranks_timed(out, stacked, torch.cuda.Event(enable_timing=True), ev[1])  # never recorded
    for _ in range(3):
        ev[0].record(stream)
        df.fold_ranks_timed(out, stacked, ev[2], ev[3], scaled=inv_w is not None,
                            inv_w=inv_w if inv_w is not None else 1.0)
        ev[1].record(stream)
        ev[1].synchronize()
        outer, inner = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
        assert 0.0 < inner <= outer * 1.01 + 0.002, (inner, outer)
    want = oracle.fold_stacked(host) if inv_w is None else oracle.fold_stacked_scaled(host, np.float32(inv_w))
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_timed_fold_without_events_and_empty(detfold_lib):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    host = fold_inputs.slots("vecf", 3, 1027, 7200)
    stacked = torch.from_numpy(host).to(dev)
    out = torch.empty(1027, dtype=torch.float32, device=dev)
    df.fold_ranks_timed(out, stacked, None, None)          # no events: a plain fold
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.fold_stacked(host).view(np.uint32))
    empty = torch.empty((3, 0), dtype=torch.float32, device=dev)
    df.fold_ranks_timed(torch.empty(0, dtype=torch.float32, device=dev), empty, None, None)
    torch.cuda.synchronize()
