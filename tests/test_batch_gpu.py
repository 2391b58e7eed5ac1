"""The batched fold (fold_ranks_batch / fold_ranks_batch_scaled, through the C
ABI) against the CPU oracle, bit for bit.

* the owner-shard dataflow of mamba-rs src/dist/reducer.rs
  (reduce_sum_fixed_order_nccl, LoopbackWorld::run_round) on one device: the
  W=16 arena of 10,000,019 floats starting one element past an aligned
  allocation, its 16 owner shards gathered by device copies (ascending and
  reversed delivery) into per-owner [16][l_p] scratch, all 16 shard folds in
  one launch into one output at the owners' offsets -- equal to the whole
  fold and to the oracle;
* mixed batches: up to DETFOLD_MAX_JOBS jobs of one width with ragged and
  empty lengths, outputs and arenas at every 16-byte phase, unscaled and
  scaled, and the widths that run one launch per job (W = 1, W > 16).
"""
import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_owner_shards_in_one_launch_equal_the_whole_fold(detfold_lib):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    W, n = 16, 10_000_019
    print("case: W=16 len=%d at base+1, 16 owner shards in one batched launch" % n, flush=True)
    host = fold_inputs.slots("vecf", W, n, 3000)
    want = oracle.fold_stacked(host)
    alloc = torch.empty(W * n + 1, dtype=torch.float32, device=dev)
    stacked = alloc[1:].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    shards = df.shard_plan(n, W)
    for reverse in (False, True):
        scratch = []
        for s, ln in shards:
            sc = torch.empty((W, ln), dtype=torch.float32, device=dev)
            for src in (range(W - 1, -1, -1) if reverse else range(W)):
                sc[src].copy_(stacked[src, s:s + ln])
            scratch.append(sc)
        out = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
        df.fold_ranks_batch([out[s:s + ln] for s, ln in shards], scratch)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out.cpu().numpy()), _bits(want)), "reverse=%s" % reverse
        del scratch
    whole = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(whole, stacked)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(whole.cpu().numpy()), _bits(want))


LENS = [0, 1, 2, 3, 4, 5, 7, 64, 255, 256, 257, 1000, 4099, 65539, 100_003, 0, 12_345, 3]


@pytest.mark.parametrize("W", [2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("scaled", [False, True])
def test_mixed_batches(detfold_lib, W, scaled):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1000 * W + scaled)
    count = df.MAX_JOBS if W in (3, 8) else len(LENS)
    lens = [LENS[j % len(LENS)] for j in range(count)]
    print("case: batch W=%d scaled=%s jobs=%d" % (W, scaled, count), flush=True)
    outs, arenas, hosts, bufs = [], [], [], []
    for j, ln in enumerate(lens):
        host = fold_inputs.slots("varied", W, ln, 5000 + 37 * j + W, spread=float(1 + j % 5))
        o_off, a_off = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        ob = torch.full((ln + o_off,), float("nan"), dtype=torch.float32, device=dev)
        ab = torch.empty(W * ln + a_off, dtype=torch.float32, device=dev)
        st = ab[a_off:].view(W, ln)
        st.copy_(torch.from_numpy(host))
        outs.append(ob[o_off:])
        arenas.append(st)
        hosts.append(host)
        bufs += [ob, ab]
    inv_w = 1.0 / W if scaled else None
    df.fold_ranks_batch(outs, arenas, inv_w=inv_w)
    torch.cuda.synchronize()
    for j, (o, host) in enumerate(zip(outs, hosts)):
        want = oracle.fold_stacked(host) if not scaled else oracle.fold_stacked_scaled(host, np.float32(inv_w))
        assert np.array_equal(_bits(o.cpu().numpy()), _bits(want)), "job %d len %d" % (j, lens[j])


@pytest.mark.parametrize("W", [1, 17, 33])
def test_batches_of_widths_with_one_launch_per_job(detfold_lib, W):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    print("case: batch W=%d (one launch per job)" % W, flush=True)
    lens = [1, 4099, 0, 70_001, 5]
    outs, arenas, hosts = [], [], []
    for j, ln in enumerate(lens):
        host = fold_inputs.slots("varied", W, ln, 6100 + j, spread=2.0)
        alloc = torch.empty(W * ln + 1, dtype=torch.float32, device=dev)
        st = alloc[j % 2:j % 2 + W * ln].view(W, ln)
        st.copy_(torch.from_numpy(host))
        outs.append(torch.empty(ln, dtype=torch.float32, device=dev))
        arenas.append(st)
        hosts.append(host)
    df.fold_ranks_batch(outs, arenas)
    torch.cuda.synchronize()
    for o, host in zip(outs, hosts):
        assert np.array_equal(_bits(o.cpu().numpy()), _bits(oracle.fold_stacked(host)))


def test_adjacent_outputs_in_one_buffer_and_shared_arena(detfold_lib):
    # jobs writing neighbouring ranges of one output (ragged starts), all
    # reading one arena: every range must hold its own fold, nothing more
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    W, n = 6, 50_001
    host = fold_inputs.slots("mixed", W, n, 6300)
    st = torch.from_numpy(host).to(dev)
    cuts = [0, 1, 2, 5, 4099, 4100, 30_000, n]
    out = torch.full((len(cuts) - 1, n), float("nan"), dtype=torch.float32, device=dev)
    flat = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    # the same arena, folded whole into every row of `out`
    df.fold_ranks_batch([out[r] for r in range(len(cuts) - 1)], [st] * (len(cuts) - 1))
    # and piecewise into `flat`: job k writes [cuts[k], cuts[k+1]) from a contiguous copy of that piece
    pieces = [st[:, a:b].contiguous() for a, b in zip(cuts, cuts[1:])]
    df.fold_ranks_batch([flat[a:b] for a, b in zip(cuts, cuts[1:])], pieces)
    torch.cuda.synchronize()
    want = oracle.fold_stacked(host)
    for r in range(len(cuts) - 1):
        assert np.array_equal(_bits(out[r].cpu().numpy()), _bits(want)), r
    assert np.array_equal(_bits(flat.cpu().numpy()), _bits(want))


@pytest.mark.parametrize("W,pad", [(2, 3), (5, 1024), (8, 1 << 20), (16, 7), (16, (1 << 22) - 625_002)])
def test_padded_slots_give_the_bits_of_a_packed_arena(detfold_lib, W, pad):
    # each job's slots sit len + pad floats apart (a receive buffer with
    # padded slots): the bits must be those of the packed fold
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    lens = [625_002, 1, 4099, 0, 77_777] if W == 16 else [1000, 3, 65_539, 12_345]
    print("case: padded batch W=%d pad=%d" % (W, pad), flush=True)
    outs, views, hosts, bufs = [], [], [], []
    for j, ln in enumerate(lens):
        pitch = ln + pad
        host = fold_inputs.slots("varied", W, ln, 6500 + j + W, spread=3.0)
        off = j % 4
        buf = torch.full((W * pitch + off,), float("nan"), dtype=torch.float32, device=dev)
        view = buf[off:off + W * pitch].view(W, pitch)[:, :ln]
        view.copy_(torch.from_numpy(host))
        o = torch.full((ln,), float("nan"), dtype=torch.float32, device=dev)
        outs.append(o)
        views.append(view)
        hosts.append(host)
        bufs.append(buf)
    for inv_w in (None, 1.0 / W):
        df.fold_ranks_batch(outs, views, inv_w=inv_w)
        torch.cuda.synchronize()
        for j, (o, host) in enumerate(zip(outs, hosts)):
            want = oracle.fold_stacked(host) if inv_w is None else oracle.fold_stacked_scaled(host, np.float32(inv_w))
            assert np.array_equal(_bits(o.cpu().numpy()), _bits(want)), "job %d len %d" % (j, lens[j])


@pytest.mark.parametrize("W", [1, 17])
def test_padded_slots_with_one_launch_per_job(detfold_lib, W):
    import torch
    df = detfold_lib
    dev = torch.device("cuda:0")
    print("case: padded batch W=%d (one launch per job)" % W, flush=True)
    lens, pad = [5, 70_001, 4096], 13
    outs, views, hosts = [], [], []
    for j, ln in enumerate(lens):
        host = fold_inputs.slots("varied", W, ln, 6600 + j, spread=2.0)
        buf = torch.empty(W * (ln + pad) + 1, dtype=torch.float32, device=dev)
        view = buf[1:1 + W * (ln + pad)].view(W, ln + pad)[:, :ln]
        view.copy_(torch.from_numpy(host))
        outs.append(torch.empty(ln, dtype=torch.float32, device=dev))
        views.append(view)
        hosts.append(host)
    df.fold_ranks_batch(outs, views)
    torch.cuda.synchronize()
    for o, host in zip(outs, hosts):
        assert np.array_equal(_bits(o.cpu().numpy()), _bits(oracle.fold_stacked(host)))
