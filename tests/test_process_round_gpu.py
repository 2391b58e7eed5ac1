"""Ranks as processes on one GPU (mamba-rs src/dist/reducer.rs: the owner-shard
dataflow of reduce_sum_fixed_order_nccl, with the process boundary the
transport path has; memra-engine tests/tp_ar_gpu.rs: the one-shot arm, one
kernel per rank).

Each of W processes (W = 2 or 4) is a rank owning one arena; the arenas are
shared between the processes through device memory handles (torch's IPC
sharing of device tensors).  Rank r folds its owner shard in place, reading the other ranks' arenas
directly through the mapped handles (fold_slots over [arena_0, ...] at the
shard), then writes its reduced shard into the other ranks' arenas.  A CPU barrier
(gloo, host-side only) separates the phases.  Every arena must end equal to the
oracle's fold of the original arenas, bit for bit.

The fused test has every rank run the one-kernel fold-and-write-back round
over its own shard of all the arenas at once, reading and writing the other
ranks' arenas through the mapped handles.

The one-shot test gives each of two processes its own rank's one-shot kernel
(detfold_one_shot_rank); the staging buffers, barrier counters and refusal
words are shared the same way, and the two kernels meet only through those
counters.  Three rounds must double the sum twice, with both words zero.

The shared tensors reach each child inside a one-element list that the child
empties, so that its last reference to them is its own and it can drop them
before it exits: the parent's record of what it shared is then released
before the parent ends.
"""
import os
import socket

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu


def _free_port():
    with socket.socket(socket.AF_INET, socket.SOCK_STREAM) as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _release_shared():
    """Free the mapped tensors a child dropped, while its device context lives."""
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.ipc_collect()


def _rank_main(rank, box, n, port, world):
    import sys
    import torch
    import torch.distributed as dist
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import deterministic_fixed_order_amd as df

    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    arenas = box.pop()
    try:
        torch.cuda.set_device(0)
        start, length = df.shard_plan(n, world)[rank]
        mine = arenas[rank]
        if length:
            # phase A: fold my owner shard from every rank's arena, in place
            df.fold_slots(mine[start:start + length], [a[start:start + length] for a in arenas])
        torch.cuda.synchronize()
        dist.barrier()
        # phase B: my reduced shard goes into every other rank's arena (byte movement)
        if length:
            for p, a in enumerate(arenas):
                if p != rank:
                    a[start:start + length].copy_(mine[start:start + length])
        torch.cuda.synchronize()
        dist.barrier()
    finally:
        arenas = mine = a = None  # this child's last references to the shared arenas
        _release_shared()
        dist.destroy_process_group()


@pytest.mark.parametrize("world,n", [(2, 1), (2, 1001), (2, 1 << 20), (4, 3), (4, 1 << 20)])
def test_processes_fold_through_shared_arenas(detfold_lib, world, n):
    import torch
    import torch.multiprocessing as mp

    host = fold_inputs.slots("varied", world, n, 8800 + n, spread=2.0)
    want = oracle.fold_stacked(host)
    dev = torch.device("cuda:0")
    arenas = [torch.from_numpy(host[r]).to(dev) for r in range(world)]
    torch.cuda.synchronize()
    print("case: %d processes, n=%d" % (world, n), flush=True)
    mp.spawn(_rank_main, args=([arenas], n, _free_port(), world), nprocs=world, join=True)
    torch.cuda.ipc_collect()  # release the handles the children held
    for r in range(world):
        got = arenas[r].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "arena %d, n=%d" % (r, n)


def _fused_rank_main(rank, box, n, port, world):
    import sys
    import torch
    import torch.distributed as dist
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import deterministic_fixed_order_amd as df

    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    arenas = box.pop()
    try:
        torch.cuda.set_device(0)
        start, length = df.shard_plan(n, world)[rank]
        dist.barrier()
        if length:
            # one kernel: my shard of every rank's arena, folded and written back to all of them
            df.loopback_round([a[start:start + length] for a in arenas], fused=True)
        torch.cuda.synchronize()
        dist.barrier()
    finally:
        arenas = None
        _release_shared()
        dist.destroy_process_group()


@pytest.mark.parametrize("world,n", [(2, 1001), (4, 3), (4, 1 << 20)])
def test_processes_fused_round_through_shared_arenas(detfold_lib, world, n):
    # The one-sided shape of the sharded round: every rank runs the fused
    # fold-and-write-back kernel over its own shard of all the arenas, reading
    # and writing the other ranks' arenas through the mapped handles, all
    # ranks at once (the shards are disjoint).  Every arena must end equal to
    # the oracle's fold.
    import torch
    import torch.multiprocessing as mp

    host = fold_inputs.slots("varied", world, n, 8900 + n, spread=2.0)
    want = oracle.fold_stacked(host)
    dev = torch.device("cuda:0")
    arenas = [torch.from_numpy(host[r]).to(dev) for r in range(world)]
    torch.cuda.synchronize()
    print("case: fused round in %d processes, n=%d" % (world, n), flush=True)
    mp.spawn(_fused_rank_main, args=([arenas], n, _free_port(), world), nprocs=world, join=True)
    torch.cuda.ipc_collect()
    for r in range(world):
        got = arenas[r].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "arena %d, n=%d" % (r, n)


def _one_shot_rank_main(rank, box, n, rounds, port, world):
    import sys
    import torch
    import torch.distributed as dist
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import deterministic_fixed_order_amd as df

    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    xs, buffers = box.pop()
    link = None
    try:
        torch.cuda.set_device(0)
        link = df.OneShotLink(n, device="cuda:0", buffers=buffers, init=False)
        # load the library's code object before the first barrier, so the
        # peer's kernel never waits through this process's first launch
        warm = torch.zeros(8, device="cuda:0")
        df.fold_into(warm[:4], warm[4:])
        torch.cuda.synchronize()
        for _ in range(rounds):
            dist.barrier()  # both ranks launch their kernel within moments of each other
            link.rank(rank, xs[rank], stream=link.stream)
            torch.cuda.synchronize()
        dist.barrier()
    finally:
        xs = buffers = link = None
        _release_shared()
        dist.destroy_process_group()


@pytest.mark.parametrize("n", [4096, 65536])
def test_one_shot_ranks_as_processes(detfold_lib, n):
    # The one-shot arm in its per-rank shape: each process launches its own
    # rank's kernel; the stage buffers, the barrier counters and the words are
    # shared through device memory handles.  Every wait in the kernel is
    # bounded, so a late peer can only produce a refusal word, never a hang.
    import torch
    import torch.multiprocessing as mp

    rounds = 3
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    want = oracle.fold_into(ha, hb)
    for _ in range(rounds - 1):
        want = oracle.fold_into(want, want)
    dev = torch.device("cuda:0")
    link = detfold_lib.OneShotLink(n, device=dev)  # zeroes the counters and words
    xs = [torch.from_numpy(ha).to(dev), torch.from_numpy(hb).to(dev)]
    torch.cuda.synchronize()
    print("case: one-shot ranks as 2 processes, n=%d, %d rounds" % (n, rounds), flush=True)
    mp.spawn(_one_shot_rank_main, args=([(xs, (link.stage, link.flags, link.words))], n, rounds,
                                        _free_port(), 2), nprocs=2, join=True)
    torch.cuda.ipc_collect()
    assert link.barrier_words() == [0, 0]
    for r in range(2):
        got = xs[r].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "rank %d, n=%d" % (r, n)
