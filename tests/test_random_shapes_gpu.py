"""GPU parity over seeded random shapes: every fold entry point against the
CPU oracle, bit for bit, on shapes drawn from a fixed-seed generator instead
of a hand-picked grid.

Each case draws a width, a length, the 16-byte phases of the output and of
the inputs, an input family and (for the stacked fold) the scale, so that the
plan's choices -- LDS row body with one or two slots per wave, the wide
row body's two pass shapes, the direct bodies, head and tail lengths, one-pass
grids of every size -- are crossed with each other far more often than a grid
would.  Widths reach 70 (five passes of the wide row body), lengths reach
70,000 with a ragged tail; the shapes are printed before each launch.
"""
import sys

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu

FAMILIES = ("vecf", "varied", "mixed")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _assert_bits(got, want, what):
    g, w = _bits(got), _bits(want)
    bad = np.flatnonzero(g != w)
    if bad.size:
        i = int(bad[0])
        raise AssertionError("%s: %d of %d words differ; first at %d: got %08x want %08x"
                             % (what, bad.size, g.size, i, g[i], w[i]))


@pytest.fixture(scope="module")
def env(detfold_lib):
    import torch
    torch.cuda.init()
    return detfold_lib, torch, torch.device("cuda:0")


def _length(rng):
    """Mostly small and ragged; one case in four spans several hundred tiles."""
    if rng.random() < 0.25:
        return int(rng.integers(20_000, 70_001))
    return int(rng.integers(0, 3_000))


def _host_slots(rng, W, n, seed):
    fam = FAMILIES[int(rng.integers(0, len(FAMILIES)))]
    return fam, fold_inputs.slots(fam, W, n, seed, spread=4.0)


@pytest.mark.parametrize("block", range(6))
def test_stacked_folds_on_random_shapes(env, block):
    df, torch, dev = env
    rng = np.random.default_rng(9100 + block)
    for case in range(25):
        W = int(rng.choice([1, 2, 3, 4, 5, 8, 8, 12, 16, 16, 17, 24, 33, 70]))
        n = _length(rng)
        out_off, in_off = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        fam, host = _host_slots(rng, W, n, 40_000 + 100 * block + case)
        scaled = bool(rng.random() < 0.3)
        inv_w = np.float32(1.0 / W) if scaled else None
        what = ("block %d case %d: W=%d n=%d out+%d in+%d %s%s"
                % (block, case, W, n, out_off, in_off, fam, " scaled 1/%d" % W if scaled else ""))
        _say(what)
        in_alloc = torch.empty(W * n + 4, dtype=torch.float32, device=dev)
        stacked = in_alloc[in_off:in_off + W * n].view(W, n)
        stacked.copy_(torch.from_numpy(host))
        out_alloc = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
        out = out_alloc[out_off:out_off + n]
        if scaled:
            df.fold_ranks_scaled(out, stacked, float(inv_w))
            want = oracle.fold_stacked_scaled(host, inv_w)
        else:
            df.fold_ranks(out, stacked)
            want = oracle.fold_stacked(host)
        torch.cuda.synchronize()
        full = out_alloc.cpu().numpy()
        _assert_bits(full[out_off:out_off + n], want, what)
        assert np.isnan(full[:out_off]).all() and np.isnan(full[out_off + n:]).all(), what


@pytest.mark.parametrize("block", range(4))
def test_separate_slot_folds_on_random_shapes(env, block):
    df, torch, dev = env
    rng = np.random.default_rng(9200 + block)
    for case in range(25):
        W = int(rng.integers(1, 17))
        n = _length(rng)
        fam, host = _host_slots(rng, W, n, 50_000 + 100 * block + case)
        offs = [int(rng.integers(0, 4)) for _ in range(W)]
        in_place = W >= 2 and rng.random() < 0.4
        me = int(rng.integers(0, W))
        what = ("block %d case %d: W=%d n=%d %s slot offsets %s%s"
                % (block, case, W, n, fam, offs, " in place on slot %d" % me if in_place else ""))
        _say(what)
        allocs = [torch.empty(n + 4, dtype=torch.float32, device=dev) for _ in range(W)]
        slots = [a[o:o + n] for a, o in zip(allocs, offs)]
        for r in range(W):
            slots[r].copy_(torch.from_numpy(host[r]))
        out = slots[me] if in_place else torch.empty(n, dtype=torch.float32, device=dev)
        df.fold_slots(out, slots)
        torch.cuda.synchronize()
        _assert_bits(out.cpu().numpy(), oracle.fold_stacked(host), what)


def test_in_place_folds_on_random_shapes(env):
    df, torch, dev = env
    rng = np.random.default_rng(9300)
    for case in range(60):
        n = _length(rng)
        d_off, s_off = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        fam, host = _host_slots(rng, 2, n, 60_000 + case)
        what = "case %d: fold_into n=%d dst+%d stage+%d %s" % (case, n, d_off, s_off, fam)
        _say(what)
        da = torch.empty(n + 4, dtype=torch.float32, device=dev)
        sa = torch.empty(n + 4, dtype=torch.float32, device=dev)
        dst, stage = da[d_off:d_off + n], sa[s_off:s_off + n]
        dst.copy_(torch.from_numpy(host[0]))
        stage.copy_(torch.from_numpy(host[1]))
        df.fold_into(dst, stage)
        torch.cuda.synchronize()
        _assert_bits(dst.cpu().numpy(), oracle.fold_into(host[0], host[1]), what)


def test_concurrent_folds_on_four_streams(env):
    # forty folds of random shapes queued on four streams with no host
    # synchronization between them (stacked, separate-slot and in-place
    # entry points mixed), so that kernels of different shapes run side by
    # side; every output must still equal its oracle fold
    df, torch, dev = env
    rng = np.random.default_rng(9400)
    streams = [torch.cuda.Stream(device=dev) for _ in range(4)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream(dev))
    jobs = []
    for case in range(40):
        kind = ("stacked", "slots", "into")[case % 3]
        W = 2 if kind == "into" else int(rng.choice([2, 3, 5, 8, 12, 16, 20]))
        if kind == "slots":
            W = min(W, 16)
        n = int(rng.integers(1, 200_000))
        fam, host = _host_slots(rng, W, n, 70_000 + case)
        off = int(rng.integers(0, 4))
        st = streams[case % 4]
        with torch.cuda.stream(st):
            if kind == "stacked":
                alloc = torch.empty(W * n + 4, dtype=torch.float32, device=dev)
                stacked = alloc[off:off + W * n].view(W, n)
                stacked.copy_(torch.from_numpy(host), non_blocking=False)
                out = torch.empty(n, dtype=torch.float32, device=dev)
                df.fold_ranks(out, stacked)
                jobs.append((out, oracle.fold_stacked(host), "stacked W=%d n=%d +%d" % (W, n, off), alloc))
            elif kind == "slots":
                slots = [torch.from_numpy(host[r]).to(dev) for r in range(W)]
                out = torch.empty(n, dtype=torch.float32, device=dev)
                df.fold_slots(out, slots)
                jobs.append((out, oracle.fold_stacked(host), "slots W=%d n=%d" % (W, n), slots))
            else:
                dst = torch.from_numpy(host[0]).to(dev)
                stage = torch.from_numpy(host[1]).to(dev)
                df.fold_into(dst, stage)
                jobs.append((dst, oracle.fold_into(host[0], host[1]), "into n=%d" % n, stage))
    _say("case: 40 folds on 4 streams queued")
    torch.cuda.synchronize()
    for out, want, what, _keep in jobs:
        _assert_bits(out.cpu().numpy(), want, what)
