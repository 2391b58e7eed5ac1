"""GPU parity for the fold over separate buffers, the one-GPU reduction round
and the two-stream pair all-reduce (through the C ABI), against the oracle.

* fold_slots: W separate tensors at every 16-byte phase, in place on one of
  them, with repeated slots (mamba-rs src/dist/reducer.rs: the addends of one
  owner shard come from W different arenas).
* loopback_round: W arenas, each owner folds its shard, then distributes it
  (mamba-rs src/dist/reducer.rs, LoopbackWorld::run_round), staged with
  ascending and with reversed delivery order (the `reverse_delivery` flag),
  direct, and fused into one fold-and-write-back kernel; every arena must end
  equal to the oracle's fold of all the arenas, bit for bit.
* pair all-reduce: two streams as two ranks, push into the peer's reused
  staging buffer, event-ordered fold (memra-engine tests/tp_ar_gpu.rs, ArLink
  pipeline arm): sweep n in {1, 4, 1024, 4096, 16384, 65536} and beyond,
  seeds 11+n / 77+n, the repeat call doubling the sum, and the same beside a
  stream kept busy with large folds.
"""
import sys

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu


PAIR_CAPTURE_OFF = ("capturing the pair link into a HIP graph ended the test process with a segmentation "
                    "fault inside hipStreamEndCapture, twice: first with the link's dispatch-recorded "
                    "events under capture, then with plain launches and event records inside the capture "
                    "and no wait on events recorded outside it.  The cause is not known, so the link "
                    "refuses stream capture (DETFOLD_ECAPTURE) and these cases stay off")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env(detfold_lib):
    import torch
    torch.cuda.init()
    return detfold_lib, torch, torch.device("cuda:0")


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _assert_bits(got, want, what):
    g, w = _bits(got), _bits(want)
    assert g.shape == w.shape, what
    bad = g != w
    n_bad = int(np.count_nonzero(bad))
    if n_bad:
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError("%s: %d of %d words differ; first at %d: got %08x want %08x"
                             % (what, n_bad, g.size, i, g.flat[i], w.flat[i]))


def _host(torch, t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _placed(torch, dev, host, offset):
    """A device copy of `host` starting `offset` elements into a fresh allocation."""
    alloc = torch.empty(host.size + 4, dtype=torch.float32, device=dev)
    view = alloc[offset:offset + host.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(host)))
    return view


# --------------------------------------------------------------------------
# fold over separate buffers

@pytest.mark.parametrize("W", [1, 2, 3, 8, 13, 16])
@pytest.mark.parametrize("n", [1, 5, 4096, 70001])
def test_fold_slots_matches_oracle_at_every_phase(env, W, n):
    df, torch, dev = env
    host = fold_inputs.slots("mixed", W, n, 31 * W + n)
    want = oracle.fold([host[r] for r in range(W)])
    want_s = oracle.fold_stacked_scaled(host, np.float32(0.25))
    for trial in range(3):
        offs = [(r * 3 + trial) % 4 for r in range(W)]  # slots at mixed 16-byte phases
        slots = [_placed(torch, dev, host[r], offs[r]) for r in range(W)]
        out = _placed(torch, dev, np.full(n, np.nan, np.float32), trial % 4)
        _say("case: fold_slots W=%d n=%d offsets %s" % (W, n, offs))
        df.fold_slots(out, slots)
        _assert_bits(_host(torch, out), want, "fold_slots W=%d n=%d offsets %s" % (W, n, offs))
        df.fold_slots_scaled(out, slots, 0.25)
        _assert_bits(_host(torch, out), want_s, "fold_slots_scaled W=%d n=%d" % (W, n))


@pytest.mark.parametrize("W", [2, 5, 8, 16])
def test_fold_slots_in_place_and_repeated_slots(env, W):
    df, torch, dev = env
    n = 100_003
    host = fold_inputs.slots("varied", W, n, 900 + W, spread=4.0)
    want = oracle.fold([host[r] for r in range(W)])
    for k in (0, W - 1):  # out is slot k
        slots = [_placed(torch, dev, host[r], r % 4) for r in range(W)]
        df.fold_slots(slots[k], slots)
        _assert_bits(_host(torch, slots[k]), want, "in place on slot %d, W=%d" % (k, W))
    # the same buffer passed as two slots folds it twice, in order
    a = _placed(torch, dev, host[0], 1)
    b = _placed(torch, dev, host[1], 0)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_slots(out, [a, b, a])
    _assert_bits(_host(torch, out), oracle.fold([host[0], host[1], host[0]]), "repeated slot")


@pytest.mark.parametrize("W", [5, 6, 7, 8, 9, 11, 12, 13, 14, 15, 16])
@pytest.mark.parametrize("n", [5, 4096, 70001, 1 << 20])
def test_co_aligned_folds_take_the_two_slots_per_wave_shape(env, W, n):
    # every buffer at one 16-byte phase: the row body streams two slots per
    # wave (an odd width's last wave one); fold_slots out of place and in
    # place, and fold_ranks over a stacked arena at the same phase
    df, torch, dev = env
    host = fold_inputs.slots("varied", W, n, 700 + W + n, spread=3.0)
    want = oracle.fold([host[r] for r in range(W)])
    for phase in (0, 2):
        slots = [_placed(torch, dev, host[r], phase) for r in range(W)]
        out = _placed(torch, dev, np.full(n, np.nan, np.float32), phase)
        _say("case: co-aligned fold_slots W=%d n=%d phase %d" % (W, n, phase))
        df.fold_slots(out, slots)
        _assert_bits(_host(torch, out), want, "W=%d n=%d phase %d" % (W, n, phase))
        df.fold_slots(slots[W - 1], slots)  # in place on the last slot
        _assert_bits(_host(torch, slots[W - 1]), want, "W=%d n=%d phase %d in place" % (W, n, phase))
        inv = np.float32(1.0 / W)
        out3 = _placed(torch, dev, np.full(n, np.nan, np.float32), phase)
        df.fold_slots_scaled(out3, slots[:W - 1] + [_placed(torch, dev, host[W - 1], phase)], float(inv))
        _assert_bits(_host(torch, out3), oracle.fold_stacked_scaled(host, inv),
                     "scaled W=%d n=%d phase %d" % (W, n, phase))
        if n % 4 == 0:  # a stacked arena is co-aligned only when its slot length is
            _say("case: co-aligned fold_ranks W=%d n=%d phase %d" % (W, n, phase))
            stacked = _placed(torch, dev, host.reshape(-1), phase).view(W, n)
            out2 = _placed(torch, dev, np.full(n, np.nan, np.float32), phase)
            df.fold_ranks(out2, stacked)
            _assert_bits(_host(torch, out2), want, "stacked W=%d n=%d phase %d" % (W, n, phase))
            df.fold_ranks_scaled(out2, stacked, float(inv))
            _assert_bits(_host(torch, out2), oracle.fold_stacked_scaled(host, inv),
                         "stacked scaled W=%d n=%d phase %d" % (W, n, phase))


# --------------------------------------------------------------------------
# the one-GPU reduction round

ROUND_CASES = [(2, 1), (2, 10_007), (3, 7), (8, 3), (8, 10_007), (8, 1 << 20), (16, 10_000_019),
               (16, 99_991), (5, 3_000_001)]


@pytest.mark.parametrize("W,n", ROUND_CASES)
def test_loopback_round_every_arena_holds_the_fold(env, W, n):
    df, torch, dev = env
    host = fold_inputs.slots("vecf" if W in (8, 16) else "mixed", W, n, 3000 + 7 * W)
    want = oracle.fold_stacked(host)
    stage = torch.empty(df.round_stage_elems(n, W) + 1, dtype=torch.float32, device=dev)
    for mode in ("ascending", "reversed", "direct", "fused"):
        _say("case: loopback round W=%d n=%d %s" % (W, n, mode))
        # arenas at mixed 16-byte phases, each in its own allocation
        arenas = [_placed(torch, dev, host[r], (r + n) % 4) for r in range(W)]
        staged = mode in ("ascending", "reversed")
        df.loopback_round(arenas, stage[1:] if staged else None, reverse_delivery=(mode == "reversed"),
                          direct=(mode == "direct"), fused=(mode == "fused"))
        for r in range(W):
            _assert_bits(_host(torch, arenas[r]), want, "W=%d n=%d %s arena %d" % (W, n, mode, r))


@pytest.mark.parametrize("W", [2, 4, 5, 7, 8, 13, 16])
@pytest.mark.parametrize("n", [1, 6, 4096, 70_001, 1 << 20])
def test_fused_round_on_co_aligned_arenas(env, W, n):
    # every arena at one 16-byte phase: the eight- and sixteen-arena rounds
    # take the several-slots-per-wave shapes; nothing outside [a, a + n) is
    # written
    df, torch, dev = env
    host = fold_inputs.slots("varied", W, n, 900 + W + n, spread=3.0)
    want = oracle.fold_stacked(host)
    for phase in (0, 3):
        _say("case: fused round W=%d n=%d phase %d" % (W, n, phase))
        allocs = [torch.full((n + 8,), float("nan"), dtype=torch.float32, device=dev) for _ in range(W)]
        arenas = [a[phase:phase + n] for a in allocs]
        for r in range(W):
            arenas[r].copy_(torch.from_numpy(host[r]))
        df.loopback_round(arenas, fused=True)
        for r in range(W):
            full = _host(torch, allocs[r])
            _assert_bits(full[phase:phase + n], want, "W=%d n=%d phase %d arena %d" % (W, n, phase, r))
            assert np.isnan(full[:phase]).all() and np.isnan(full[phase + n:]).all()


def test_loopback_round_twice_doubles(env):
    # after one round every arena holds S; a second round over W copies of S
    # folds S W times in ascending order
    df, torch, dev = env
    W, n = 4, 65_537
    host = fold_inputs.slots("vecf", W, n, 77)
    s = oracle.fold_stacked(host)
    want = oracle.fold([s] * W)
    for mode in ("direct", "fused"):
        arenas = [_placed(torch, dev, host[r], 0) for r in range(W)]
        df.loopback_round(arenas, direct=(mode == "direct"), fused=(mode == "fused"))
        df.loopback_round(arenas, direct=(mode == "direct"), fused=(mode == "fused"))
        for r in range(W):
            _assert_bits(_host(torch, arenas[r]), want, "%s second round arena %d" % (mode, r))


def test_loopback_round_one_rank_is_a_no_op(env):
    df, torch, dev = env
    host = fold_inputs.vecf(1000, 1)
    a = _placed(torch, dev, host, 0)
    df.loopback_round([a])
    _assert_bits(_host(torch, a), host, "W=1 round")


# --------------------------------------------------------------------------
# two ranks on two streams

def _pair_round(df, torch, link, xa, xb):
    link.all_reduce(xa, xb)
    for st in link.streams:
        st.synchronize()


def test_pair_all_reduce_sweep_doubles_on_repeat(env):
    df, torch, dev = env
    link = df.PairLink(1 << 18, device=dev)  # staging reused by every size and call
    for n in (1, 4, 1024, 4096, 16384, 65536, 1 << 18):
        _say("case: pair all-reduce n=%d" % n)
        ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
        want = oracle.fold_into(ha, hb)
        xa = torch.from_numpy(ha).to(dev)
        xb = torch.from_numpy(hb).to(dev)
        torch.cuda.synchronize()
        _pair_round(df, torch, link, xa, xb)
        _assert_bits(xa.cpu().numpy(), want, "rank 0 n=%d" % n)
        _assert_bits(xb.cpu().numpy(), want, "rank 1 n=%d" % n)
        _pair_round(df, torch, link, xa, xb)
        twice = oracle.fold_into(want, want)
        _assert_bits(xa.cpu().numpy(), twice, "rank 0 second call n=%d" % n)
        _assert_bits(xb.cpu().numpy(), twice, "rank 1 second call n=%d" % n)


def test_pair_all_reduce_back_to_back_without_host_sync(env):
    # ten calls queued with no synchronization between them: the events alone
    # keep each push from overwriting a staging buffer the peer still reads
    df, torch, dev = env
    n = 65536
    link = df.PairLink(n, device=dev)
    ha, hb = fold_inputs.varied(n, 3, 1.0), fold_inputs.varied(n, 4, 1.0)
    xa = torch.from_numpy(ha).to(dev)
    xb = torch.from_numpy(hb).to(dev)
    torch.cuda.synchronize()
    want = oracle.fold_into(ha, hb)
    for _ in range(10):
        link.all_reduce(xa, xb)
        want = oracle.fold_into(want, want) if _ else want
    for st in link.streams:
        st.synchronize()
    _assert_bits(xa.cpu().numpy(), want, "rank 0 after 10 calls")
    _assert_bits(xb.cpu().numpy(), want, "rank 1 after 10 calls")


def test_pair_all_reduce_beside_a_busy_stream(env):
    df, torch, dev = env
    big = torch.from_numpy(fold_inputs.slots("vecf", 8, 1 << 22, 5)).to(dev)
    big_out = torch.empty(1 << 22, dtype=torch.float32, device=dev)
    n = 1 << 16
    link = df.PairLink(n, device=dev)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    xa = torch.from_numpy(ha).to(dev)
    xb = torch.from_numpy(hb).to(dev)
    torch.cuda.synchronize()
    busy = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(busy):
        for _ in range(30):
            df.fold_ranks(big_out, big)
    link.all_reduce(xa, xb)
    for st in link.streams:
        st.synchronize()
    _assert_bits(xa.cpu().numpy(), oracle.fold_into(ha, hb), "rank 0 beside a busy stream")
    _assert_bits(xb.cpu().numpy(), oracle.fold_into(ha, hb), "rank 1 beside a busy stream")
    busy.synchronize()


@pytest.mark.skip(reason=PAIR_CAPTURE_OFF)
@pytest.mark.parametrize("n", [4096, 65536])
def test_pair_all_reduce_graph_replays(env, n):
    # One call captured in a HIP graph (both rank streams forked from the
    # capture stream and joined back), replayed with eager work and host
    # synchronizations between the replays: replay k must hold 2^(k-1) times
    # the sum on both ranks, bit for bit.
    df, torch, dev = env
    _say("case: pair all-reduce captured into a graph, n=%d" % n)
    link = df.PairLink(n, device=dev)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    xa = torch.from_numpy(ha).to(dev)
    xb = torch.from_numpy(hb).to(dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        link.all_reduce(xa, xb)
    want = oracle.fold_into(ha, hb)
    for k in range(4):
        graph.replay()
        torch.cuda.synchronize()
        _assert_bits(xa.cpu().numpy(), want, "rank 0 replay %d" % k)
        _assert_bits(xb.cpu().numpy(), want, "rank 1 replay %d" % k)
        want = oracle.fold_into(want, want)


@pytest.mark.skip(reason=PAIR_CAPTURE_OFF)
def test_pair_movement_graph_replays(env):
    # A broadcast and an all-gather captured into one HIP graph, replayed
    # three times with eager writes to every destination between replays:
    # each replay must leave the bytes exactly (the events are graph edges).
    df, torch, dev = env
    span = 1027
    _say("case: pair all-gather and broadcast captured into a graph, span=%d" % span)
    link = df.PairLink(span, device=dev)
    ha, hb = fold_inputs.vecf(span, 5), fold_inputs.vecf(span, 6)
    xa = torch.from_numpy(ha).to(dev)
    xb = torch.from_numpy(hb).to(dev)
    f0 = torch.zeros(2 * span, dtype=torch.float32, device=dev)
    f1 = torch.zeros(2 * span, dtype=torch.float32, device=dev)
    d = torch.zeros(span, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        link.all_gather(xa, xb, f0, f1)
        link.broadcast(1, xb, d)
    want = np.concatenate([ha, hb])
    for k in range(3):
        f0.fill_(-1.0)
        f1.fill_(-2.0)
        d.fill_(-3.0)
        graph.replay()
        torch.cuda.synchronize()
        _assert_bits(f0.cpu().numpy(), want, "all-gather rank 0, replay %d" % k)
        _assert_bits(f1.cpu().numpy(), want, "all-gather rank 1, replay %d" % k)
        _assert_bits(d.cpu().numpy(), hb, "broadcast from rank 1, replay %d" % k)


def test_pair_all_reduce_orders_against_the_current_stream(env):
    # The inputs are written on the caller's current stream right before the
    # call, with no host synchronization: the call must see those writes,
    # and work queued after it on the current stream must see its result.
    df, torch, dev = env
    n = 1 << 18
    link = df.PairLink(n, device=dev)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    src_a = torch.from_numpy(ha).to(dev)
    src_b = torch.from_numpy(hb).to(dev)
    big = torch.from_numpy(fold_inputs.slots("vecf", 8, 1 << 22, 9)).to(dev)
    big_out = torch.empty(1 << 22, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    xa = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    xb = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for _ in range(10):
        df.fold_ranks(big_out, big)  # keep the current stream busy for a while
    xa.copy_(src_a)
    xb.copy_(src_b)
    link.all_reduce(xa, xb)
    got_a, got_b = xa.clone(), xb.clone()  # queued on the current stream after the call
    torch.cuda.synchronize()
    want = oracle.fold_into(ha, hb)
    _assert_bits(got_a.cpu().numpy(), want, "rank 0 seen from the current stream")
    _assert_bits(got_b.cpu().numpy(), want, "rank 1 seen from the current stream")
