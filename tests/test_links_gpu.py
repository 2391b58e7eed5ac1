"""GPU parity for the two-rank movement calls and the one-shot all-reduce
(through the C ABI), against the oracle.

* broadcast / all-gather (memra-engine tests/tp_ar_gpu.rs,
  broadcast_and_all_gather_move_bytes_exactly): pure movement, so every word
  must arrive unchanged; the all-gather is read on both ranks.
* one-shot all-reduce (same file, one_shot_all_reduce_matches_the_host_sum_
  bitwise): one kernel, an in-kernel entry and exit barrier, three rounds per
  size on one link; the barrier words are read before the numbers, and round
  k must equal the fold of round k-1 with itself.
* refusal words: forced from the host -- one rank's kernel launched with the
  peer never launched and a tiny poll limit, so every wait ends by expiry and
  every kernel exits.
"""
import sys

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu

ONE_SHOT_SIZES = [1, 4, 1024, 4096, 16384, 65536, 65537, 1 << 18, 1 << 20, 3_000_001]


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


def _dev(torch, dev, host, offset=0):
    alloc = torch.empty(host.size + 4, dtype=torch.float32, device=dev)
    view = alloc[offset:offset + host.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(host)))
    return view


# --------------------------------------------------------------------------
# pure movement

@pytest.mark.parametrize("span", [1, 1024, 16384, 1 << 20])
def test_broadcast_moves_bytes_exactly(env, span):
    df, torch, dev = env
    link = df.PairLink(1, device=dev)
    for root in (0, 1):
        _say("case: broadcast span=%d root=%d" % (span, root))
        hsrc = fold_inputs.mixed(span, 31 + span + root)
        src = _dev(torch, dev, hsrc, root)
        dst = _dev(torch, dev, np.full(span, np.nan, np.float32), 0 if root == 0 else 3)
        link.broadcast(root, src, dst)
        link.streams[1 - root].synchronize()
        _assert_bits(dst.cpu().numpy(), hsrc, "broadcast span=%d root=%d" % (span, root))


@pytest.mark.parametrize("span", [1, 1024, 16384, 1 << 20])
def test_all_gather_is_rank_order_concatenation_on_both_ranks(env, span):
    df, torch, dev = env
    link = df.PairLink(1, device=dev)
    pa, pb = fold_inputs.mixed(span, 41 + span), fold_inputs.mixed(span, 42 + span)
    want = np.concatenate([pa, pb])
    for trial in range(2):  # the second call reuses the link's events
        _say("case: all_gather span=%d trial %d" % (span, trial))
        da, db = _dev(torch, dev, pa, trial), _dev(torch, dev, pb, 0)
        fa = _dev(torch, dev, np.full(2 * span, np.nan, np.float32), 1)
        fb = _dev(torch, dev, np.full(2 * span, np.nan, np.float32), trial)
        link.all_gather(da, db, fa, fb)
        link.streams[0].synchronize()
        link.streams[1].synchronize()
        _assert_bits(fa.cpu().numpy(), want, "all_gather rank 0 span=%d" % span)
        _assert_bits(fb.cpu().numpy(), want, "all_gather rank 1 span=%d" % span)


# --------------------------------------------------------------------------
# one-shot all-reduce

def _rounds_want(ha, hb, rounds):
    out = [oracle.fold_into(ha, hb)]
    for _ in range(rounds - 1):
        out.append(oracle.fold_into(out[-1], out[-1]))
    return out


def test_one_shot_matches_the_oracle_over_three_rounds(env):
    df, torch, dev = env
    link = df.OneShotLink(max(ONE_SHOT_SIZES), device=dev)  # one link, every size, every round
    for n in ONE_SHOT_SIZES:
        ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
        wants = _rounds_want(ha, hb, 3)
        xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
        for rnd, want in enumerate(wants):
            _say("case: one-shot n=%d round %d" % (n, rnd))
            link.all_reduce(xa, xb)
            # the words first: an expired entry barrier leaves x untouched, which
            # read as numbers would look like a wrong sum, not a refusal
            assert link.barrier_words() == [0, 0], "barrier expired at n=%d round %d" % (n, rnd)
            _assert_bits(xa.cpu().numpy(), want, "rank 0 n=%d round %d" % (n, rnd))
            _assert_bits(xb.cpu().numpy(), want, "rank 1 n=%d round %d" % (n, rnd))


@pytest.mark.parametrize("n", [3, 4099, 70001])
def test_one_shot_at_unaligned_addresses(env, n):
    df, torch, dev = env
    link = df.OneShotLink(n, device=dev)
    ha, hb = fold_inputs.mixed(n, 500 + n), fold_inputs.mixed(n, 600 + n)
    want = oracle.fold_into(ha, hb)
    for oa, ob in ((1, 0), (3, 2)):
        _say("case: one-shot n=%d offsets %d,%d" % (n, oa, ob))
        xa, xb = _dev(torch, dev, ha, oa), _dev(torch, dev, hb, ob)
        link.all_reduce(xa, xb)
        assert link.barrier_words() == [0, 0]
        _assert_bits(xa.cpu().numpy(), want, "rank 0 n=%d" % n)
        _assert_bits(xb.cpu().numpy(), want, "rank 1 n=%d" % n)


def test_one_shot_refusal_words_when_the_peer_never_arrives(env):
    # Each rank's kernel is launched alone on one stream, one after the other,
    # with a poll limit of 64: every wait either finds its peer's count or
    # expires, so each kernel exits on its own.
    #   rank 0 alone: the entry wait expires (40043), x0 is left untouched, but
    #                 its push already put x0 into rank 1's stage;
    #   rank 1 alone: its entry wait finds rank 0's arrival, it folds
    #                 x1 + x0 (the right sum), and its exit wait expires (40044).
    df, torch, dev = env
    n = 4096
    link = df.OneShotLink(n, device=dev, spin_limit=64)
    ha, hb = fold_inputs.vecf(n, 5), fold_inputs.vecf(n, 6)
    xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
    _say("case: one-shot rank 0 alone, poll limit 64")
    link.rank(0, xa)
    assert link.barrier_words() == [df.BARRIER_ENTRY_EXPIRED, 0]
    _assert_bits(xa.cpu().numpy(), ha, "rank 0 after an expired entry barrier")
    _say("case: one-shot rank 1 alone, poll limit 64")
    link.rank(1, xb)
    assert link.barrier_words() == [df.BARRIER_ENTRY_EXPIRED, df.BARRIER_EXIT_EXPIRED]
    _assert_bits(xb.cpu().numpy(), oracle.fold_into(hb, ha), "rank 1 after the peer's push")
    # a refused sum is not the sum: the red arm of the numbers
    assert not np.array_equal(_bits(xa.cpu().numpy()), _bits(oracle.fold_into(ha, hb)))
    # re-initialised, the same link works again
    link._c.spin_limit = 0
    link.init()
    assert link.barrier_words() == [0, 0]
    xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
    link.all_reduce(xa, xb)
    assert link.barrier_words() == [0, 0]
    _assert_bits(xa.cpu().numpy(), oracle.fold_into(ha, hb), "rank 0 after re-init")
    _assert_bits(xb.cpu().numpy(), oracle.fold_into(ha, hb), "rank 1 after re-init")


def test_one_shot_graph_replays_are_fresh_calls(env):
    # the barrier counters are advanced by the kernel, so each replay of one
    # captured call is a new round: the sum doubles on every replay
    df, torch, dev = env
    n = 16384
    s = torch.cuda.Stream(device=dev)
    link = df.OneShotLink(n, device=dev, stream=s)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    wants = _rounds_want(ha, hb, 4)
    xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        link.all_reduce(xa, xb)
    torch.cuda.synchronize()
    for k, want in enumerate(wants):
        _say("case: one-shot graph replay %d" % k)
        g.replay()
        torch.cuda.synchronize()
        assert link.barrier_words() == [0, 0]
        _assert_bits(xa.cpu().numpy(), want, "rank 0 replay %d" % k)
        _assert_bits(xb.cpu().numpy(), want, "rank 1 replay %d" % k)
        xa.mul_(1.0)  # eager work between replays (x * 1 is x, bit for bit)


def test_one_shot_beside_a_busy_stream(env):
    df, torch, dev = env
    big = torch.from_numpy(fold_inputs.slots("vecf", 8, 1 << 22, 5)).to(dev)
    big_out = torch.empty(1 << 22, dtype=torch.float32, device=dev)
    n = 1 << 16
    link = df.OneShotLink(n, device=dev, stream=torch.cuda.Stream(device=dev))
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
    torch.cuda.synchronize()
    busy = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(busy):
        for _ in range(30):
            df.fold_ranks(big_out, big)
    _say("case: one-shot beside 30 large folds")
    link.all_reduce(xa, xb)
    assert link.barrier_words() == [0, 0]
    _assert_bits(xa.cpu().numpy(), oracle.fold_into(ha, hb), "rank 0 beside a busy stream")
    _assert_bits(xb.cpu().numpy(), oracle.fold_into(ha, hb), "rank 1 beside a busy stream")


def test_one_shot_per_rank_kernels_on_two_streams(env):
    # The shape each rank runs on its own device, here as two streams of one
    # process.  Streams created one after the other sit on different hardware
    # queues, so the two kernels run concurrently and their barriers must
    # meet: no refusal word, and both ranks hold the exact sum, on every one
    # of five calls in a row.  Rank 1 is launched first each time: were the
    # two serialized, its waits would expire and the words would say so.
    df, torch, dev = env
    n = 4096
    link = df.OneShotLink(n, device=dev)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    want = oracle.fold_into(ha, hb)
    xa, xb = _dev(torch, dev, ha), _dev(torch, dev, hb)
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    torch.cuda.synchronize()
    for call in range(5):
        _say("case: one-shot per-rank kernels on two streams, call %d" % call)
        link.rank(1, xb, stream=streams[1])
        link.rank(0, xa, stream=streams[0])
        assert link.barrier_words() == [0, 0], "the per-rank kernels did not meet (call %d)" % call
        _assert_bits(xa.cpu().numpy(), want, "rank 0 call %d" % call)
        _assert_bits(xb.cpu().numpy(), want, "rank 1 call %d" % call)
        want = oracle.fold_into(want, want)
