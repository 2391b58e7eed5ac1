"""GPU parity: the HIP fold (through the C ABI) against the CPU oracle, bit for bit.

Workloads (all inputs from ``fold_inputs``, seeded; none from the HIP path):

* decode join, memra-engine tests/tp_ar_gpu.rs: in-place fold at n = 4096
  (16 KiB per buffer) and the sweep n in {1, 4, 1024, 4096, 16384, 65536}
  with seeds 11+n / 77+n, reused staging buffers, the repeat call that doubles
  the sum, and the red arm (a fold with nothing pushed must not reproduce the
  sum);
* W = 8 stacked [8][16777216] (64 MiB per slot), slot r = vecf(2^24, 1000+r);
* W = 4 gradient arena [4][100000000], slot r = mixed(1e8, 2000+r), with the
  exact 1/4 mean scale and without it;
* W = 16 arena of len 10000019 starting one element past an aligned
  allocation, slot r = vecf(len, 3000+r), folded whole and as 16 owner shards
  gathered into per-owner scratch by device copies in ascending and in
  reversed delivery order (mamba-rs src/dist/reducer.rs, `LoopbackWorld`);
* geometry and alignment sweeps, chained two-addend folds against one W-slot
  fold (memra-engine tests/gdn_packed_gpu.rs, packed vs chained), subnormal
  and special values, one slot, zero length, and the error codes.

Bar: 0 ULP -- every output word equal to the oracle's (NaN payloads are not
pinned by the pages; only NaN-ness is compared where NaNs arise).
"""
import os
import sys

import numpy as np
import pytest

import fold_inputs
import oracle

pytestmark = pytest.mark.gpu


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
    gn = ((g & 0x7F800000) == 0x7F800000) & ((g & 0x7FFFFF) != 0)
    wn = ((w & 0x7F800000) == 0x7F800000) & ((w & 0x7FFFFF) != 0)
    bad = (g != w) & ~(gn & wn)
    n_bad = int(np.count_nonzero(bad))
    if n_bad:
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError("%s: %d of %d words differ; first at %d: got %08x want %08x"
                             % (what, n_bad, g.size, i, g.flat[i], w.flat[i]))


def _to_dev(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


# --------------------------------------------------------------------------
# decode join (in-place, two addends)

def _exchange_and_fold(df, torch, xa, xb, stage_a, stage_b, n):
    """One TP-2 round emulated on one device: each rank's partial is pushed
    into the peer's reused staging buffer (pure byte movement), then each rank
    folds in place.  Both pushes precede both folds, as in a real exchange."""
    stage_a[:n].copy_(xb)
    stage_b[:n].copy_(xa)
    df.fold_into(xa, stage_a[:n])
    df.fold_into(xb, stage_b[:n])


@pytest.mark.parametrize("n", [4096])
def test_decode_join_16kib_and_second_fold_doubles(env, n):
    df, torch, dev = env
    _say("case: decode join n=%d" % n)
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    want = oracle.fold_into(ha, hb)
    xa, xb = _to_dev(torch, dev, ha), _to_dev(torch, dev, hb)
    stage_a = torch.zeros(65536, dtype=torch.float32, device=dev)
    stage_b = torch.zeros(65536, dtype=torch.float32, device=dev)
    _exchange_and_fold(df, torch, xa, xb, stage_a, stage_b, n)
    _assert_bits(_host(xa), want, "rank 0 after the first fold")
    _assert_bits(_host(xb), want, "rank 1 after the first fold")
    _exchange_and_fold(df, torch, xa, xb, stage_a, stage_b, n)
    twice = oracle.fold_into(want, want)
    _assert_bits(_host(xa), twice, "rank 0 after the second fold (2x the sum)")
    _assert_bits(_host(xb), twice, "rank 1 after the second fold (2x the sum)")
    # 2x by exponent increment (the sums are normal and far from overflow here)
    w = _bits(want)
    nz = (w & 0x7FFFFFFF) != 0
    assert np.array_equal(_bits(_host(xa))[nz], (w + (1 << 23))[nz])


def test_decode_join_sweep_on_reused_staging(env):
    df, torch, dev = env
    stage_a = torch.zeros(65536, dtype=torch.float32, device=dev)
    stage_b = torch.zeros(65536, dtype=torch.float32, device=dev)
    for n in (1, 4, 1024, 4096, 16384, 65536):
        _say("case: decode join sweep n=%d" % n)
        ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
        want = oracle.fold_into(ha, hb)
        xa, xb = _to_dev(torch, dev, ha), _to_dev(torch, dev, hb)
        _exchange_and_fold(df, torch, xa, xb, stage_a, stage_b, n)
        _assert_bits(_host(xa), want, "rank 0 n=%d" % n)
        _assert_bits(_host(xb), want, "rank 1 n=%d" % n)
        _exchange_and_fold(df, torch, xa, xb, stage_a, stage_b, n)
        _assert_bits(_host(xa), oracle.fold_into(want, want), "second call n=%d" % n)


def test_decode_join_full_mantissa(env):
    # vecf pairs sum exactly; full-mantissa addends make every fold round
    df, torch, dev = env
    for n in (1, 4, 1023, 4096, 65536, 65537):
        ha = fold_inputs.varied(n, 500 + n, 3.0)
        hb = fold_inputs.varied(n, 900 + n, 0.7)
        xa, xb = _to_dev(torch, dev, ha), _to_dev(torch, dev, hb)
        df.fold_into(xa, xb)
        _assert_bits(_host(xa), oracle.fold_into(ha, hb), "varied n=%d" % n)


@pytest.mark.parametrize("n", [1, 4, 1024, 4096, 16384, 65536])
def test_red_arm_fold_without_the_push_diverges(env, n):
    """memra-engine tests/tp_ar_gpu.rs red arm: with nothing pushed the stage
    holds zeros, rank 0 keeps its own partial, and the check must see it."""
    df, torch, dev = env
    ha = fold_inputs.vecf(n, 5 if n == 4096 else 11 + n)
    hb = fold_inputs.vecf(n, 6 if n == 4096 else 77 + n)
    want = oracle.fold_into(ha, hb)
    xa = _to_dev(torch, dev, ha)
    stage = torch.zeros(n, dtype=torch.float32, device=dev)
    df.fold_into(xa, stage)
    got = _host(xa)
    _assert_bits(got, oracle.fold_into(ha, np.zeros(n, np.float32)), "zero-stage fold n=%d" % n)
    same = int(np.count_nonzero(_bits(got) == _bits(want)))
    assert same < n, "a fold with no peer push reproduced the sum at n=%d" % n


# --------------------------------------------------------------------------
# W = 8, 64 MiB per slot

@pytest.fixture(scope="module")
def w8_arena():
    return fold_inputs.slots("vecf", 8, 1 << 24, 1000)


def test_w8_64mib_per_slot_bit_exact(env, w8_arena):
    df, torch, dev = env
    _say("case: W=8 [8][16777216] fold_ranks")
    want = oracle.fold_stacked(w8_arena)
    stacked = _to_dev(torch, dev, w8_arena)
    out = torch.empty(1 << 24, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    got = _host(out)
    _assert_bits(got, want, "W=8 fold_ranks")
    # repeat-run determinism with a non-vacuity report
    for rep in range(3):
        out.fill_(0.0)
        df.fold_ranks(out, stacked)
        _assert_bits(_host(out), got, "W=8 repeat %d" % rep)
    down = oracle.fold_stacked(np.ascontiguousarray(w8_arena[::-1]))
    frac = float(np.count_nonzero(_bits(down) != _bits(want))) / want.size
    nz = int(np.count_nonzero(got))
    _say("W=8: order-sensitive share %.3f, nonzero %d, absmax %.4f, nan %d"
         % (frac, nz, float(np.abs(got).max()), int(np.isnan(got).sum())))
    assert frac > 0.05 and nz > 0.99 * got.size
    # dropping the last addend must diverge
    out7 = torch.empty_like(out)
    df.fold_ranks(out7, stacked[:7])
    assert int(np.count_nonzero(_bits(_host(out7)) != _bits(got))) > 0


def test_w8_scaled_mean(env, w8_arena):
    df, torch, dev = env
    _say("case: W=8 fold_ranks_scaled 1/8")
    stacked = _to_dev(torch, dev, w8_arena)
    out = torch.empty(1 << 24, dtype=torch.float32, device=dev)
    df.fold_ranks_scaled(out, stacked, 0.125)
    _assert_bits(_host(out), oracle.fold_stacked_scaled(w8_arena, np.float32(0.125)), "W=8 scaled")


# --------------------------------------------------------------------------
# W = 4 gradient arena, mixed magnitudes, exact 1/4 mean

def test_w4_gradient_arena_mixed_magnitudes(env):
    df, torch, dev = env
    n = 100_000_000
    _say("case: W=4 [4][100000000] mixed, scaled 1/4 and unscaled")
    host = fold_inputs.slots("mixed", 4, n, 2000)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks_scaled(out, stacked, 0.25)
    got_scaled = _host(out)
    want_scaled = oracle.fold_stacked_scaled(host, np.float32(0.25))
    _assert_bits(got_scaled, want_scaled, "W=4 scaled")
    df.fold_ranks(out, stacked)
    got = _host(out)
    want = oracle.fold_stacked(host)
    _assert_bits(got, want, "W=4 sum")
    # the 1/4 scale of a normal sum is exact: exponent field down by 2
    w = _bits(want)
    normal = ((w >> 23) & 0xFF) > 2
    assert np.array_equal(_bits(got_scaled)[normal], (w - (2 << 23))[normal])
    down = oracle.fold_stacked(np.ascontiguousarray(host[::-1]))
    frac = float(np.count_nonzero(_bits(down) != w)) / n
    _say("W=4 mixed: order-sensitive share %.3f" % frac)
    assert frac > 0.05


# --------------------------------------------------------------------------
# W = 16, len 10000019 at base + 1 element: whole fold and 16 owner shards

def test_w16_offset_arena_shards_equal_whole(env):
    df, torch, dev = env
    W, n = 16, 10_000_019
    _say("case: W=16 len=%d at base+1, whole and 16 shards" % n)
    host = fold_inputs.slots("vecf", W, n, 3000)
    want = oracle.fold_stacked(host)
    alloc = torch.empty(W * n + 1, dtype=torch.float32, device=dev)
    stacked = alloc[1:].view(W, n)
    assert stacked.data_ptr() % 16 == 4
    stacked.copy_(torch.from_numpy(host))
    out_w = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out_w, stacked)  # the LDS row body, slots at three phases other than out's
    whole = _host(out_w)
    _assert_bits(whole, want, "W=16 whole arena")
    out_w.fill_(float("nan"))
    df.fold_ranks_ex(out_w, stacked, path=df.PATH_SCALAR)  # the direct 4-byte body
    _assert_bits(_host(out_w), want, "W=16 whole arena, scalar body")
    plan = df.shard_plan(n, W)
    assert [ln for _, ln in plan] == [625_002] * 3 + [625_001] * 13
    for reverse in (False, True):
        _say("case: W=16 shards, reverse_delivery=%s" % reverse)
        out_s = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
        for p, (s, ln) in enumerate(plan):
            if ln == 0:
                continue
            scratch = torch.empty((W, ln), dtype=torch.float32, device=dev)
            order = range(W - 1, -1, -1) if reverse else range(W)
            for src in order:  # slot = source rank, whatever the delivery order
                scratch[src].copy_(stacked[src, s:s + ln])
            df.fold_ranks(out_s[s:s + ln], scratch)
        _assert_bits(_host(out_s), whole, "shards (reverse=%s) vs whole" % reverse)
    down = oracle.fold_stacked(np.ascontiguousarray(host[::-1]))
    frac = float(np.count_nonzero(_bits(down) != _bits(want))) / n
    _say("W=16: order-sensitive share %.3f" % frac)
    assert frac > 0.05


# --------------------------------------------------------------------------
# geometry and alignment: the bits never depend on them

GEOMS = [dict(path=p, block=b, grid=g, unroll=u, policy=pol)
         for p in (1, 2) for b in (64, 256, 1024) for g in (0, 1, 7) for u in (1, 2, 4)
         for pol in ((0, 2) if u == 1 else (0,))]
ROW_GEOMS = [dict(path=3, block=b, grid=g, unroll=0, policy=0) for b in (0, -1) for g in (0, 1, 7)]


def _row_shape_blocks(W):
    """Every workgroup size that names a row-body shape at width W."""
    if W > 16:
        return [1024, 512]
    two = 8 if W in (13, 14) else -(-W // 2)  # waves of the two-slot shape
    return [64 * W] + ([64 * two] if W >= 5 else [])


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 7, 8, 9, 13, 14, 16, 17, 24, 33, 64])
def test_geometry_independence(env, W):
    df, torch, dev = env
    n = 3 * (1 << 15) + 4  # several tiles; a multiple of 4 so the vector body is legal
    host = fold_inputs.slots("varied", W, n, 40 + W, spread=2.0)
    want = oracle.fold_stacked(host)
    want_s = oracle.fold_stacked_scaled(host, np.float32(1.0 / 8))
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    geoms = list(GEOMS)
    if W >= 2:  # the LDS row bodies; block -1 stands for the size the plan gives them
        cu = torch.cuda.get_device_properties(dev).multi_processor_count
        rb = df.plan_fold_ranks(out.data_ptr(), stacked.data_ptr(), W, n, cu)["block"]
        geoms += [dict(g, block=rb if g["block"] < 0 else 0) for g in ROW_GEOMS]
        # every shape, with XCD tile groups, in one pass and looping over the tiles
        geoms += [dict(path=3, block=b, grid=g, unroll=0, policy=0, group=x)
                  for b in _row_shape_blocks(W) for x in (1, 4, 64) for g in (0, 7)]
    for geom in geoms:
        if W >= 16 and geom["unroll"] == 4 and geom["block"] == 1024:
            continue  # legal but spills registers; covered at smaller blocks
        _say("case: geometry W=%d %s" % (W, geom))
        out.fill_(float("nan"))
        df.fold_ranks_ex(out, stacked, **geom)
        _assert_bits(_host(out), want, "W=%d %s" % (W, geom))
        df.fold_ranks_ex(out, stacked, scaled=True, inv_w=1.0 / 8, **geom)
        _assert_bits(_host(out), want_s, "W=%d scaled %s" % (W, geom))


@pytest.mark.parametrize("out_off,in_off", [(0, 0), (1, 1), (2, 2), (3, 3), (0, 1), (3, 0), (2, 1)])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 4099, 4100, 65536 + 3])
@pytest.mark.parametrize("W", [1, 2, 4, 7, 8, 19])
def test_alignment_phases_and_ragged_lengths(env, out_off, in_off, n, W):
    df, torch, dev = env
    host = fold_inputs.slots("mixed", W, n, 7 * n + W)
    want = oracle.fold_stacked(host)
    in_alloc = torch.empty(W * n + 4, dtype=torch.float32, device=dev)
    stacked = in_alloc[in_off:in_off + W * n].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    paths = [df.PATH_AUTO, df.PATH_SCALAR] + ([df.PATH_ROWS] if 2 <= W <= 16 else [])
    for path in paths:
        out_alloc = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
        out = out_alloc[out_off:out_off + n]
        df.fold_ranks_ex(out, stacked, path=path)
        full = _host(out_alloc)
        _assert_bits(full[out_off:out_off + n], want,
                     "W=%d n=%d offsets %d/%d path %d" % (W, n, out_off, in_off, path))
        # nothing outside [out, out + n) is written
        assert np.isnan(full[:out_off]).all() and np.isnan(full[out_off + n:]).all()


def test_in_place_fold_alignment_phases(env):
    df, torch, dev = env
    # up to 8 MiB per buffer: the latency path; above it, the streaming row body in place
    for n in (1, 3, 4, 5, 4095, 4096, 65537, 3_000_001):
        for d_off, s_off in ((0, 0), (1, 1), (3, 3), (0, 2), (1, 0)):
            ha, hb = fold_inputs.varied(n, n, 1.0), fold_inputs.varied(n, n + 1, 1.0)
            da = torch.empty(n + 4, dtype=torch.float32, device=dev)
            sa = torch.empty(n + 4, dtype=torch.float32, device=dev)
            dst, stage = da[d_off:d_off + n], sa[s_off:s_off + n]
            dst.copy_(torch.from_numpy(ha))
            stage.copy_(torch.from_numpy(hb))
            df.fold_into(dst, stage)
            _assert_bits(_host(dst), oracle.fold_into(ha, hb), "fold_into n=%d %d/%d" % (n, d_off, s_off))


# --------------------------------------------------------------------------
# chained two-addend folds vs one W-slot fold

@pytest.mark.parametrize("W", [2, 3, 8, 16])
def test_chained_in_place_folds_equal_one_stacked_fold(env, W):
    df, torch, dev = env
    n = 200_003
    host = fold_inputs.slots("mixed", W, n, 600 + W)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    acc = stacked[0].clone()
    for r in range(1, W):
        df.fold_into(acc, stacked[r])
    _assert_bits(_host(acc), _host(out), "chained W=%d" % W)
    _assert_bits(_host(out), oracle.fold_stacked(host), "stacked W=%d" % W)


# --------------------------------------------------------------------------
# special values, one slot, nothing to do, errors

def test_subnormals_are_kept(env):
    df, torch, dev = env
    rng = np.random.default_rng(3)
    W, n = 8, 1 << 16
    exp = rng.integers(0, 3, size=(W, n)).astype(np.uint32)
    mant = rng.integers(0, 1 << 23, size=(W, n)).astype(np.uint32)
    sign = rng.integers(0, 2, size=(W, n)).astype(np.uint32)
    host = ((sign << 31) | (exp << 23) | mant).view(np.float32)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    got = _host(out)
    _assert_bits(got, oracle.fold_stacked(host), "subnormal addends")
    assert np.count_nonzero((_bits(got) & 0x7F800000) == 0) > n // 20  # some sums stay subnormal
    for inv in (0.125, 0.5, 0.3):
        df.fold_ranks_scaled(out, stacked, inv)
        _assert_bits(_host(out), oracle.fold_stacked_scaled(host, np.float32(inv)), "subnormal scaled %g" % inv)


def test_special_values(env):
    df, torch, dev = env
    pool = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF,
                     0x00000001, 0x80000001, 0x3F800000, 0x33800000, 0x4B800000, 0x7FC00000],
                    dtype=np.uint32)
    rng = np.random.default_rng(9)
    W, n = 5, 50_000
    host = pool[rng.integers(0, pool.size, size=(W, n))].view(np.float32)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    _assert_bits(_host(out), oracle.fold_stacked(host), "special values")


def test_one_slot_is_a_bit_copy(env):
    df, torch, dev = env
    n = 100_001
    host = fold_inputs.slots("mixed", 1, n, 1)
    host[0, :3] = np.array([0x80000000, 0x00000001, 0x807FFFFF], np.uint32).view(np.float32)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    _assert_bits(_host(out), host[0], "W=1")


def test_zero_length_launches_nothing(env):
    df, torch, dev = env
    out = torch.empty(0, dtype=torch.float32, device=dev)
    stacked = torch.empty((8, 0), dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    df.fold_ranks_scaled(out, stacked, 0.5)
    df.fold_into(out, torch.empty(0, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()


def test_error_codes_through_the_binding(env):
    df, torch, dev = env
    stacked = torch.zeros((4, 1024), dtype=torch.float32, device=dev)
    with pytest.raises(df.DetfoldError) as e:
        df.fold_ranks(stacked[1], stacked)  # out aliases slot 1
    assert e.value.rc == df.EOVERLAP
    with pytest.raises(df.DetfoldError) as e:
        df.fold_into(stacked[0], stacked[0])
    assert e.value.rc == df.EOVERLAP
    with pytest.raises(df.DetfoldError) as e:
        df.fold_ranks_ex(torch.empty(1024, device=dev), stacked, block=100)
    assert e.value.rc == df.EINVAL
    with pytest.raises(TypeError):
        df.fold_ranks(torch.empty(1024, dtype=torch.float64, device=dev), stacked)
    with pytest.raises(ValueError):
        df.fold_ranks(torch.empty(1024), stacked)  # host tensor


def test_fold_into_next_to_a_busy_stream(env):
    """The in-place fold waits on nothing, so it completes while another
    stream keeps the device busy with a large fold."""
    df, torch, dev = env
    big = torch.from_numpy(fold_inputs.slots("vecf", 8, 1 << 22, 77)).to(dev)
    big_out = torch.empty(1 << 22, dtype=torch.float32, device=dev)
    n = 65536
    ha, hb = fold_inputs.vecf(n, 11 + n), fold_inputs.vecf(n, 77 + n)
    xa, xb = _to_dev(torch, dev, ha), _to_dev(torch, dev, hb)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        for _ in range(20):
            df.fold_ranks(big_out, big)
    df.fold_into(xa, xb)
    torch.cuda.current_stream(dev).synchronize()
    _assert_bits(xa.cpu().numpy(), oracle.fold_into(ha, hb), "fold_into beside a busy stream")
    side.synchronize()
    _assert_bits(_host(big_out), oracle.fold_stacked(big.cpu().numpy()), "the busy stream's fold")


def test_graph_replays_match_eager(env):
    """A HIP graph holding fold_ranks, fold_ranks_scaled and fold_into must give
    the eager results on every replay, with eager work and synchronizations
    between the replays."""
    df, torch, dev = env
    W, n = 8, 300_007
    host = fold_inputs.slots("mixed", W, n, 4242)
    stacked = _to_dev(torch, dev, host)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    scaled = torch.empty(n, dtype=torch.float32, device=dev)
    a0, b0 = fold_inputs.varied(n, 1, 2.0), fold_inputs.varied(n, 2, 2.0)
    xa = _to_dev(torch, dev, a0)
    xb = _to_dev(torch, dev, b0)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        df.fold_ranks(out, stacked)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        df.fold_ranks(out, stacked)
        df.fold_ranks_scaled(scaled, stacked, 0.125)
        df.fold_into(xa, xb)
    want = oracle.fold_stacked(host)
    want_s = oracle.fold_stacked_scaled(host, np.float32(0.125))
    acc = a0
    for rep in range(4):
        out.fill_(float("nan"))
        scaled.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        acc = oracle.fold_into(acc, b0)
        _assert_bits(_host(out), want, "graph replay %d fold_ranks" % rep)
        _assert_bits(_host(scaled), want_s, "graph replay %d fold_ranks_scaled" % rep)
        _assert_bits(_host(xa), acc, "graph replay %d fold_into" % rep)
        eager = torch.empty_like(out)
        df.fold_ranks(eager, stacked)  # eager work between replays
        _assert_bits(_host(eager), want, "eager between replays %d" % rep)


def _golden_cases():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "binary32_fold_cases.txt")
    cases = []
    for line in open(path):
        line = line.split(";")[0].strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        toks = lhs.split()
        inv = int(toks[-1][4:], 16) if toks[-1].startswith("inv=") else None
        ops = [int(t, 16) for t in (toks[1:-1] if inv is not None else toks[1:])]
        cases.append((toks[0], ops, inv, int(rhs.strip(), 16)))
    return cases


def test_golden_cases_on_the_device(env):
    # every hand-derived IEEE 754 case of tests/golden, through the HIP path:
    # each case's operands fill every column of a [W][1031] arena (so the row
    # body's tiles, its head and its tail all see them) and every output word
    # must be the case's expected word
    df, torch, dev = env
    n = 1031
    cases = _golden_cases()
    assert len(cases) > 40
    for kind, ops, inv, want in cases:
        what = "%s %s%s" % (kind, " ".join("%08x" % o for o in ops), " inv=%08x" % inv if inv else "")
        col = np.array(ops, dtype=np.uint32).view(np.float32)
        if kind == "into":
            dst = _to_dev(torch, dev, np.full(n, col[0], np.float32))
            stage = _to_dev(torch, dev, np.full(n, col[1], np.float32))
            df.fold_into(dst, stage)
            got = _host(dst)
        else:
            host = np.repeat(col.reshape(-1, 1), n, axis=1)
            alloc = torch.empty(host.size + 1, dtype=torch.float32, device=dev)
            for off in (0, 1):  # aligned, and shifted one element from out's phase
                stacked = alloc[off:off + host.size].view(host.shape)
                stacked.copy_(torch.from_numpy(host))
                out = torch.empty(n, dtype=torch.float32, device=dev)
                if kind.startswith("scaled"):
                    df.fold_ranks_scaled(out, stacked, float(np.array([inv], np.uint32).view(np.float32)[0]))
                else:
                    df.fold_ranks(out, stacked)
                got = _host(out)
                bad = np.flatnonzero(got.view(np.uint32) != want)
                assert bad.size == 0, "%s at +%d: got %08x want %08x" % (what, off, got.view(np.uint32)[bad[0]], want)
            continue
        bad = np.flatnonzero(got.view(np.uint32) != want)
        assert bad.size == 0, "%s: got %08x want %08x" % (what, got.view(np.uint32)[bad[0]], want)


def test_repeat_runs_are_bit_identical(env):
    # run-to-run determinism: thirty folds of one order-sensitive arena,
    # alternating between two streams and between the stacked, separate-slot
    # and scaled entry points, each into its own output; every result must
    # equal the first and the oracle, word for word
    df, torch, dev = env
    W, n = 8, (1 << 20) + 3
    host = fold_inputs.slots("mixed", W, n, 4242)
    want = oracle.fold_stacked(host)
    stacked = _to_dev(torch, dev, host)
    slots = [stacked[r] for r in range(W)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream(dev))
    outs = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(30)]
    for k, out in enumerate(outs):
        st = streams[k % 2]
        with torch.cuda.stream(st):
            if k % 3 == 0:
                df.fold_ranks(out, stacked)
            elif k % 3 == 1:
                df.fold_slots(out, slots)
            else:
                df.fold_ranks_scaled(out, stacked, 1.0)  # a multiply by one changes no bit
    torch.cuda.synchronize()
    first = _host(outs[0])
    _assert_bits(first, want, "run 0")
    for k, out in enumerate(outs[1:], 1):
        _assert_bits(_host(out), first, "run %d" % k)


def test_lengths_beyond_int32(env):
    """The pages' kernel took an i32 length; here len is 64-bit.  A W=2 fold of
    2^31 + 13 elements per slot (8 GiB each), checked on sampled outputs: 2^20
    random positions, the last 100 and the 113 around 2^31."""
    df, torch, dev = env
    n = (1 << 31) + 13
    _say("case: W=2 len=2^31+13 (16 GiB of addends)")
    host = fold_inputs.slots("vecf", 2, n, 555)
    stacked = torch.empty((2, n), dtype=torch.float32, device=dev)
    for r in range(2):
        stacked[r].copy_(torch.from_numpy(host[r]))
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(n - 100, n),
                                    np.arange((1 << 31) - 100, (1 << 31) + 13)]))
    want = oracle.fold([host[0][idx], host[1][idx]])
    idx_dev = torch.from_numpy(idx).to(dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    df.fold_ranks(out, stacked)
    _assert_bits(_host(out[idx_dev]), want, "fold_ranks at 2^31+13")
    del out
    df.fold_into(stacked[0], stacked[1])  # in place, streaming path
    _assert_bits(_host(stacked[0][idx_dev]), want, "fold_into at 2^31+13")


@pytest.mark.parametrize("W,n,off", [(32, 1 << 23, 0), (33, 3_000_001, 1), (64, 1 << 20, 2), (17, 7_000_003, 3)])
def test_wide_arena_rows_equal_direct_and_oracle(env, W, n, off):
    # beyond 16 slots the wide row body folds in passes of 16 slots; its bits
    # must equal the oracle's and both direct bodies'
    df, torch, dev = env
    host = fold_inputs.slots("varied", W, n, 7000 + W, spread=2.0)
    want = oracle.fold_stacked(host)
    want_s = oracle.fold_stacked_scaled(host, np.float32(1.0 / W))
    alloc = torch.empty(W * n + 4, dtype=torch.float32, device=dev)
    stacked = alloc[off:off + W * n].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    del host
    out = torch.empty(n, dtype=torch.float32, device=dev)
    _say("case: wide arena W=%d n=%d off=%d rows" % (W, n, off))
    df.fold_ranks(out, stacked)
    _assert_bits(_host(out), want, "W=%d rows" % W)
    df.fold_ranks_scaled(out, stacked, 1.0 / W)
    _assert_bits(_host(out), want_s, "W=%d rows scaled" % W)
    paths = [2] + ([1] if off == 0 and n % 4 == 0 else [])
    for path in paths:
        _say("case: wide arena W=%d n=%d off=%d path %d" % (W, n, off, path))
        out.fill_(float("nan"))
        df.fold_ranks_ex(out, stacked, path=path)
        _assert_bits(_host(out), want, "W=%d path %d" % (W, path))


@pytest.mark.parametrize("W", [100, 257])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 1027, 1028, 70000, 70001])
@pytest.mark.parametrize("off", [0, 1])
def test_very_wide_folds_at_small_and_ragged_lengths(env, W, n, off):
    # many passes of 16 slots (7 and 17 here, the last one partial), lengths
    # that are all head and tail, one tile, or several tiles and a tail; the
    # co-aligned cases (off 0, n a multiple of 4) take the 8-wave pass shape
    df, torch, dev = env
    host = fold_inputs.slots("mixed", W, n, 8100 + W + n)
    want = oracle.fold_stacked(host)
    want_s = oracle.fold_stacked_scaled(host, np.float32(0.5))
    alloc = torch.empty(W * n + 4, dtype=torch.float32, device=dev)
    stacked = alloc[off:off + W * n].view(W, n)
    stacked.copy_(torch.from_numpy(host))
    out = torch.empty(n + 4, dtype=torch.float32, device=dev)[(3 * off) % 4:(3 * off) % 4 + n]
    _say("case: very wide W=%d n=%d off=%d" % (W, n, off))
    out.fill_(float("nan"))
    df.fold_ranks(out, stacked)
    _assert_bits(_host(out), want, "W=%d n=%d off=%d" % (W, n, off))
    df.fold_ranks_scaled(out, stacked, 0.5)
    _assert_bits(_host(out), want_s, "W=%d n=%d off=%d scaled" % (W, n, off))
