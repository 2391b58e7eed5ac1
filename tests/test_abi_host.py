"""Host-side checks of the C-ABI library (CPU only; nothing is launched).

The library must load, export every function ``include/detfold.h`` declares,
reject bad arguments before touching the device, and plan the path and
geometry the kernels assume.  Every call here either fails validation or has
nothing to do, so no fake address is ever handed to a kernel.
"""
import ctypes
import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "detfold.h")

KiB = 1024
BASE = 0x7F0000000000  # a 4 KiB-aligned fake device address, never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("fold_ranks", "fold_into", "fold_ranks_scaled", "detfold_strerror"):
        assert required in names


def test_library_exports_every_declared_function(detfold_lib):
    lib = detfold_lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), "libdetfold.so does not export %s" % name
    assert set(detfold_lib.EXPORTS) == set(_declared_functions())


def test_library_exports_nothing_but_the_c_abi(detfold_lib):
    # the link's version script keeps every internal symbol local
    import subprocess
    res = subprocess.run(["nm", "-D", "--defined-only", detfold_lib.LIB_PATH], capture_output=True,
                         text=True, check=True)
    exported = {line.split()[-1] for line in res.stdout.splitlines() if line.strip()}
    assert exported == set(_declared_functions())


def test_abi_version(detfold_lib):
    assert detfold_lib.load().detfold_abi_version() == detfold_lib.ABI_VERSION == 12


def test_strerror_covers_every_code(detfold_lib):
    seen = set()
    for rc in range(0, 7):
        s = detfold_lib.strerror(rc)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in detfold_lib.strerror(99)


# --------------------------------------------------------------------------
# argument validation happens before any HIP call

def test_rejects_bad_arguments_without_a_device(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    out, st = BASE, BASE + 64 * KiB * KiB
    assert lib.fold_ranks(out, st, 0, 16, None) == EINVAL            # W = 0
    assert lib.fold_ranks(out, st, -3, 16, None) == EINVAL
    assert lib.fold_ranks(out, st, 4, -1, None) == EINVAL            # negative length
    assert lib.fold_ranks(None, st, 4, 16, None) == EINVAL           # NULL
    assert lib.fold_ranks(out, None, 4, 16, None) == EINVAL
    assert lib.fold_ranks(out + 2, st, 4, 16, None) == EINVAL        # not 4-byte aligned
    assert lib.fold_ranks(out, st + 1, 4, 16, None) == EINVAL
    assert lib.fold_ranks(out, st, 4, (1 << 62), None) == EINVAL     # W*len*4 overflows
    assert lib.fold_ranks(st + 8, st, 4, 16, None) == EOVERLAP       # out inside stacked
    assert lib.fold_ranks(st - 4, st, 4, 16, None) == EOVERLAP       # out straddles the start
    assert lib.fold_ranks(st + 4 * 64 - 4, st, 4, 16, None) == EOVERLAP  # last element
    assert lib.fold_ranks_scaled(out, st, 0, 16, ctypes.c_float(0.5), None) == EINVAL
    assert lib.fold_ranks_scaled(st, st, 2, 16, ctypes.c_float(0.5), None) == EOVERLAP
    assert lib.fold_into(out, st, -1, None) == EINVAL
    assert lib.fold_into(None, st, 8, None) == EINVAL
    assert lib.fold_into(out, out + 16, 8, None) == EOVERLAP         # stage inside dst
    assert lib.fold_into(out, out, 8, None) == EOVERLAP
    # zero elements: nothing to do, no launch, even with NULL pointers
    assert lib.fold_ranks(None, None, 8, 0, None) == OK
    assert lib.fold_ranks_scaled(None, None, 1, 0, ctypes.c_float(1.0), None) == OK
    assert lib.fold_into(None, None, 0, None) == OK
    # W is still checked when there is nothing to fold
    assert lib.fold_ranks(None, None, 0, 0, None) == EINVAL


def test_rejects_bad_launch_overrides(detfold_lib):
    lib = detfold_lib.load()
    L = detfold_lib.Launch
    out, st = BASE, BASE + 64 * KiB * KiB
    for bad in (L(4, 0, 0, 0, 0), L(-1, 0, 0, 0, 0), L(0, 65, 0, 0, 0), L(0, 32, 0, 0, 0),
                L(0, 2048, 0, 0, 0), L(0, 0, -1, 0, 0), L(0, 0, 1 << 40, 0, 0), L(0, 0, 0, 3, 0),
                L(0, 0, 0, 8, 0), L(0, 0, 0, 0, 3), L(0, 0, 0, 0, -1), L(0, 0, 0, 2, 2)):
        rc = lib.detfold_fold_ranks_ex(out, st, 8, 16, 0, ctypes.c_float(1.0), ctypes.byref(bad), None)
        assert rc == detfold_lib.EINVAL
        rc = lib.detfold_fold_ranks_ex(out, st, 8, 0, 0, ctypes.c_float(1.0), ctypes.byref(bad), None)
        assert rc == detfold_lib.EINVAL, "a bad override is rejected even with nothing to fold"
    # forcing the vector body where the slots are not co-aligned
    vec = L(detfold_lib.PATH_VECTOR, 0, 0, 0, 0)
    rc = lib.detfold_fold_ranks_ex(out, st + 4, 8, 16, 0, ctypes.c_float(1.0), ctypes.byref(vec), None)
    assert rc == detfold_lib.EINVAL


# --------------------------------------------------------------------------
# planning (pure host logic)

CU = 256


def test_plan_w8_64mib_per_slot(detfold_lib):
    n = 1 << 24
    p = detfold_lib.plan_fold_ranks(BASE, BASE + 4 * n + 4096, 8, n, CU)
    # LDS row body: one wave per slot, each streaming 2 KiB of its slot per tile
    assert p["path"] == detfold_lib.PATH_ROWS
    assert (p["head"], p["tail"], p["body"]) == (0, 0, n // 4)
    assert p["block"] == 512 and p["tile"] == 128
    assert p["grid"] == (n // 4) // 128 == 32768
    assert p["policy"] == detfold_lib.POLICY_STREAM


@pytest.mark.parametrize("W", [2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 14, 16])
def test_plan_rows_tile_per_width(detfold_lib, W):
    # a slot length that is a multiple of 2^24 and slots shifted 4 bytes from
    # out's 16-byte phase: one slot per wave of ceil(W/4) KiB (8 KiB at two
    # slots) up to six slots and at eight, two slots per wave of 1 KiB at
    # seven and from nine up (eight waves at 13 and 14)
    n = 1 << 24
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 32) + 4, W, n, CU)
    assert p["path"] == detfold_lib.PATH_ROWS
    assert (p["block"], p["tile"], p["group"]) == _rule_shape(W, n, False)
    if W <= 6 or W == 8:
        assert p["block"] == 64 * W and p["tile"] == 64 * (8 if W == 2 else -(-W // 4))
    else:
        assert p["block"] == 64 * (8 if W in (13, 14) else -(-W // 2)) and p["tile"] == 64
    assert p["grid"] == -(-(n // 4) // p["tile"])


def _rows_waves(W, spw):
    """Waves of a row-body workgroup: W with one slot per wave; with two,
    ceil(W/2), but eight at 13 and 14 slots (workgroups of seven waves fill
    only 28 of a CU's 32 wave slots)."""
    return 8 if spw == 2 and W in (13, 14) else -(-W // spw)


def _rule_shape(W, n, coaligned):
    """The row-body shape and XCD group the plan should pick for a stacked
    arena of W slots of n floats (slot stride n*4 bytes).  Slots per wave:
    eight slots take one where n is a multiple of 2^24 or the slots do not
    repeat the address bits below 16 MiB, else two; seven and nine to sixteen
    take two; five and six take two only when co-aligned and repeating.  XCD
    group: shifted slots take runs of 32 tiles (8 at three and four slots that
    do not repeat); co-aligned ones plain round-robin when repeating, else
    runs of 32 from five to ten slots and of 8 otherwise."""
    repeat = (n * 4) % (1 << 24) == 0
    if W < 5 or W > 16:
        spw = 1
    elif W == 8:
        spw = 1 if (n % (1 << 24) == 0 or not repeat) else 2
    elif W == 7 or W >= 9:
        spw = 2
    else:
        spw = 2 if (coaligned and repeat) else 1
    if W < 3 or W > 16:
        group = 1
    elif not coaligned:
        group = 8 if (W <= 4 and not repeat) else 32
    elif repeat:
        group = 1
    else:
        group = 32 if 5 <= W <= 10 else 8
    block = 64 * _rows_waves(W, spw)
    tile = 64 * (1 if spw == 2 else (8 if W <= 2 else -(-W // 4)))
    return block, tile, group


@pytest.mark.parametrize("n,spw", [(1 << 24, 1), (1 << 25, 1), (3 << 24, 1), (1 << 22, 2), (1 << 23, 2),
                                   ((1 << 24) + 4, 1), (10_000_000, 1), (12_000_001, 1), (1 << 26, 1),
                                   (6_291_456, 1)])
def test_plan_eight_slot_shape_follows_the_slot_length(detfold_lib, n, spw):
    # W = 8: one slot per wave (8 waves x 2 KiB) at slot lengths that are
    # multiples of 2^24 floats and at lengths whose slots do not repeat the
    # low 16 MiB of address (the latter with runs of 32 tiles per XCD); two
    # slots per wave (4 waves x 1 KiB each) at the other multiples of 2^22
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34), 8, n, CU)
    assert p["path"] == detfold_lib.PATH_ROWS
    assert (p["block"], p["tile"]) == ((512, 128) if spw == 1 else (256, 64))
    assert (p["block"], p["tile"], p["group"]) == _rule_shape(8, n, True)
    assert p["grid"] == -(-p["body"] // p["tile"])
    # an override may name either shape by its workgroup size, and nothing else
    other = 256 if spw == 1 else 512
    q = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34), 8, n, CU,
                                    dict(path=detfold_lib.PATH_ROWS, block=other, grid=0, unroll=0, policy=0))
    assert (q["block"], q["tile"]) == ((512, 128) if other == 512 else (256, 64))
    for bad in (128, 384, 448, 1024):
        with pytest.raises(detfold_lib.DetfoldError):
            detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34), 8, n, CU,
                                        dict(path=detfold_lib.PATH_ROWS, block=bad, grid=0, unroll=0, policy=0))
    # the other widths, co-aligned and with slot 0 four bytes off out's phase
    for W in (2, 3, 4, 5, 6, 7, 9, 10, 12, 13, 14, 15, 16):
        for shift in (0, 4):
            q = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34) + shift, W, n, CU)
            co = shift == 0 and n % 4 == 0
            assert (q["block"], q["tile"], q["group"]) == _rule_shape(W, n, co), (W, n, shift)


@pytest.mark.parametrize("W", [1, 17, 24])
@pytest.mark.parametrize("n,block", [(1 << 20, 512), (1 << 19, 512), (1 << 18, 256), (1 << 16, 64),
                                     (4096, 64), (4, 64)])
def test_plan_direct_block_shrinks_to_cover_the_chip(detfold_lib, W, n, block):
    # W = 1 takes the direct vector body by default; wider folds only when asked
    launch = None if W == 1 else dict(path=detfold_lib.PATH_VECTOR, block=0, grid=0, unroll=0, policy=0)
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), W, n, CU, launch)
    assert p["path"] == detfold_lib.PATH_VECTOR
    assert p["block"] == block and p["tile"] == block
    assert p["grid"] == max(1, -(-p["body"] // block))


def test_plan_w4_gradient_arena(detfold_lib):
    n = 100_000_000
    p = detfold_lib.plan_fold_ranks(BASE, BASE + 4 * n + 4096, 4, n, CU)
    assert p["path"] == detfold_lib.PATH_ROWS and p["body"] == n // 4 and p["tail"] == 0
    assert p["block"] == 256 and p["tile"] == 64 and p["grid"] == -(-(n // 4) // 64)
    assert p["group"] == 8  # 4e8-byte slots do not repeat the low 16 MiB of address


def test_plan_w16_offset_arena(detfold_lib):
    n = 10_000_019
    stacked = BASE + 4 * n + 4096 + 4  # one element past an aligned allocation
    # slot phases cycle through all four offsets: no direct 16-byte body ...
    phases = {((stacked + 4 * r * n) >> 2) & 3 for r in range(16)}
    assert phases == {0, 1, 2, 3}
    with pytest.raises(detfold_lib.DetfoldError):
        detfold_lib.plan_fold_ranks(BASE, stacked, 16, n, CU, dict(path=detfold_lib.PATH_VECTOR,
                                                                   block=0, grid=0, unroll=0, policy=0))
    # ... but the LDS row body loads each slot's tile from its own dword: 16-byte
    # groups of out, 3 tail elements
    p = detfold_lib.plan_fold_ranks(BASE, stacked, 16, n, CU)
    assert p["path"] == detfold_lib.PATH_ROWS
    assert (p["head"], p["body"], p["tail"]) == (0, n // 4, 3)
    # two slots per wave (8 waves x 1 KiB each), runs of 32 tiles per XCD
    assert (p["block"], p["tile"], p["group"]) == (512, 64, 32)
    # the direct scalar body stays available
    p = detfold_lib.plan_fold_ranks(BASE, stacked, 16, n, CU, dict(path=detfold_lib.PATH_SCALAR,
                                                                   block=0, grid=0, unroll=0, policy=0))
    assert p["path"] == detfold_lib.PATH_SCALAR and p["body"] == n


@pytest.mark.parametrize("phase_out,phase_in,n", [(1, 1, 64), (2, 2, 4096), (3, 3, 8), (0, 0, 3),
                                                   (1, 1, 2), (3, 3, 0)])
def test_plan_head_and_tail(detfold_lib, phase_out, phase_in, n):
    out = BASE + 4 * phase_out
    st = BASE + (1 << 30) + 4 * phase_in
    W = 4 if n % 4 == 0 else 1  # several slots share a phase only when len % 4 == 0
    p = detfold_lib.plan_fold_ranks(out, st, W, n, CU)
    assert p["path"] == (detfold_lib.PATH_ROWS if W > 1 else detfold_lib.PATH_VECTOR)
    head = min((4 - phase_out) % 4, n)
    assert p["head"] == head
    assert p["body"] == (n - head) // 4 and p["tail"] == (n - head) % 4
    assert p["head"] + 4 * p["body"] + p["tail"] == n
    if n:
        assert p["grid"] >= 1


def test_plan_ragged_length_with_several_slots(detfold_lib):
    # len % 4 != 0 puts slot 1 at another 16-byte phase than slot 0: the row
    # body takes it as it is, the direct bodies fall back to 4-byte loads
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 2, 1001, CU)
    assert p["path"] == detfold_lib.PATH_ROWS and (p["body"], p["tail"]) == (250, 1)
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 17, 1001, CU)
    assert p["path"] == detfold_lib.PATH_ROWS and (p["body"], p["tail"]) == (250, 1)
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 17, 1001, CU,
                                    dict(path=detfold_lib.PATH_AUTO, block=0, grid=0, unroll=0,
                                         policy=detfold_lib.POLICY_CACHED))
    assert p["path"] == detfold_lib.PATH_SCALAR  # the unhinted direct body, 4-byte loads
    # one slot: only out and slot 0 matter
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 1, 1001, CU)
    assert p["path"] == detfold_lib.PATH_VECTOR and p["tail"] == 1


def test_plan_override(detfold_lib):
    n = 1 << 20
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 8, n, CU,
                                    dict(path=detfold_lib.PATH_SCALAR, block=1024, grid=7, unroll=4))
    assert (p["path"], p["block"], p["grid"], p["unroll"]) == (detfold_lib.PATH_SCALAR, 1024, 7, 4)
    assert p["body"] == n
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 8, n, CU,
                                    dict(path=0, block=0, grid=0, unroll=0,
                                         policy=detfold_lib.POLICY_CACHED))
    # the unhinted policy has only the direct bodies
    assert p["policy"] == detfold_lib.POLICY_CACHED and p["unroll"] == 1
    assert p["path"] == detfold_lib.PATH_VECTOR
    # 2^20 is not a multiple of 2^24: the eight-slot row body with two slots per wave
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), 8, n, CU,
                                    dict(path=detfold_lib.PATH_ROWS, block=256, grid=5, unroll=1,
                                         policy=0))
    assert (p["path"], p["block"], p["grid"], p["tile"]) == (detfold_lib.PATH_ROWS, 256, 5, 64)


@pytest.mark.parametrize("W,launch", [(8, dict(block=384)), (8, dict(unroll=2)), (4, dict(block=128)),
                                      (8, dict(policy=2)), (1, {}), (17, dict(block=256)),
                                      (24, dict(unroll=2)), (8, dict(group=-1)), (8, dict(group=65)),
                                      (8, dict(group=3)), (8, dict(group=128))])
def test_plan_rejects_impossible_row_overrides(detfold_lib, W, launch):
    cfg = dict(path=detfold_lib.PATH_ROWS, block=0, grid=0, unroll=0, policy=0)
    cfg.update(launch)
    with pytest.raises(detfold_lib.DetfoldError):
        detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 30), W, 1 << 20, CU, cfg)


@pytest.mark.parametrize("n", [1, 4, 1024, 4096, 16384, 65536])
def test_plan_decode_join_is_one_pass(detfold_lib, n):
    p = detfold_lib.plan_fold_into(BASE, BASE + (1 << 20), n, CU)
    assert p["unroll"] == 1 and p["policy"] == detfold_lib.POLICY_CACHED
    # every position gets its own thread: one pass, no grid-stride loop
    assert p["grid"] * p["block"] >= p["body"]
    assert p["grid"] == max(1, -(-p["body"] // p["block"]))
    if n == 4096:
        assert p["path"] == detfold_lib.PATH_VECTOR and p["block"] == 64 and p["grid"] == 16


def test_plan_large_in_place_fold_streams(detfold_lib):
    p = detfold_lib.plan_fold_into(BASE, BASE + (1 << 32), 100_000_000, CU)
    assert p["policy"] == detfold_lib.POLICY_STREAM and p["path"] == detfold_lib.PATH_ROWS
    assert p["block"] == 128 and p["tile"] == 512 and p["grid"] == -(-25_000_000 // 512)


# --------------------------------------------------------------------------
# owner shards

@pytest.mark.parametrize("n,world", [(10_000_019, 16), (0, 4), (3, 8), (16, 16), (1 << 24, 8), (7, 1)])
def test_shard_plan_covers_contiguously_and_balanced(detfold_lib, n, world):
    plan = detfold_lib.shard_plan(n, world)
    assert len(plan) == world
    pos = 0
    for start, ln in plan:
        assert start == pos and ln >= 0
        pos += ln
    assert pos == n
    lens = [ln for _, ln in plan]
    assert max(lens) - min(lens) <= 1
    assert lens == sorted(lens, reverse=True)


def test_shard_plan_for_the_offset_arena(detfold_lib):
    lens = [ln for _, ln in detfold_lib.shard_plan(10_000_019, 16)]
    assert lens == [625_002] * 3 + [625_001] * 13


def test_shard_plan_rejects_bad_world(detfold_lib):
    with pytest.raises(detfold_lib.DetfoldError):
        detfold_lib.shard_plan(10, 0)
    lib = detfold_lib.load()
    a = (ctypes.c_int64 * 2)()
    assert lib.detfold_shard_plan(-1, 2, a, a) == detfold_lib.EINVAL
    assert lib.detfold_shard_plan(5, 2, None, a) == detfold_lib.EINVAL


# --------------------------------------------------------------------------
# separate slots, rounds and the two-stream link: argument checks only

def _ptrs(*addrs):
    return (ctypes.c_void_p * len(addrs))(*addrs)


def test_fold_slots_rejects_bad_arguments(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    a, b, out = BASE, BASE + (1 << 20), BASE + (1 << 21)
    assert lib.fold_slots(out, _ptrs(a, b), 0, 16, None) == EINVAL
    assert lib.fold_slots(out, _ptrs(*[a] * 17), 17, 16, None) == EINVAL   # more than 16 slots
    assert lib.fold_slots(out, None, 2, 16, None) == EINVAL
    assert lib.fold_slots(out, _ptrs(a, None), 2, 16, None) == EINVAL
    assert lib.fold_slots(out, _ptrs(a, b + 2), 2, 16, None) == EINVAL   # misaligned slot
    assert lib.fold_slots(out + 1, _ptrs(a, b), 2, 16, None) == EINVAL
    assert lib.fold_slots(out, _ptrs(a, b), 2, -1, None) == EINVAL
    assert lib.fold_slots(a + 4, _ptrs(a, b), 2, 16, None) == EOVERLAP   # partial overlap with slot 0
    assert lib.fold_slots(b - 4, _ptrs(a, b), 2, 16, None) == EOVERLAP
    assert lib.fold_slots_scaled(a + 8, _ptrs(a, b), 2, 16, ctypes.c_float(0.5), None) == EOVERLAP
    assert lib.fold_slots(None, None, 3, 0, None) == OK                 # nothing to do


def test_loopback_round_rejects_bad_arguments(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    n = 1000
    ar = [BASE + i * (1 << 20) for i in range(4)]
    stage = BASE + (1 << 30)
    need = detfold_lib.round_stage_elems(n, 4)
    assert need == 1000
    assert lib.detfold_loopback_round(_ptrs(*ar), 0, n, stage, need, 0, None) == EINVAL
    assert lib.detfold_loopback_round(_ptrs(*[BASE + i * (1 << 20) for i in range(17)]), 17, n, stage,
                                      10 ** 6, 0, None) == EINVAL
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, -1, stage, need, 0, None) == EINVAL
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, n, stage, need, 8, None) == EINVAL     # unknown flag
    fused = detfold_lib.ROUND_FUSED
    for other in (detfold_lib.ROUND_DIRECT, detfold_lib.ROUND_REVERSE_DELIVERY):
        assert lib.detfold_loopback_round(_ptrs(*ar), 4, n, None, 0, fused | other, None) == EINVAL
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, n, stage, need - 1, 0, None) == EINVAL  # stage short
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, n, None, 0, 0, None) == EINVAL
    assert lib.detfold_loopback_round(_ptrs(ar[0], ar[1], ar[1] + 8, ar[3]), 4, n, stage, need, 0,
                                      None) == EOVERLAP                                   # arenas overlap
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, n, ar[2] + 100, need, 0, None) == EOVERLAP
    assert lib.detfold_loopback_round(_ptrs(*ar[:1]), 1, n, None, 0, 0, None) == OK        # one rank
    assert lib.detfold_loopback_round(_ptrs(*ar), 4, 0, None, 0, 0, None) == OK            # empty
    # direct and fused modes need no stage, but still check the arenas
    for mode in (detfold_lib.ROUND_DIRECT, fused):
        assert lib.detfold_loopback_round(_ptrs(ar[0], ar[0], ar[2], ar[3]), 4, n, None, 0,
                                          mode, None) == EOVERLAP
        assert lib.detfold_loopback_round(_ptrs(ar[0], ar[1] + 2, ar[2], ar[3]), 4, n, None, 0,
                                          mode, None) == EINVAL                     # misaligned arena
    assert lib.detfold_loopback_round(_ptrs(*ar[:1]), 1, n, None, 0, fused, None) == OK    # one rank


def test_pair_all_reduce_rejects_bad_arguments(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    link = detfold_lib.PairLinkC()
    link.capacity = 4096
    link.stage[0], link.stage[1] = BASE, BASE + (1 << 20)
    x0, x1 = BASE + (2 << 20), BASE + (3 << 20)
    assert lib.detfold_pair_all_reduce(None, x0, x1, 16) == EINVAL
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0, x1, 16) == EINVAL      # no events
    assert lib.detfold_pair_link_init(ctypes.byref(link)) == EINVAL
    for i in range(2):  # fake event handles: never passed to HIP by the checks below
        link.pushed[i], link.folded[i] = 0x1000 + i, 0x2000 + i
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0, x1, 4097) == EINVAL    # over capacity
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0, x1, -1) == EINVAL
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0, x0 + 4, 16) == EOVERLAP
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), BASE + 8, x1, 16) == EOVERLAP  # x0 vs stage 0
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0 + 2, x1, 16) == EINVAL  # misaligned
    assert lib.detfold_pair_all_reduce(ctypes.byref(link), x0, x1, 0) == OK           # nothing to do


def test_pair_broadcast_and_all_gather_reject_bad_arguments(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    link = detfold_lib.PairLinkC()
    src, dst = BASE, BASE + (1 << 20)
    assert lib.detfold_pair_broadcast(None, 0, src, dst, 16) == EINVAL
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 0, src, dst, 16) == EINVAL   # no events
    for i in range(2):  # fake event handles: never passed to HIP by the checks below
        link.pushed[i], link.folded[i] = 0x1000 + i, 0x2000 + i
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 2, src, dst, 16) == EINVAL   # no rank 2
    assert lib.detfold_pair_broadcast(ctypes.byref(link), -1, src, dst, 16) == EINVAL
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 0, src, dst, -1) == EINVAL
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 0, None, dst, 16) == EINVAL
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 1, src, dst + 1, 16) == EINVAL  # misaligned
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 1, src, src + 60, 16) == EOVERLAP
    assert lib.detfold_pair_broadcast(ctypes.byref(link), 0, src, dst, 0) == OK        # nothing to do
    x0, x1, f0, f1 = BASE, BASE + (1 << 20), BASE + (2 << 20), BASE + (3 << 20)
    assert lib.detfold_pair_all_gather(None, x0, x1, f0, f1, 16) == EINVAL
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, x1, f0, f1, -1) == EINVAL
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, None, f0, f1, 16) == EINVAL
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, x1, f0 + 2, f1, 16) == EINVAL
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, x1, f0, f0 + 64, 16) == EOVERLAP  # f0 is 128 B
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, f1 + 100, f0, f1, 16) == EOVERLAP
    assert lib.detfold_pair_all_gather(ctypes.byref(link), f0 + 64, x1, f0, f1, 16) == EOVERLAP
    assert lib.detfold_pair_all_gather(ctypes.byref(link), x0, x1, f0, f1, 0) == OK


def test_one_shot_rejects_bad_arguments(detfold_lib):
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.OK
    assert detfold_lib.ONE_SHOT_FLAG_WORDS == 256
    link = detfold_lib.OneShotLinkC()
    link.capacity = 4096
    link.stage[0], link.stage[1] = BASE, BASE + (1 << 20)
    x0, x1 = BASE + (2 << 20), BASE + (3 << 20)
    ar = lib.detfold_one_shot_all_reduce
    assert ar(None, x0, x1, 16) == EINVAL
    assert ar(ctypes.byref(link), x0, x1, 16) == EINVAL                  # no flags or words
    assert lib.detfold_one_shot_init(ctypes.byref(link)) == EINVAL
    link.flags, link.words = BASE + (4 << 20), BASE + (5 << 20)
    link.spin_limit = -1
    assert ar(ctypes.byref(link), x0, x1, 16) == EINVAL                  # negative spin limit
    assert lib.detfold_one_shot_init(ctypes.byref(link)) == EINVAL
    link.spin_limit = 0
    link.words = link.flags + 4 * 255                                     # words inside the counters
    assert ar(ctypes.byref(link), x0, x1, 16) == EOVERLAP
    assert lib.detfold_one_shot_init(ctypes.byref(link)) == EOVERLAP
    link.words = link.flags + 4 * 256                                     # right after them: fine
    link.flags += 2
    assert ar(ctypes.byref(link), x0, x1, 16) == EINVAL                  # misaligned counters
    link.flags -= 2
    assert ar(ctypes.byref(link), x0, x1, 4097) == EINVAL                # over capacity
    assert ar(ctypes.byref(link), x0, x1, -1) == EINVAL
    assert ar(ctypes.byref(link), x0, x0 + 4, 16) == EOVERLAP
    assert ar(ctypes.byref(link), BASE + 8, x1, 16) == EOVERLAP          # x0 vs stage 0
    assert ar(ctypes.byref(link), x0 + 1, x1, 16) == EINVAL              # misaligned
    assert ar(ctypes.byref(link), x0, x1, 0) == OK                       # nothing to do
    rk = lib.detfold_one_shot_rank
    assert rk(ctypes.byref(link), 2, x0, 16, None) == EINVAL
    assert rk(ctypes.byref(link), -1, x0, 16, None) == EINVAL
    assert rk(ctypes.byref(link), 1, BASE + (1 << 20) + 32, 16, None) == EOVERLAP  # x vs stage 1
    assert rk(ctypes.byref(link), 0, x0, 4097, None) == EINVAL
    assert rk(ctypes.byref(link), 0, x0, 0, None) == OK


@pytest.mark.parametrize("W", [17, 24, 32, 33, 64, 100])
@pytest.mark.parametrize("n", [1 << 22, 10_000_019, 4099])
def test_plan_wide_rows(detfold_lib, W, n):
    # beyond 16 slots: passes of 16 slots -- 8 waves x 2 slots x 1 KiB over
    # 64-group tiles when out and every slot share one 16-byte phase, or when
    # the slots repeat the low 16 MiB of address and the last pass holds at
    # least 8 slots, else 16 waves x 1 slot x 4 KiB over 256-group tiles;
    # shifted slots take runs of tiles per XCD (32 where they repeat, else
    # 16), co-aligned wide arenas plain round-robin
    repeat = (n * 4) % (1 << 24) == 0 and (W % 16 == 0 or W % 16 >= 8)
    for out, stacked in ((BASE, BASE + (1 << 36)), (BASE + 4, BASE + (1 << 36) + 12)):
        aligned = out % 16 == stacked % 16 and n % 4 == 0
        p = detfold_lib.plan_fold_ranks(out, stacked, W, n, CU)
        assert p["path"] == detfold_lib.PATH_ROWS
        assert (p["block"], p["tile"], p["unroll"]) == ((512, 64, 1) if aligned or repeat else (1024, 256, 1))
        assert p["group"] == (1 if aligned else 32 if (n * 4) % (1 << 24) == 0 else 16)
        assert p["grid"] == max(1, -(-p["body"] // p["tile"]))
        assert p["head"] + 4 * p["body"] + p["tail"] == n
    p = detfold_lib.plan_fold_ranks(BASE + 4, BASE + (1 << 36) + 12, W, n, CU,
                                    dict(path=detfold_lib.PATH_ROWS, block=1024, grid=3, unroll=0, policy=0))
    assert (p["block"], p["grid"]) == (1024, 3)


@pytest.mark.parametrize("n", [1 << 22, 1 << 24, 3 << 20, 6_000_000, 10_000_000, 10_000_019])
def test_plan_sixteen_slot_shape_follows_alignment(detfold_lib, n):
    # W = 16: two slots per wave (8 waves x 1 KiB each) on every stacked
    # arena; co-aligned slots take runs of 8 tiles per XCD where they do not
    # repeat the low 16 MiB of address (plain round-robin where they do),
    # shifted slots runs of 32
    repeat = (n * 4) % (1 << 24) == 0
    p = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34), 16, n, CU)
    if n % 4:  # slot r at phase r*n mod 4: shifted slots
        assert (p["block"], p["tile"], p["group"]) == (512, 64, 32)
    else:
        assert (p["block"], p["tile"], p["group"]) == ((512, 64, 1) if repeat else (512, 64, 8))
    q = detfold_lib.plan_fold_ranks(BASE, BASE + (1 << 34) + 4, 16, n, CU)  # slot 0 shifted
    assert (q["block"], q["tile"], q["group"]) == (512, 64, 32)
    for plan in (p, q):
        assert plan["path"] == detfold_lib.PATH_ROWS
        assert plan["grid"] == -(-plan["body"] // plan["tile"])


def test_static_round_rejects_before_any_device_work(detfold_lib):
    # every rejection here happens before the library looks up its stage
    lib = detfold_lib.load()
    EINVAL, EOVERLAP, ESIZE, OK = detfold_lib.EINVAL, detfold_lib.EOVERLAP, detfold_lib.ESIZE, detfold_lib.OK
    cap = detfold_lib.STATIC_STAGE_FLOATS
    ar = [BASE + i * (1 << 26) for i in range(4)]
    for flags in (detfold_lib.ROUND_DIRECT, detfold_lib.ROUND_FUSED, 8,
                  detfold_lib.ROUND_DIRECT | detfold_lib.ROUND_REVERSE_DELIVERY):
        assert lib.detfold_loopback_round_static(_ptrs(*ar), 4, 1000, flags, None) == EINVAL
    assert lib.detfold_loopback_round_static(_ptrs(*ar), 0, 1000, 0, None) == EINVAL
    assert lib.detfold_loopback_round_static(_ptrs(*ar), 4, -1, 0, None) == EINVAL
    assert lib.detfold_loopback_round_static(_ptrs(ar[0], ar[1] + 2, ar[2], ar[3]), 4, 1000, 0, None) == EINVAL
    assert lib.detfold_loopback_round_static(_ptrs(ar[0], ar[0] + 8, ar[2], ar[3]), 4, 1000, 0,
                                             None) == EOVERLAP
    assert lib.detfold_loopback_round_static(_ptrs(*ar), 4, cap + 1, 0, None) == ESIZE
    assert lib.detfold_loopback_round_static(_ptrs(*ar[:3]), 3, cap, 1, None) == ESIZE  # 3*ceil(n/3) > cap
    assert lib.detfold_loopback_round_static(_ptrs(*ar[:1]), 1, 10 ** 9, 0, None) == OK  # one rank
    assert lib.detfold_loopback_round_static(_ptrs(*ar), 4, 0, 0, None) == OK            # empty
    assert "static stage" in detfold_lib.strerror(ESIZE)


# --------------------------------------------------------------------------
# the batched fold: argument checks and its one-launch plan

def _jobs(detfold_lib, *jobs):
    arr = (detfold_lib.FoldJob * max(len(jobs), 1))()
    for j, (o, st, n) in enumerate(jobs):
        arr[j].out, arr[j].stacked, arr[j].len = o, st, n
    return arr


def test_batch_rejects_bad_arguments(detfold_lib):
    df = detfold_lib
    lib = df.load()
    EINVAL, EOVERLAP, OK = df.EINVAL, df.EOVERLAP, df.OK
    M = 1 << 24  # bytes between fake buffers
    o = [BASE + k * M for k in range(4)]
    st = [BASE + (1 << 32) + k * 16 * M for k in range(4)]
    good = _jobs(df, (o[0], st[0], 1000), (o[1], st[1], 1000))
    assert lib.fold_ranks_batch(good, 2, 0, None) == EINVAL                        # W < 1
    assert lib.fold_ranks_batch(good, -1, 4, None) == EINVAL
    assert lib.fold_ranks_batch(good, df.MAX_JOBS + 1, 4, None) == EINVAL        # too many jobs
    assert lib.fold_ranks_batch(None, 2, 4, None) == EINVAL
    assert lib.fold_ranks_batch(None, 0, 4, None) == OK                          # nothing to do
    assert lib.fold_ranks_batch(_jobs(df, (o[0], st[0], 0), (0, 0, 0)), 2, 4, None) == OK
    assert lib.fold_ranks_batch(_jobs(df, (o[0], st[0], -1)), 1, 4, None) == EINVAL
    assert lib.fold_ranks_batch(_jobs(df, (o[0] + 2, st[0], 16)), 1, 4, None) == EINVAL   # misaligned
    assert lib.fold_ranks_batch(_jobs(df, (0, st[0], 16)), 1, 4, None) == EINVAL          # NULL out
    assert lib.fold_ranks_batch(_jobs(df, (st[0] + 64, st[0], 1000)), 1, 4, None) == EOVERLAP  # own arena
    # one job's output inside another job's output or arena
    assert lib.fold_ranks_batch(_jobs(df, (o[0], st[0], 1000), (o[0] + 3996, st[1], 1000)), 2, 4,
                                None) == EOVERLAP
    assert lib.fold_ranks_batch(_jobs(df, (o[0], st[0], 1000), (st[0] + 8000, st[1], 1000)), 2, 4,
                                None) == EOVERLAP
    # adjacent outputs, and arenas shared between jobs, are fine to plan
    p = df.plan_fold_ranks_batch([(o[0], st[0], 1000), (o[0] + 4000, st[0], 1000)], 4, 256)
    assert p["grid"] >= 2
    assert lib.fold_ranks_batch_scaled(good, 2, 0, ctypes.c_float(0.5), None) == EINVAL
    # a slot pitch: 0 (packed) or at least len; the arena spans (W-1)*pitch + len
    j = _jobs(df, (o[0], st[0], 1000))
    j[0].pitch = 999
    assert lib.fold_ranks_batch(j, 1, 4, None) == EINVAL
    j[0].pitch = -1
    assert lib.fold_ranks_batch(j, 1, 4, None) == EINVAL
    j[0].pitch = 2 ** 61
    assert lib.fold_ranks_batch(j, 1, 4, None) == EINVAL                          # span overflows
    j = _jobs(df, (st[0] + 3 * 4096 * 4 + 64, st[0], 1000))                       # inside slot 3 at pitch 4096
    j[0].pitch = 4096
    assert lib.fold_ranks_batch(j, 1, 4, None) == EOVERLAP
    j[0].pitch = 0                                                                # packed: past the arena
    assert df.plan_fold_ranks_batch([(st[0] + 3 * 4096 * 4 + 64, st[0], 1000)], 4, 256)["grid"] >= 1
    # a padded arena spans 3*5000 + 1000 floats, its padding included: another
    # job's output may start right after it, not inside it
    assert df.plan_fold_ranks_batch([(o[0], st[0], 1000, 5000), (st[0] + 4 * 16_000, st[1], 1000)], 4,
                                    256)["grid"] >= 2
    for inside in (5_500, 12_000, 15_999):
        with pytest.raises(df.DetfoldError):
            df.plan_fold_ranks_batch([(o[0], st[0], 1000, 5000), (st[0] + 4 * inside, st[1], 1000)], 4, 256)


def test_batch_plan_covers_every_job(detfold_lib):
    df = detfold_lib
    # the owner shards of a W=16 arena of 10,000,019: 3 x 625,002 and 13 x 625,001 per
    # owner, each gathered into its own [16][l_p] scratch, written at the owners' offsets
    shards = df.shard_plan(10_000_019, 16)
    out = BASE
    scratch = BASE + (1 << 34)
    jobs, s_addr = [], scratch
    for s, ln in shards:
        jobs.append((out + 4 * s, s_addr, ln))
        s_addr += 16 * ln * 4 + 4096
    p = df.plan_fold_ranks_batch(jobs, 16, 256)
    assert p["path"] == df.PATH_ROWS
    # the shape is the one the longest shard would get alone
    alone = df.plan_fold_ranks(jobs[0][0], jobs[0][1], 16, jobs[0][2], 256)
    assert p["block"] == alone["block"] and p["tile"] == alone["tile"]
    want_grid, want_body = 0, 0
    for o, _, ln in jobs:
        head = min((4 - (o // 4) % 4) % 4, ln)
        groups = (ln - head) // 4
        want_grid += max(1, -(-groups // p["tile"]))
        want_body += groups
    assert p["grid"] == want_grid and p["body"] == want_body
    # an element-less job takes no workgroup; a job of 1..3 elements takes one
    q = df.plan_fold_ranks_batch([(BASE, scratch, 0), (BASE + 64, scratch + 4096, 3),
                                  (BASE + 4096, scratch + 8192, 5)], 4, 256)
    assert q["grid"] == 2
    assert df.plan_fold_ranks_batch([(BASE, scratch, 0)], 4, 256)["grid"] == 0
    with pytest.raises(df.DetfoldError):
        df.plan_fold_ranks_batch([(BASE, scratch, 10)], 1, 256)   # one launch needs 2 <= W <= 16
    with pytest.raises(df.DetfoldError):
        df.plan_fold_ranks_batch([(BASE, scratch, 10)], 17, 256)


def test_plan_row_shapes_by_block_and_group(detfold_lib):
    df = detfold_lib
    rows = dict(path=df.PATH_ROWS, grid=0, unroll=0, policy=0)
    for W in range(5, 17):
        n = 1_000_003
        one = df.plan_fold_ranks(BASE, BASE + (1 << 34) + 4, W, n, CU, dict(rows, block=64 * W))
        two = df.plan_fold_ranks(BASE, BASE + (1 << 34) + 4, W, n, CU, dict(rows, block=64 * _rows_waves(W, 2)))
        assert one["tile"] == 64 * (-(-W // 4)) and two["tile"] == 64
        assert two["grid"] == -(-two["body"] // 64)
        if W in (13, 14):  # seven waves name no shape: the two-slot shape has eight
            with pytest.raises(df.DetfoldError):
                df.plan_fold_ranks(BASE, BASE + (1 << 34) + 4, W, n, CU, dict(rows, block=448))
    for W in (2, 3, 4):
        with pytest.raises(df.DetfoldError):
            df.plan_fold_ranks(BASE, BASE + (1 << 34), W, 1000, CU, dict(rows, block=64 * (-(-W // 2))))
    for W, block, tile in ((17, 1024, 256), (17, 512, 64), (64, 512, 64)):
        p = df.plan_fold_ranks(BASE, BASE + (1 << 34), W, 1 << 20, CU, dict(rows, block=block))
        assert (p["block"], p["tile"]) == (block, tile)
    # the XCD group: the plan's own choice, or the override's
    p = df.plan_fold_ranks(BASE, BASE + (1 << 34), 16, 10_000_019, CU)
    assert p["group"] >= 1
    for g in (1, 2, 8, 64):
        q = df.plan_fold_ranks(BASE, BASE + (1 << 34), 16, 10_000_019, CU, dict(rows, block=0, group=g))
        assert q["group"] == g
    assert df.plan_fold_into(BASE, BASE + (1 << 20), 4096, CU)["group"] == 1


def test_pair_link_refuses_stream_capture_before_any_call(detfold_lib, monkeypatch):
    # the pair link cannot be captured into a graph: with the current stream
    # capturing, every call raises before it touches a stream or the library
    import torch
    link = object.__new__(detfold_lib.PairLink)  # no device needed to reach the check
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(detfold_lib.DetfoldError) as e:
        link._fork()
    assert e.value.rc == detfold_lib.ECAPTURE
    assert "captured" in detfold_lib.strerror(detfold_lib.ECAPTURE)


def test_batch_plan_follows_the_pitch(detfold_lib):
    # the shape rule reads the slot pitch: 625,002-float slots packed sit at
    # alternating 16-byte phases and repeat no low 16 MiB of address (runs of
    # 32 tiles per XCD); padded to 2^22 floats (16 MiB) apart they are
    # co-aligned and repeat it (plain round-robin)
    df = detfold_lib
    packed = df.plan_fold_ranks_batch([(BASE, BASE + (1 << 34), 625_002)], 16, 256)
    padded = df.plan_fold_ranks_batch([(BASE, BASE + (1 << 34), 625_002, 1 << 22)], 16, 256)
    assert (packed["block"], packed["tile"], packed["group"]) == (512, 64, 32)
    assert (padded["block"], padded["tile"], padded["group"]) == (512, 64, 1)
    assert packed["body"] == padded["body"] and packed["grid"] == padded["grid"]
