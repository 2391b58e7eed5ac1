"""Pins for the CPU oracle (CPU only; no GPU, no HIP library).

The oracle (``oracle/``) is trusted as the parity reference only because it is
pinned here to things other than itself:

* hand-derived IEEE 754 binary32 cases (``tests/golden/binary32_fold_cases.txt``);
* an exact-rational brute force with an explicit round-to-nearest-even
  (``tests/binary32_exact.py``) on tiny inputs from every input family;
* the binary64 double path: ``float32(float64(acc) + float64(x))`` per step,
  which equals the binary32 sum because double rounding of a sum is innocuous
  when the wider format has at least 2p+2 significand bits (53 >= 2*24+2;
  S. A. Figueroa, "When is double rounding innocuous?", SIGNUM Newsletter 1995);
* closed forms: x + x = 2x, power-of-two scales, exact sums of the uniform
  generator, a one-slot fold is a bit copy;
* invariants of the method (mamba-rs src/dist/reducer.rs, FixedOrder-contract
  module note and `LoopbackWorld`; memra-engine tests/tp_ar_gpu.rs): doubling on
  a second fold, a dropped addend diverges, split independence, chained
  two-addend folds equal one W-slot fold;
* planted mistakes: mutants of the oracle that each pin must catch.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import binary32_exact as bx
import fold_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "binary32_fold_cases.txt")


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _load_golden():
    cases = []
    for line in open(GOLDEN):
        line = line.split(";")[0].strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        toks = lhs.split()
        kind, ops = toks[0], toks[1:]
        inv = None
        if ops and ops[-1].startswith("inv="):
            inv = int(ops[-1][4:], 16)
            ops = ops[:-1]
        cases.append((kind, [int(o, 16) for o in ops], inv, int(rhs.strip(), 16)))
    return cases


GOLDEN_CASES = _load_golden()


# --------------------------------------------------------------------------
# families of tiny inputs for the brute force

SPECIALS = [0x00000000, 0x80000000, 0x3F800000, 0xBF800000, 0x33800000, 0xB3800000,
            0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00800000, 0x80800000,
            0x7F7FFFFF, 0xFF7FFFFF, 0x4B800000, 0x3F800001, 0x3F7FFFFF, 0x34000000,
            0x00000003, 0x00400000, 0x7F000000, 0xFF000000]


def _tiny_family(kind, W, n, seed):
    if kind == "vecf":
        return fold_inputs.slots("vecf", W, n, seed)
    if kind == "varied":
        return fold_inputs.slots("varied", W, n, seed, spread=3.0)
    if kind == "mixed":
        return fold_inputs.slots("mixed", W, n, seed)
    if kind == "special":
        rng = np.random.default_rng(seed)
        picks = rng.integers(0, len(SPECIALS), size=(W, n))
        b = np.array(SPECIALS, dtype=np.uint32)[picks]
        # mix in some mixed-magnitude values so carries and cancellations vary
        m = fold_inputs.slots("mixed", W, n, seed).view(np.uint32)
        sel = rng.random((W, n)) < 0.3
        b = np.where(sel, m, b)
        return b.view(np.float32)
    if kind == "subnormal":
        rng = np.random.default_rng(seed)
        exp = rng.integers(0, 3, size=(W, n)).astype(np.uint32)
        mant = rng.integers(0, 1 << 23, size=(W, n)).astype(np.uint32)
        sign = rng.integers(0, 2, size=(W, n)).astype(np.uint32)
        return ((sign << 31) | (exp << 23) | mant).view(np.float32)
    raise ValueError(kind)


def _brute(stacked):
    return bx.fold([[int(v) for v in row] for row in _bits(stacked)])


def _brute_scaled(stacked, inv):
    return bx.fold_scaled([[int(v) for v in row] for row in _bits(stacked)],
                          int(_bits(np.float32(inv))))


def _same_bits(got, want):
    got = [int(v) for v in _bits(got)]
    return all(bx.same(g, w) for g, w in zip(got, want)) and len(got) == len(want)


def _double_path(stacked):
    s = np.asarray(stacked, dtype=np.float32)
    acc = s[0].astype(np.float64)
    # A double sum beyond the binary32 range rounds to +-inf in the cast: that is
    # the rounding each step of the chain must take, so numpy's overflow warning
    # is expected here and silenced.
    with np.errstate(over="ignore"):
        for r in range(1, s.shape[0]):
            acc = (acc + s[r].astype(np.float64)).astype(np.float32).astype(np.float64)
    return acc.astype(np.float32)


# --------------------------------------------------------------------------
# the pin suite, reusable against mutants

def _pin_failures(fold_fn, scaled_fn):
    """Run golden + brute-force + double-path pins; return the names that fail."""
    failed = []
    for kind, ops, inv, want in GOLDEN_CASES:
        if kind == "into":
            continue
        S = _f32(ops).reshape(len(ops), 1)
        got = scaled_fn(S, _f32([inv])[0]) if kind.startswith("scaled") else fold_fn(S)
        if not bx.same(int(_bits(got)[0]), want):
            failed.append("golden:%s:%s" % (kind, " ".join("%08x" % o for o in ops)))
    for kind in ("vecf", "varied", "mixed", "special", "subnormal"):
        for W in (1, 2, 3, 5, 8, 16):
            S = _tiny_family(kind, W, 24, 17 * W + len(kind))
            if not _same_bits(fold_fn(S), _brute(S)):
                failed.append("brute:%s:W%d" % (kind, W))
            if W in (2, 4, 8, 16) or kind == "subnormal":
                inv = np.float32(1.0 / W) if W in (2, 4, 8, 16) else np.float32(0.5)
                if not _same_bits(scaled_fn(S, inv), _brute_scaled(S, inv)):
                    failed.append("brute-scaled:%s:W%d" % (kind, W))
    for kind, W in (("varied", 8), ("mixed", 4), ("vecf", 16)):
        S = _tiny_family(kind, W, 4096, 99 + W)
        if not np.array_equal(_bits(fold_fn(S)), _bits(_double_path(S))):
            failed.append("double-path:%s:W%d" % (kind, W))
    return failed


# --------------------------------------------------------------------------
# the brute-force checker itself is checked against the machine's conversion

def test_exact_rounding_model_agrees_with_numpy_conversion():
    rng = np.random.default_rng(0)
    # binary64 values in every binary32 regime, including ties and overflow
    d = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-45, 39, 2000),
        (np.arange(1, 200) * 2.0**-150),                     # subnormal ties
        1.0 + np.arange(0, 64) * 2.0**-26,                    # around 1, ties included
        np.array([3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2.0**-25)]),
    ])
    with np.errstate(over="ignore"):
        want = d.astype(np.float32).view(np.uint32)
    for x, w in zip(d.tolist(), want.tolist()):
        assert bx.round_rne(Fraction(x), 1 if x < 0 else 0) == w, x


def test_exact_model_reproduces_golden_cases():
    for kind, ops, inv, want in GOLDEN_CASES:
        if kind.startswith("scaled"):
            got = bx.fold_scaled([[o] for o in ops], inv)[0]
        elif kind == "into":
            got = bx.add(ops[0], ops[1])
        else:
            got = bx.fold([[o] for o in ops])[0]
        assert got == want, (kind, ops)


# --------------------------------------------------------------------------
# the oracle against the pins

@pytest.mark.parametrize("case", GOLDEN_CASES, ids=lambda c: c[0] + ":" + "-".join("%08x" % o for o in c[1]))
def test_oracle_golden(case):
    kind, ops, inv, want = case
    if kind == "into":
        got = oracle.fold_into(_f32([ops[0]]), _f32([ops[1]]))
    elif kind.startswith("scaled"):
        got = oracle.fold_stacked_scaled(_f32(ops).reshape(len(ops), 1), _f32([inv])[0])
    else:
        got = oracle.fold_stacked(_f32(ops).reshape(len(ops), 1))
    assert "%08x" % int(_bits(got)[0]) == "%08x" % want


@pytest.mark.parametrize("kind", ["vecf", "varied", "mixed", "special", "subnormal"])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 7, 8, 16])
def test_oracle_matches_bruteforce(kind, W):
    for seed in range(3):
        n = [1, 13, 64][seed]
        S = _tiny_family(kind, W, n, 1000 * W + seed)
        assert _same_bits(oracle.fold_stacked(S), _brute(S))
        slots = [S[r] for r in range(W)]
        assert _same_bits(oracle.fold(slots), _brute(S))
        inv = np.float32(0.25)
        assert _same_bits(oracle.fold_stacked_scaled(S, inv), _brute_scaled(S, inv))


@pytest.mark.parametrize("kind,W", [("vecf", 8), ("mixed", 4), ("vecf", 16), ("varied", 8),
                                    ("subnormal", 8), ("special", 5)])
def test_oracle_matches_double_path(kind, W):
    S = _tiny_family(kind, W, 1 << 16, 7 + W)
    assert np.array_equal(_bits(oracle.fold_stacked(S)), _bits(_double_path(S)))


def test_oracle_into_matches_bruteforce():
    for kind in ("vecf", "varied", "mixed", "special", "subnormal"):
        S = _tiny_family(kind, 2, 64, 5)
        got = oracle.fold_into(S[0], S[1])
        want = [bx.add(int(a), int(b)) for a, b in zip(_bits(S[0]), _bits(S[1]))]
        assert _same_bits(got, want)


# --------------------------------------------------------------------------
# closed forms

def _twice_bits(b):
    """2x by bit manipulation for finite x whose double is finite."""
    b = b.astype(np.uint64)
    sign = b & 0x80000000
    mag = b & 0x7FFFFFFF
    normal = (mag >> 23) > 0
    return np.where(normal, b + (1 << 23), sign | (mag * 2)).astype(np.uint32)


def test_second_fold_is_exact_double():
    # memra-engine tests/tp_ar_gpu.rs: both ranks hold the sum, so a second
    # reduce gives S + S = 2S exactly.
    for kind in ("vecf", "varied", "mixed", "subnormal"):
        S = _tiny_family(kind, 2, 1 << 14, 3)
        s = oracle.fold_stacked(S)
        again = oracle.fold_into(s, s)
        assert np.array_equal(_bits(again), _twice_bits(_bits(s)))


def test_two_uniform_addends_sum_exactly():
    # vecf values are multiples of 2^-23 in [-1, 1): every two-addend sum is
    # representable, so the oracle must equal the exact rational sum.
    a = fold_inputs.vecf(4096, 4107)
    b = fold_inputs.vecf(4096, 4173)
    got = oracle.fold_into(a, b)
    for x, y, g in zip(a.tolist(), b.tolist(), got.tolist()):
        assert Fraction(g) == Fraction(x) + Fraction(y)


def test_one_slot_is_a_bit_copy():
    for kind in ("special", "subnormal", "mixed"):
        S = _tiny_family(kind, 1, 4096, 11)
        assert np.array_equal(_bits(oracle.fold_stacked(S)), _bits(S[0]))


@pytest.mark.parametrize("W,k", [(2, 1), (4, 2), (8, 3), (16, 4)])
def test_power_of_two_scale_is_exact_and_equals_division(W, k):
    S = _tiny_family("mixed", W, 1 << 14, 50 + W)
    s = _bits(oracle.fold_stacked(S))
    scaled = _bits(oracle.fold_stacked_scaled(S, np.float32(2.0**-k)))
    expo = (s >> 23) & 0xFF
    ok = expo > k  # results that stay normal: exponent field drops by k
    assert ok.mean() > 0.99
    assert np.array_equal(scaled[ok], s[ok] - (k << 23))
    # one rounding of the exact real sum/W, whatever the regime
    div = (s.view(np.float32) / np.float32(W)).view(np.uint32)
    assert np.array_equal(scaled, div)
    # subnormal sums too
    T = _tiny_family("subnormal", W, 1 << 14, 60 + W)
    t = oracle.fold_stacked(T)
    assert np.array_equal(_bits(oracle.fold_stacked_scaled(T, np.float32(2.0**-k))),
                          _bits(t / np.float32(W)))


# --------------------------------------------------------------------------
# invariants of the method

def test_into_is_the_two_slot_fold():
    a, b = fold_inputs.varied(5000, 1), fold_inputs.varied(5000, 2)
    assert np.array_equal(_bits(oracle.fold_into(a, b)), _bits(oracle.fold([a, b])))


def test_chained_into_equals_stacked_fold():
    # memra-engine tests/gdn_packed_gpu.rs: one W-slot launch must equal the
    # chain of per-step launches bit for bit; the accumulator is binary32
    # between steps either way.
    S = _tiny_family("mixed", 8, 1 << 15, 77)
    acc = S[0].copy()
    for r in range(1, 8):
        acc = oracle.fold_into(acc, S[r])
    assert np.array_equal(_bits(acc), _bits(oracle.fold_stacked(S)))


def test_split_independence():
    # mamba-rs src/dist/reducer.rs: owner shards are folded separately; the
    # bits cannot depend on where the arena is cut.
    S = _tiny_family("vecf", 16, 10007, 3000)
    whole = oracle.fold_stacked(S)
    cuts = [0, 1, 626, 1251, 5000, 10006, 10007]
    parts = [oracle.fold_stacked(np.ascontiguousarray(S[:, a:b])) for a, b in zip(cuts, cuts[1:])]
    assert np.array_equal(_bits(np.concatenate(parts)), _bits(whole))


def test_dropped_addend_diverges():
    # memra-engine tests/tp_ar_gpu.rs red arm: a fold missing one addend must
    # not reproduce the sum.
    a, b = fold_inputs.vecf(4096, 5), fold_inputs.vecf(4096, 6)
    want = oracle.fold([a, b])
    got = oracle.fold_into(a, np.zeros_like(b))
    assert np.count_nonzero(_bits(got) == _bits(want)) < 4096
    S = fold_inputs.slots("vecf", 8, 1 << 14, 1000)
    assert np.count_nonzero(_bits(oracle.fold_stacked(S[:7])) != _bits(oracle.fold_stacked(S))) > 0


@pytest.mark.parametrize("family,W,seed0", [("vecf", 8, 1000), ("mixed", 4, 2000), ("vecf", 16, 3000)])
def test_order_matters_on_the_test_inputs(family, W, seed0):
    """Non-vacuity: ascending and descending chains must differ on a share of
    elements, or bitwise agreement would not show the order was kept."""
    S = fold_inputs.slots(family, W, 1 << 16, seed0)
    up = _bits(oracle.fold_stacked(S))
    down = _bits(oracle.fold_stacked(np.ascontiguousarray(S[::-1])))
    frac = float(np.count_nonzero(up != down)) / up.size
    print("order-sensitive share %s W=%d: %.3f" % (family, W, frac))
    assert frac > 0.05


# --------------------------------------------------------------------------
# planted mistakes: every mutant must fail at least one pin

def _np_chain(S, order):
    acc = S[order[0]].copy()
    for r in order[1:]:
        acc = (acc + S[r]).astype(np.float32)
    return acc


def _ftz(x):
    b = _bits(x)
    sub = ((b >> 23) & 0xFF) == 0
    return np.where(sub, b & 0x80000000, b).astype(np.uint32).view(np.float32)


def _pairwise(S):
    rows = [S[r].copy() for r in range(S.shape[0])]
    while len(rows) > 1:
        nxt = [(rows[i] + rows[i + 1]).astype(np.float32) for i in range(0, len(rows) - 1, 2)]
        if len(rows) % 2:
            nxt.append(rows[-1])
        rows = nxt
    return rows[0]


MUTANTS = {
    "reversed order": lambda S: _np_chain(S, list(range(S.shape[0]))[::-1]),
    "starts from +0": lambda S: _np_chain(np.concatenate([np.zeros((1, S.shape[1]), np.float32), S]),
                                          list(range(S.shape[0] + 1))),
    "drops last addend": lambda S: _np_chain(S, list(range(max(1, S.shape[0] - 1)))),
    "reads slot r-1 twice": lambda S: _np_chain(S, [0] + [max(1, r - 1) if r == 2 else r
                                                          for r in range(1, S.shape[0])]),
    "flushes subnormals": lambda S: _ftz(_np_chain_ftz(S)),
    "binary64 accumulator": lambda S: S.astype(np.float64).sum(axis=0).astype(np.float32),
    "pairwise tree": _pairwise,
}


def _np_chain_ftz(S):
    acc = _ftz(S[0])
    for r in range(1, S.shape[0]):
        acc = _ftz((acc + _ftz(S[r])).astype(np.float32))
    return acc


def _oracle_scaled(S, inv):
    return oracle.fold_stacked_scaled(S, inv)


def test_pins_accept_the_oracle():
    assert _pin_failures(oracle.fold_stacked, _oracle_scaled) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name):
    fn = MUTANTS[name]

    def scaled(S, inv):
        return (fn(S) * np.float32(inv)).astype(np.float32)

    with np.errstate(over="ignore", invalid="ignore"):
        failed = _pin_failures(fn, scaled)
    assert failed, "mutant %r passed every pin" % name


def test_pins_reject_scale_before_sum():
    def scaled(S, inv):
        return _np_chain((S * np.float32(inv)).astype(np.float32), list(range(S.shape[0])))

    with np.errstate(over="ignore", invalid="ignore"):
        failed = _pin_failures(oracle.fold_stacked, scaled)
    assert failed


def test_pins_reject_divide_by_the_width():
    # the scale multiplies by the caller's inverse (one rounding of sum*inv);
    # a mutant that divides by the width the inverse names (round(1/inv))
    # agrees whenever inv is a power of two, so only the hand-derived golden
    # case 2+2+1 times RN(1/3) tells the two apart
    def scaled(S, inv):
        return (oracle.fold_stacked(S) / np.float32(round(1.0 / float(inv)))).astype(np.float32)

    with np.errstate(over="ignore", invalid="ignore"):
        failed = _pin_failures(oracle.fold_stacked, scaled)
    assert failed == ["golden:scaled3:40000000 40000000 3f800000"], failed


def test_oracle_on_disjoint_ranges_equals_the_whole_fold():
    # the host oracle run on contiguous element ranges (as the threaded CPU
    # baseline does, one range per thread) gives the whole fold's bits: the
    # chain is per element, so the split cannot matter
    import threading
    W, n = 7, 100_003
    host = fold_inputs.slots("varied", W, n, 91, spread=3.0)
    want = oracle.fold_stacked(host)
    T = 5
    bounds = [(n * t // T, n * (t + 1) // T) for t in range(T)]
    parts = [None] * T

    def work(t):
        a, b = bounds[t]
        parts[t] = oracle.fold([host[r, a:b] for r in range(W)])

    pool = [threading.Thread(target=work, args=(t,)) for t in range(T)]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    got = np.concatenate(parts)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
