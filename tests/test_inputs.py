"""Self-checks of the seeded input generators (CPU only).

The C generators are compared with an independent big-integer model of the
same xorshift stream (memra-engine tests/tp_ar_gpu.rs, helper `vecf`;
memra-engine tests/gdn_packed_gpu.rs, helper `varied`), and the value grids
and ranges the fold's tests rely on are checked.
"""
from fractions import Fraction

import numpy as np
import pytest

import fold_inputs

M64 = (1 << 64) - 1


def _stream(seed, n):
    x = (seed * 0x9E3779B97F4A7C15 & M64) | 1
    for _ in range(n):
        x ^= (x << 13) & M64
        x ^= x >> 7
        x ^= (x << 17) & M64
        yield x


def _vecf_model(n, seed):
    # ((x >> 40) / 2^24 - 0.5) * 2, computed exactly
    return [float((Fraction(x >> 40, 1 << 24) - Fraction(1, 2)) * 2) for x in _stream(seed, n)]


def _mixed_model(n, seed):
    out = []
    for x in _stream(seed, n):
        sign = x >> 63
        mant = (x >> 40) & 0x7FFFFF
        e = ((x & 0xFFFFFFFF) * 41 >> 32) - 20
        out.append((sign << 31) | ((e + 127) << 23) | mant)
    return out


def _varied_model(n, seed, spread):
    out = []
    for x in _stream(seed, n):
        u = float(Fraction(x >> 11, 1 << 53) * 2 - 1)  # exact in binary64
        out.append(np.float32(u) * np.float32(spread))
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("seed", [0, 1, 5, 6, 11 + 4096, 77 + 65536, 1000, 2**63 + 12345])
def test_vecf_matches_stream_model(seed):
    got = fold_inputs.vecf(300, seed)
    want = np.array(_vecf_model(300, seed), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("seed", [2000, 2003, 7])
def test_mixed_matches_stream_model(seed):
    got = fold_inputs.mixed(300, seed).view(np.uint32)
    assert got.tolist() == _mixed_model(300, seed)


@pytest.mark.parametrize("spread", [1.0, 3.5, 1e-3])
def test_varied_matches_stream_model(spread):
    got = fold_inputs.varied(300, 42, spread)
    want = _varied_model(300, 42, spread)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_vecf_grid_and_range():
    v = fold_inputs.vecf(1 << 18, 1234)
    assert v.min() >= -1.0 and v.max() < 1.0
    k = v.astype(np.float64) * 2.0**23
    assert np.array_equal(k, np.round(k)), "every value is a multiple of 2^-23"
    assert abs(float(v.mean())) < 0.01
    # uniform: each quarter of [-1, 1) holds about a quarter of the values
    h, _ = np.histogram(v, bins=4, range=(-1.0, 1.0))
    assert np.all(np.abs(h / v.size - 0.25) < 0.01)


def test_mixed_exponent_range_and_signs():
    b = fold_inputs.mixed(1 << 18, 99).view(np.uint32)
    e = ((b >> 23) & 0xFF).astype(np.int64) - 127
    assert e.min() == -20 and e.max() == 20
    counts = np.bincount(e + 20, minlength=41)
    assert np.all(counts > 0.8 * b.size / 41)
    assert 0.45 < float((b >> 31).mean()) < 0.55


def test_slots_use_consecutive_seeds():
    s = fold_inputs.slots("vecf", 5, 1000, 3000)
    for r in range(5):
        assert np.array_equal(s[r].view(np.uint32), fold_inputs.vecf(1000, 3000 + r).view(np.uint32))
    m = fold_inputs.slots("mixed", 3, 500, 2000)
    for r in range(3):
        assert np.array_equal(m[r].view(np.uint32), fold_inputs.mixed(500, 2000 + r).view(np.uint32))


def test_different_seeds_differ():
    a = fold_inputs.vecf(4096, 5)
    b = fold_inputs.vecf(4096, 6)
    assert np.count_nonzero(a != b) > 4000
