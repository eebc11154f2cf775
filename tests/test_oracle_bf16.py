"""Pins of the oracle's bf16 rounding (CPU only).

The oracle rounds float64 directly to bf16, ties to even.  Pins: the value
the pages print (tests/golden/bf16_pages.txt), the textbook integer form of
float32 -> bf16 rounding over every float32 pattern (and, cheaply, a sample
plus every exponent's tie neighbourhood), torch's own conversion, an exact-fraction
implementation (oracle/brute.py) on float64 inputs, and the special cases
(double rounding, subnormal ties, the normal boundary, overflow, signed zero).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_pages.txt")


def _int_rne_f32(u32: np.ndarray) -> np.ndarray:
    """Textbook float32 -> bf16 bits: add 0x7FFF + lsb, shift; NaN -> quiet."""
    u = u32.astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = (u32 & 0x7FFFFFFF) > 0x7F800000
    r[nan] = 0x7FC0
    return r


def _f32_patterns(n_random=1 << 21, seed=7):
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    # every exponent and sign, mantissa low halves around the tie point
    exps = np.arange(256, dtype=np.uint32) << 23
    lows = np.array([0x0000, 0x0001, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xFFFE,
                     0xFFFF], dtype=np.uint32)
    highs = np.array([0x00, 0x01, 0x7E, 0x7F], dtype=np.uint32) << 16
    grid = (exps[:, None, None] | highs[None, :, None] | lows[None, None, :]).ravel()
    grid = np.concatenate([grid, grid | np.uint32(0x80000000)])
    return np.concatenate([rand, grid])


def test_golden_value_from_pages():
    with open(GOLDEN) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for x_hex, bits_hex in rows:
        x = float.fromhex(x_hex)
        assert int(bf16.bits_from_f64(np.array([x]))[0]) == int(bits_hex, 16)
        assert int(bf16.bits_from_f64(np.array([x]))[0]) == 0x8000


def test_against_integer_rounding_of_f32_patterns():
    u = _f32_patterns()
    x = u.view(np.float32).astype(np.float64)
    got = bf16.bits_from_f64(x)
    want = _int_rne_f32(u)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(bf16.is_nan_bits(got[nan]))


def _sweep_chunk(lo: int, n: int) -> int:
    """Mismatches between the oracle and the integer form over float32
    patterns lo .. lo + n - 1 (NaN patterns: the oracle must give a NaN)."""
    u = np.arange(lo, lo + n, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32).astype(np.float64)
    got = bf16.bits_from_f64(x)
    want = _int_rne_f32(u)
    nan = np.isnan(x)
    bad = int(np.count_nonzero(got[~nan] != want[~nan]))
    bad += int(np.count_nonzero(~bf16.is_nan_bits(got[nan])))
    return bad


def test_every_f32_pattern():
    """All 2^32 float32 bit patterns, in chunks over the host's cores."""
    from concurrent.futures import ProcessPoolExecutor
    n = 1 << 24
    workers = max(1, min(8, os.cpu_count() or 1))
    with ProcessPoolExecutor(max_workers=workers) as ex:
        bad = sum(ex.map(_sweep_chunk, range(0, 1 << 32, n), [n] * (1 << 8)))
    assert bad == 0


def test_against_torch_conversion():
    u = _f32_patterns(n_random=1 << 20, seed=11)
    x32 = u.view(np.float32)
    fin = np.isfinite(x32)
    t = torch.from_numpy(x32[fin].copy()).to(torch.bfloat16).view(torch.int16)
    want = t.numpy().view(np.uint16)
    got = bf16.bits_from_f64(x32[fin].astype(np.float64))
    assert np.array_equal(got, want)


def test_against_exact_fractions_on_float64():
    rng = np.random.default_rng(3)
    xs = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)),
        rng.standard_normal(200) * 2.0 ** -130,
    ])
    got = bf16.round_f64(xs)
    want = np.array([brute.bf16_value(float(x)) for x in xs])
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, want)


def test_direct_rounding_from_float64_not_via_float32():
    # 1 + 2^-8 + 2^-30 lies above the bf16 tie 1 + 2^-8; float32 would first
    # drop the 2^-30 and then round the tie to even (1.0).
    x = 1 + 2.0 ** -8 + 2.0 ** -30
    assert bf16.round_f64(np.array([x]))[0] == 1 + 2.0 ** -7
    assert brute.bf16_value(x) == 1 + 2.0 ** -7


@pytest.mark.parametrize("x,expect", [
    (2.0 ** -134, 0.0),                    # half the least subnormal: tie -> 0
    (3 * 2.0 ** -134, 2.0 ** -132),        # 1.5 quanta: tie -> 2 quanta
    (127.5 * 2.0 ** -133, 2.0 ** -126),    # tie at the normal boundary -> even
    (126.5 * 2.0 ** -133, 126 * 2.0 ** -133),
    ((2 - 2.0 ** -8) * 2.0 ** 127, math.inf),           # tie past max -> inf
    ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
    ((2 - 2.0 ** -8 - 2.0 ** -20) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
    (1e39, math.inf),
    (-1e39, -math.inf),
    (1 + 2.0 ** -8, 1.0),                  # tie -> even
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),    # tie -> even (up)
])
def test_special_cases(x, expect):
    got = bf16.round_f64(np.array([x]))[0]
    assert got == expect
    assert brute.bf16_value(x) == expect


def test_signed_zero_and_nan():
    b = bf16.bits_from_f64(np.array([-0.0, 0.0, -1e-300, 1e-300, np.nan, np.inf, -np.inf]))
    assert b.tolist()[:4] == [0x8000, 0x0000, 0x8000, 0x0000]
    assert bf16.is_nan_bits(b[4:5]).all()
    assert b[5] == 0x7F80 and b[6] == 0xFF80


def test_ordered_keys_are_monotone_in_value():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    keep = ~bf16.is_nan_bits(bits)
    bits = bits[keep]
    vals = bf16.f64_from_bits(bits)
    keys = bf16.ordered(bits)
    # sort by value, -0 before +0
    order = np.lexsort((~np.signbit(vals), vals))
    assert np.all(np.diff(keys[order]) == 1)
    assert bf16.ordered(np.array([0x8000]))[0] + 1 == bf16.ordered(np.array([0x0000]))[0]


def test_bits_value_roundtrip_matches_brute_decoder():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16.f64_from_bits(bits)
    for b in list(range(0, 1 << 16, 97)) + [0x0001, 0x007F, 0x0080, 0x7F7F, 0x8001]:
        want = brute.bf16_bits_value(b)
        got = vals[b]
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want)
