"""Pins of the rounding emulators (oracle/numerics.py) against the format
definitions and against torch's own casts (library routines)."""

import numpy as np
import pytest
import torch

from oracle.numerics import (bf16_rne, bf16_neighbors, e4m3_rne_sat, e4m3_decode,
                             e4m3_encode, BF16_MAX)


def _torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_matches_torch_cast_on_random_fp32():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000),
        rng.standard_normal(20_000) * 1e-39,   # bf16 subnormals
        rng.standard_normal(20_000) * 1e30,
        rng.uniform(-1, 1, 20_000) * 3e38,
    ]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(bf16_rne(x), _torch_bf16(x))


def test_bf16_midpoints_round_to_even():
    rng = np.random.default_rng(1)
    a = np.abs(_torch_bf16(rng.standard_normal(10_000)))
    a = a[a > 0]
    lo, hi = bf16_neighbors(a)
    assert np.all(lo == a) and np.all(hi == a)
    _, e = np.frexp(a)
    ulp = np.ldexp(1.0, e - 8)          # quantum of a normal bf16 with leading bit 2**(e-1)
    up = a + ulp                         # the next bf16 above a
    mid = (a + up) / 2                   # exactly representable in fp64
    r = bf16_rne(mid)
    assert np.all((r == a) | (r == up))
    k = np.rint(r / ulp)                 # integer mantissa in units of a's quantum
    assert np.all(k % 2 == 0)            # ties go to the even mantissa
    np.testing.assert_array_equal(r, _torch_bf16(mid))
    np.testing.assert_array_equal(bf16_rne(-mid), -r)


def _bf16_code(v):
    """Sign-magnitude 16-bit pattern of a bf16 value (via torch's cast, a library routine)."""
    t = torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    c = t.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    return np.where(c & 0x8000, -(c & 0x7FFF), c)  # signed magnitude order


def test_bf16_neighbors_bracket_non_representable_values():
    """For values that are NOT bfloat16 numbers (random fp64 of both signs,
    bf16 subnormals, values just below and above powers of two), the two
    neighbours are bf16 values (torch's cast leaves them unchanged), bracket x
    strictly, are consecutive bf16 codes, and round-to-nearest picks one of
    them. A wrong quantum (off by one exponent step) or a swapped floor/ceil
    fails one of these."""
    rng = np.random.default_rng(7)
    k = rng.integers(-20, 20, 3000).astype(np.float64)
    x = np.concatenate([
        rng.standard_normal(50_000) * 10.0,
        np.abs(rng.standard_normal(5_000)) * 1e-39,      # bf16 subnormal range
        np.ldexp(1.0, k.astype(int)) * (1 - 2.0 ** -12),  # just below 2^k: quantum of the lower binade
        np.ldexp(1.0, k.astype(int)) * (1 + 2.0 ** -10),  # just above 2^k
        -np.ldexp(1.0, k.astype(int)) * (1 + 2.0 ** -10),
    ])
    x = x[bf16_rne(x) != x]                               # only non-representable values
    lo, hi = bf16_neighbors(x)
    assert np.all(lo < x) and np.all(x < hi)
    np.testing.assert_array_equal(_torch_bf16(lo), lo)
    np.testing.assert_array_equal(_torch_bf16(hi), hi)
    np.testing.assert_array_equal(_bf16_code(hi) - _bf16_code(lo), np.ones(len(x), np.int64))
    r = bf16_rne(x)
    assert np.all((r == lo) | (r == hi))
    below = np.ldexp(1.0, k.astype(int)) * (1 - 2.0 ** -12)
    blo, bhi = bf16_neighbors(below)
    np.testing.assert_array_equal(bhi, np.ldexp(1.0, k.astype(int)))           # the power of two itself
    np.testing.assert_array_equal(blo, np.ldexp(1.0, k.astype(int)) * (1 - 2.0 ** -8))


def test_bf16_overflow_and_specials():
    assert bf16_rne(np.array([BF16_MAX]))[0] == BF16_MAX
    assert np.isinf(bf16_rne(np.array([3.4e38]))[0])
    assert bf16_rne(np.array([0.0]))[0] == 0.0
    assert np.signbit(bf16_rne(np.array([-0.0]))[0])
    assert np.isnan(bf16_rne(np.array([np.nan]))[0])
    assert bf16_rne(np.array([1.0 + 2 ** -8]))[0] == 1.0           # tie -> even (1.0)
    assert bf16_rne(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6  # tie -> even


def test_e4m3_decode_from_format_definition():
    codes = np.arange(256)
    v = e4m3_decode(codes)
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)  # monotone over the finite positive codes
    assert np.isnan(v).sum() == 2


def test_e4m3_encode_decode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    v = e4m3_decode(codes)
    np.testing.assert_array_equal(e4m3_encode(v), codes.astype(np.uint8))
    np.testing.assert_array_equal(e4m3_rne_sat(v), v)


def test_e4m3_midpoints_round_to_even_code():
    v = e4m3_decode(np.arange(0x00, 0x7F))
    mid = (v[:-1] + v[1:]) / 2
    r = e4m3_encode(e4m3_rne_sat(mid)).astype(np.int64)
    lo = np.arange(0x00, 0x7E)
    assert np.all((r == lo) | (r == lo + 1))
    assert np.all(r % 2 == 0)   # the even neighbour has mantissa LSB 0
    # just off the midpoint goes to the nearer code
    np.testing.assert_array_equal(e4m3_encode(e4m3_rne_sat(np.nextafter(mid, 0))), lo)
    np.testing.assert_array_equal(e4m3_encode(e4m3_rne_sat(np.nextafter(mid, 1e9))), lo + 1)


def test_e4m3_saturates():
    x = np.array([448.0, 460.0, 470.0, 1e6, -1e6, -449.0])
    np.testing.assert_array_equal(e4m3_rne_sat(x), [448, 448, 448, 448, -448, -448])


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100_000) * 50,
                        rng.standard_normal(20_000) * 1e-2,
                        rng.uniform(-448, 448, 20_000)]).astype(np.float32).astype(np.float64)
    ours = e4m3_encode(e4m3_rne_sat(x))
    theirs = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)
