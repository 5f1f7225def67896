"""Rounding emulators written from the format definitions (fp64 in, fp64 out).

Test infrastructure only (see the package docstring).

The method has one named rounding point: the RMSNorm output is rounded to
bfloat16 before the fp32 rotary multiplication, and the rotary output is
rounded to bfloat16 again when it is stored ("Optimize Wan2.2 Dataflow" pull
request, section "Fused Q/K Norm and RoPE" under Numerical Behavior). The fp8
configuration quantises Q, K and V to E4M3 with a per-tensor scale derived from
the amax (same page, section 2 "Fuse Wan ApproximateGELU With FP8
Quantization": amax, then the E4M3 inverse scale, then the cast). The pages do
not name a rounding mode; round-to-nearest-even is the IEEE default and is the
reading taken here, with saturation (never NaN) for e4m3.

Both emulators work on the exact value: the input is scaled by a power of two
(exact in binary floating point) so that one quantum of the target format
becomes 1.0, rounded half-to-even with ``numpy.rint``, and scaled back.
"""

import numpy as np

# bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits.
BF16_MANT_BITS = 7
BF16_MIN_NORMAL_EXP = -126
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127

# OCP FP8 E4M3 ("fn" variant): 1 sign bit, 4 exponent bits (bias 7), 3 stored
# mantissa bits, no infinities, exponent field 15 with mantissa 7 is NaN, so the
# largest finite magnitude is 1.75 * 2**8 = 448 and the smallest subnormal is
# 2**-9.
E4M3_MANT_BITS = 3
E4M3_BIAS = 7
E4M3_MIN_NORMAL_EXP = 1 - E4M3_BIAS  # -6
E4M3_MAX = 448.0


def _round_to_quantum(x, mant_bits, min_normal_exp):
    """Round x (fp64) to the nearest value with ``mant_bits`` stored mantissa
    bits, ties to even; below 2**min_normal_exp the quantum is fixed
    (gradual underflow)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2**e with 0.5 <= |m| < 1, so the leading bit is 2**(e-1)
    # A normal number with leading bit 2**(e-1) has quantum 2**(e-1-mant_bits).
    q = np.maximum(e - 1 - mant_bits, min_normal_exp - mant_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def bf16_rne(x):
    """Nearest bfloat16 value (ties to even) of each element, as fp64.
    Magnitudes that round past the largest finite bfloat16 become +-inf."""
    y = _round_to_quantum(x, BF16_MANT_BITS, BF16_MIN_NORMAL_EXP)
    with np.errstate(invalid="ignore"):
        return np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, y), y)


def bf16_neighbors(x):
    """The two bfloat16 values that bracket x (lo <= x <= hi); equal when x is
    itself representable. Used to build the candidate sets at rounding ties."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 1 - BF16_MANT_BITS, BF16_MIN_NORMAL_EXP - BF16_MANT_BITS)
    s = np.ldexp(x, -q)
    return np.ldexp(np.floor(s), q), np.ldexp(np.ceil(s), q)


def e4m3_rne_sat(x):
    """Nearest OCP e4m3 value (ties to even), saturating to +-448, as fp64."""
    y = _round_to_quantum(x, E4M3_MANT_BITS, E4M3_MIN_NORMAL_EXP)
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_decode(codes):
    """Value of each 8-bit e4m3 code, straight from the bit-field definition.
    NaN codes (S.1111.111) decode to NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    normal = np.ldexp(1.0 + mf / 8.0, ef - E4M3_BIAS)
    sub = np.ldexp(mf / 8.0, E4M3_MIN_NORMAL_EXP)
    v = sign * np.where(ef == 0, sub, normal)
    return np.where((ef == 15) & (mf == 7), np.nan, v)


def e4m3_encode(v):
    """8-bit code of an fp64 value that is already an e4m3 value (the output of
    ``e4m3_rne_sat``). Zero encodes with its sign bit (negative zero -> 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    _, e = np.frexp(a)
    lead = e - 1  # exponent of the leading bit
    is_normal = a >= 2.0 ** E4M3_MIN_NORMAL_EXP
    ef_normal = lead + E4M3_BIAS
    mf_normal = np.rint(np.ldexp(a, -lead) * 8.0 - 8.0)
    mf_sub = np.rint(np.ldexp(a, -E4M3_MIN_NORMAL_EXP) * 8.0)
    ef = np.where(is_normal, ef_normal, 0)
    mf = np.where(is_normal, mf_normal, mf_sub)
    return (sign | (ef.astype(np.int64) << 3) | mf.astype(np.int64)).astype(np.uint8)


def f32(x):
    """Round fp64 to IEEE binary32 (round to nearest even) and widen back."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
