"""Pins of the fp8 quantisation oracle (oracle/wan_ref.py quant_fp8_ref):
scale arithmetic in fp32, saturation of the amax element, the e4m3 error bound,
and codes against torch's float8_e4m3fn cast (a library routine)."""

import numpy as np
import torch

from oracle import wan_ref
from oracle.numerics import bf16_rne, e4m3_decode


def test_scale_special_values():
    assert wan_ref.fp8_scale(448.0) == 1.0
    assert wan_ref.fp8_scale(0.0) == 1.0
    assert wan_ref.fp8_scale(2.0) == 224.0
    assert wan_ref.fp8_scale(3.0) == float(np.float32(448.0 / 3.0))


def test_quant_codes_amax_and_error_bound():
    rng = np.random.default_rng(0)
    heads, d = 2, 128
    D = heads * d
    x = bf16_rne(rng.standard_normal((2, 40, 3 * D)) * np.array([1.0, 5.0, 0.25]).repeat(D))
    r = wan_ref.quant_fp8_ref(x, heads, d)
    for i in range(3):
        part = x[..., i * D:(i + 1) * D]
        assert r["amax"][i] == np.abs(part).max()
        codes = r["codes"][..., i * D:(i + 1) * D]
        vals = e4m3_decode(codes)
        # the largest element maps to +-448 exactly
        idx = np.unravel_index(np.argmax(np.abs(part)), part.shape)
        assert abs(vals[idx]) == 448.0
        assert np.all(np.abs(vals) <= 448.0)
        # relative error of a normal e4m3 value is at most 2**-4; subnormals 2**-10 absolute
        sc = r["scale"][i]
        err = np.abs(vals - np.float32(part * sc).astype(np.float64))
        assert np.all(err <= np.maximum(np.abs(part * sc) * 2 ** -4, 2 ** -10) * (1 + 1e-6))
        np.testing.assert_allclose(r["deq"][..., i * D:(i + 1) * D], vals / sc, rtol=1e-15)


def test_quant_codes_match_torch_cast():
    rng = np.random.default_rng(1)
    heads, d = 1, 128
    x = bf16_rne(rng.standard_normal((1, 64, 3 * heads * d)) * 3)
    r = wan_ref.quant_fp8_ref(x, heads, d)
    D = heads * d
    for i in range(3):
        part = torch.from_numpy(x[..., i * D:(i + 1) * D].astype(np.float32))
        y = (part * torch.tensor(r["scale"][i], dtype=torch.float32)).clamp(-448, 448)
        theirs = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(r["codes"][..., i * D:(i + 1) * D], theirs)


def test_all_zero_tensor():
    x = np.zeros((1, 4, 3 * 128))
    r = wan_ref.quant_fp8_ref(x, 1, 128)
    assert list(r["scale"]) == [1.0, 1.0, 1.0]
    assert np.all(r["codes"] == 0) and np.all(r["deq"] == 0)


def _normed_buffer(rng, B, grid, heads):
    D = heads * 128
    S = grid[0] * grid[1] * grid[2]
    x = bf16_rne(rng.standard_normal((B, S, 3 * D)))
    g = bf16_rne(1 + 0.1 * rng.standard_normal((2, D)))
    r = wan_ref.qknorm_rope_ref(x, g[0], g[1], grid, heads, 128)
    normed = x.copy().reshape(B * S, 3 * D)
    normed[:, :D] = r["out16_q"]
    normed[:, D:2 * D] = r["out16_k"]
    return x, g, normed.reshape(B, S, 3 * D)


def test_delayed_scale_from_the_true_amax_equals_current_scaling():
    """Given the amax of the tensors it writes (as a previous call on the same
    data reports), the delayed producer's codes, scales and amax equal the
    current-scale recipe on the norm step's output."""
    rng = np.random.default_rng(3)
    grid, heads = (2, 3, 5), 2
    x, g, normed = _normed_buffer(rng, 2, grid, heads)
    cur = wan_ref.quant_fp8_ref(normed, heads, 128)
    d = wan_ref.quant_fp8_delayed_ref(x, g[0], g[1], grid, heads, 128, cur["amax"])
    np.testing.assert_array_equal(d["codes"], cur["codes"])
    np.testing.assert_array_equal(d["scale"], cur["scale"])
    np.testing.assert_array_equal(d["amax"], cur["amax"])
    np.testing.assert_array_equal(d["deq"], cur["deq"])


def test_delayed_scale_saturates_and_follows_the_given_scale():
    """An earlier amax 4x smaller than the data's makes the scale 4x larger:
    every value beyond 448 / scale saturates to +-448 (codes 0x7E / 0xFE), the
    others are the e4m3 rounding at that scale (torch's cast, a library
    routine), and the reported amax is the data's own; amax 0 gives scale 1."""
    rng = np.random.default_rng(4)
    grid, heads = (1, 4, 6), 1
    x, g, normed = _normed_buffer(rng, 1, grid, heads)
    D = heads * 128
    true_amax = wan_ref.quant_fp8_ref(normed, heads, 128)["amax"]
    d = wan_ref.quant_fp8_delayed_ref(x, g[0], g[1], grid, heads, 128, true_amax / 4)
    np.testing.assert_array_equal(d["amax"], true_amax)
    for i in range(3):
        part = normed[..., i * D:(i + 1) * D]
        sc = d["scale"][i]
        assert sc == float(np.float32(448.0) / np.float32(true_amax[i] / 4))
        codes = d["codes"][..., i * D:(i + 1) * D]
        big = np.abs(np.float32(part * sc).astype(np.float64)) > 464.0  # past the last rounding midpoint
        assert big.any()
        assert np.all(np.isin(codes[big], [0x7E, 0xFE]))
        y = torch.from_numpy((part * sc).astype(np.float32)).clamp(-448, 448)
        np.testing.assert_array_equal(codes, y.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    z = wan_ref.quant_fp8_delayed_ref(x, g[0], g[1], grid, heads, 128, [0.0, 0.0, 0.0])
    assert list(z["scale"]) == [1.0, 1.0, 1.0]
