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
