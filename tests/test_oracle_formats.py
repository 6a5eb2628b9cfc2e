"""Pins of the oracle's number-format conversions against exact rational
rounding, numpy's float16 and torch's bfloat16."""

import numpy as np
import pytest
import torch

import oracle
from brute import exact_round_to_bf16


def _special_doubles():
    vals = [0.0, -0.0, 1.0, -1.0, 1.5, 3.0e38, -3.0e38, 1e-38, 1.1754943508222875e-38,
            2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
            1.0 + 2.0 ** -8 + 2.0 ** -40, 255.5, 256.5, 0.1, 1 / 3]
    rng = np.random.default_rng(3)
    vals += list(rng.standard_normal(2000) * np.exp(rng.uniform(-60, 60, 2000)))
    # values just around bf16 ties
    base = rng.uniform(1, 2, 500)
    q = 2.0 ** -7
    ties = (np.floor(base / q) + 0.5) * q
    vals += list(ties) + list(ties + 2.0 ** -45) + list(ties - 2.0 ** -45)
    return vals


def test_f64_to_bf16_exact_rounding():
    for x in _special_doubles():
        assert oracle.f64_to_bf16(x) == exact_round_to_bf16(x), x


def test_f64_to_bf16_agrees_with_torch_on_float32_inputs():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32)
    x[:10] = [0, -0.0, 1e-45, -1e-45, 3.4e38, 1.0, 2.0 ** -126, 2.0 ** -127, 65504, 1 + 2 ** -8]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_f32_to_f16_agrees_with_numpy():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-25, 14, 20000))).astype(np.float32)
    x[:8] = [0, -0.0, 65504, 65519.99, 65520, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26]
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(v) for v in x], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_f16_to_f32_agrees_with_numpy():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(got[~finite]) == np.isnan(ref[~finite]))


@pytest.mark.parametrize("x", [1.0, -2.5, 3.0e-39])
def test_bf16_roundtrip_of_representable(x):
    b = exact_round_to_bf16(x)
    f = (np.array([b], np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)[0]
    assert oracle.f64_to_bf16(float(f)) == b
