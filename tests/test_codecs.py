"""Pins for the oracle's stored-value decoders."""

import math

import numpy as np
import pytest
import torch

from oracle import codecs
from transformer_attention_gqa_amd import inputs


def test_e4m3fn_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125),
    (0x40, 2.0), (0xC0, -2.0), (0x7E, 448.0), (0xFE, -448.0), (0x77, 240.0)])
def test_e4m3fn_closed_form_points(code, value):
    assert codecs.e4m3fn_to_f64(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3fn_nan_codes_and_negative_zero():
    out = codecs.e4m3fn_to_f64(np.array([0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert math.isnan(out[0]) and math.isnan(out[1])
    assert out[2] == 0.0 and math.copysign(1.0, out[2]) < 0


def test_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x4049, 0x8000], dtype=np.uint16)
    out = codecs.bf16_bits_to_f64(bits)
    assert out[0] == 1.0 and out[1] == -2.0 and math.isinf(out[2])
    assert out[3] == 2.0 ** -133
    assert out[4] == 3.140625
    assert out[5] == 0.0 and math.copysign(1.0, out[5]) < 0
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    np.testing.assert_array_equal(codecs.bf16_bits_to_f64(inputs.stored_numpy(x)), x.to(torch.float64).numpy())


def test_bf16_round_to_nearest_even_of_generator():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: RNE keeps the even 1.0;
    # 1 + 3*2^-8 ties to the even 1 + 2^-6
    x = torch.tensor([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20], dtype=torch.float32)
    out = codecs.bf16_bits_to_f64(inputs.stored_numpy(x.to(torch.bfloat16)))
    assert out.tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7]


def test_dequantize_round_trip_bound():
    x = torch.randn(6, 33, 64, dtype=torch.float32)
    codes, scales = inputs.quantize_e4m3_rows(x)
    deq = codecs.dequantize_fp8_cache(codes.numpy(), scales.numpy())
    xs = x.double().numpy()
    # the row maximum maps to +-448 exactly
    amax_idx = np.abs(xs).argmax(-1)
    top = np.take_along_axis(codecs.e4m3fn_to_f64(codes.numpy()), amax_idx[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 448.0)
    # normal range: 3 mantissa bits -> relative error <= 2^-4 (plus the float32
    # rounding of x / scale)
    y = np.abs(xs) / scales.double().numpy()[..., None]
    normal = y >= 2.0 ** -6
    rel = np.abs(deq - xs)[normal] / np.abs(xs)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    # subnormal range: absolute error <= half a subnormal step (2^-10) * scale
    sub = ~normal
    if sub.any():
        absd = (np.abs(deq - xs) / scales.double().numpy()[..., None])[sub]
        assert absd.max() <= 2.0 ** -10 * (1 + 1e-6)


def test_dequantize_rejects_wrong_types():
    with pytest.raises(TypeError):
        codecs.e4m3fn_to_f64(np.zeros(3, dtype=np.int32))
    with pytest.raises(TypeError):
        codecs.dequantize_fp8_cache(np.zeros((2, 3), dtype=np.uint8), np.zeros(2, dtype=np.float64))
