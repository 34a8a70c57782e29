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


# ---- int8 / int4 caches ("KV cache quantization": INT8 / INT4 with scales)

def test_int8_codes_are_their_own_values():
    codes = np.arange(-128, 128, dtype=np.int8)
    assert codecs.int8_to_f64(codes).tolist() == list(range(-128, 128))


def test_int4_nibble_order_and_sign_hand_built():
    # byte 0x9F: low nibble 0xF = -1 (element 0), high nibble 0x9 = -7 (element 1);
    # byte 0x70: low 0x0 = 0 (element 2), high 0x7 = +7 (element 3)
    packed = np.array([[0x9F, 0x70]], dtype=np.uint8)
    assert codecs.int4_unpack(packed).tolist() == [[-1, -7, 0, 7]]


def test_int4_unpack_exhaustive_against_shift_sign_extension():
    # every byte, decoded by a different route: move each nibble to the top of
    # a signed byte and shift it back arithmetically
    b = np.arange(256, dtype=np.uint8)
    lo_ref = ((b << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int64)
    hi_ref = (b.view(np.int8) >> 4).astype(np.int64)
    out = codecs.int4_unpack(b.reshape(256, 1))
    assert np.array_equal(out[:, 0], lo_ref) and np.array_equal(out[:, 1], hi_ref)


def test_int4_pack_unpack_round_trip():
    codes = torch.randint(-8, 8, (5, 7, 64), dtype=torch.int8)
    back = codecs.int4_unpack(inputs.pack_int4(codes).numpy())
    assert np.array_equal(back, codes.numpy().astype(np.int64))


@pytest.mark.parametrize("kind,qmax", [("int8", 127), ("int4", 7)])
def test_int_quantizer_round_trip_bound(kind, qmax):
    x = torch.randn(6, 33, 64, dtype=torch.float32)
    x[0, 0] = 0.0  # an all-zero row keeps scale 1 and codes 0
    codes, scales = inputs.quantize_rows(x, kind)
    deq = codecs.dequantize_int_cache(codes.numpy(), scales.numpy(), 8 if kind == "int8" else 4)
    xs = x.double().numpy()
    sc = scales.double().numpy()[..., None]
    ints = np.rint(deq / sc)
    assert np.abs(ints).max() <= qmax
    # the row maximum maps to +-qmax; every value is within half a step
    nz = np.abs(xs).max(-1) > 0
    top = np.take_along_axis(ints, np.abs(xs).argmax(-1)[..., None], -1)[..., 0]
    assert np.all(np.abs(top[nz]) == qmax)
    assert np.all(np.abs(deq - xs) <= 0.5 * sc * (1 + 1e-6))
    assert scales[0, 0].item() == 1.0 and np.all(deq[0, 0] == 0.0)


def test_int_dequantize_is_code_times_scale():
    codes = np.array([[[-127, 0, 5, 127]]], dtype=np.int8)
    scales = np.array([[0.25]], dtype=np.float32)
    assert codecs.dequantize_int_cache(codes, scales, 8).tolist() == [[[-31.75, 0.0, 1.25, 31.75]]]
    packed = np.array([[[0x9F, 0x70]]], dtype=np.uint8)
    assert codecs.dequantize_int_cache(packed, scales, 4).tolist() == [[[-0.25, -1.75, 0.0, 1.75]]]
    with pytest.raises(TypeError):
        codecs.dequantize_int_cache(codes.astype(np.uint8), scales, 8)
    with pytest.raises(ValueError):
        codecs.dequantize_int_cache(codes, scales, 2)
