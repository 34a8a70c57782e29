"""Decoders from stored element encodings to exact float64 values.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every stored value decodes to float64 exactly, so the oracle always works on
the values the GPU also sees and parity never depends on how inputs were
rounded or quantised.

* bf16: the top 16 bits of an IEEE-754 binary32 value; widening is a 16-bit
  left shift of the pattern.  (Standard bfloat16 definition; the pages only say
  that FP16/BF16 are the compute types -- "Flash Attention 3 Features" table of
  "Evolution of AI Attention Mechanisms".)
* e4m3fn: the pages name an FP8 KV cache ("KV cache quantization" in the
  "Multi-Query Attention (MQA)" glossary; "Interaction with other techniques"
  in "Multi-query attention") without fixing the format.  The reading taken is
  the OCP 8-bit float E4M3 format: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals at exponent field 0, no infinities, and NaN only
  for exponent 1111 with mantissa 111.  Largest finite magnitude 448.
* int8 / int4: the glossary's "KV cache quantization" also names INT8 and INT4
  caches with quantization-aware scaling factors.  Reading taken: symmetric
  signed integer codes (int8 in [-127, 127], int4 in [-7, 7]) with the same
  granularity as the FP8 cache, one float32 scale per (token, kv-head) row,
  value = code * scale.  An int4 row of d elements is stored as d / 2 bytes,
  element 2i in the low nibble of byte i and element 2i + 1 in the high
  nibble, each nibble a two's-complement 4-bit integer.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16")
    widened = bits.astype(np.uint32) << np.uint32(16)
    return widened.view(np.float32).astype(np.float64)


def _e4m3fn_value(code):
    """Value of one OCP E4M3 code, written out from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        # subnormal: 2^(1 - bias) * (m / 8), bias = 7
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes):
    """uint8 e4m3fn codes -> float64 (exact; NaN codes give NaN)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3fn codes must be uint8")
    return _E4M3FN_TABLE[codes]


def dequantize_fp8_cache(codes, scales):
    """codes [..., S, d] uint8 and scales [..., S] float32 -> float64 values.

    One scale per (token, kv-head) row: value = decode(code) * scale, formed in
    float64 from the stored float32 scale, so the product is exact.
    """
    scales = np.asarray(scales)
    if scales.dtype != np.float32:
        raise TypeError("fp8 scales must be float32")
    vals = e4m3fn_to_f64(codes)
    if vals.shape[:-1] != scales.shape:
        raise ValueError("scale shape must equal code shape without the last axis")
    return vals * scales.astype(np.float64)[..., None]


def dequantize_fp8_heads(codes, descale):
    """Token-major fp8 tensor codes [B, S, H, d] uint8 and float32 descale
    factors [B, H] (one per batch entry and head, the granularity of the
    FlashAttention-3 FP8 path named in "Flash Attention 3 Features") ->
    float64 values decode(code) * descale[b, h], exact in float64."""
    descale = np.asarray(descale)
    if descale.dtype != np.float32:
        raise TypeError("fp8 descale factors must be float32")
    vals = e4m3fn_to_f64(codes)
    if vals.ndim != 4 or descale.shape != (vals.shape[0], vals.shape[2]):
        raise ValueError("descale must be [B, H] for codes [B, S, H, d]")
    return vals * descale.astype(np.float64)[:, None, :, None]


def int8_to_f64(codes):
    """int8 codes -> float64 (exact)."""
    codes = np.asarray(codes)
    if codes.dtype != np.int8:
        raise TypeError("int8 codes must be int8")
    return codes.astype(np.float64)


def int4_unpack(packed):
    """uint8 [..., d/2] packed nibbles -> int64 codes [..., d].

    Byte i holds element 2i in bits 0..3 and element 2i + 1 in bits 4..7; a
    nibble n stands for n - 16 when its top bit is set (two's complement)."""
    packed = np.asarray(packed)
    if packed.dtype != np.uint8:
        raise TypeError("int4 codes must be packed into uint8")
    lo = (packed & 0x0F).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_int_cache(codes, scales, bits):
    """int8 codes [..., S, d] (bits = 8) or packed int4 codes [..., S, d/2]
    (bits = 4), and float32 scales [..., S] -> float64 values code * scale
    (exact: small integers times a float32, formed in float64)."""
    scales = np.asarray(scales)
    if scales.dtype != np.float32:
        raise TypeError("int cache scales must be float32")
    if bits == 8:
        vals = int8_to_f64(codes)
    elif bits == 4:
        vals = int4_unpack(codes).astype(np.float64)
    else:
        raise ValueError("bits must be 8 or 4")
    if vals.shape[:-1] != scales.shape:
        raise ValueError("scale shape must equal code shape without the last axis")
    return vals * scales.astype(np.float64)[..., None]
