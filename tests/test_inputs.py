"""Seeded input generator: determinism, shapes, ranges, poisoning."""

import numpy as np
import pytest
import torch

from transformer_attention_gqa_amd import inputs


def test_lengths_are_seeded_and_in_range():
    w = inputs.GQA_RAGGED_BF16
    a = inputs.draw_lengths(w.B, *w.lens, w.seed)
    b = inputs.draw_lengths(w.B, *w.lens, w.seed)
    assert torch.equal(a, b) and a.dtype == torch.int32
    assert int(a.min()) >= 1024 and int(a.max()) <= 4096
    assert len(set(a.tolist())) > 1


def test_decode_inputs_shapes_and_determinism():
    w = inputs.DecodeWorkload("t", B=3, h_q=4, n_kv=2, d_h=64, S_max=40, q_dtype="bf16", kv_dtype="bf16",
                              lens=(5, 40), seed=11)
    a = inputs.make_decode_inputs(w)
    b = inputs.make_decode_inputs(w)
    assert a.q.shape == (3, 4, 64) and a.k.shape == (3, 2, 40, 64) and a.q.dtype == torch.bfloat16
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.q, b.q)
    c = inputs.make_decode_inputs(w, seed=12)
    assert not torch.equal(a.k, c.k)


def test_fp8_inputs_have_finite_codes_and_positive_scales():
    w = inputs.DecodeWorkload("t8", B=2, h_q=8, n_kv=2, d_h=128, S_max=33, q_dtype="bf16", kv_dtype="fp8",
                              lens=(33, 33), seed=3)
    x = inputs.make_decode_inputs(w)
    for codes in (x.k, x.v):
        c = codes.numpy()
        assert c.dtype == np.uint8
        assert not np.any((c & 0x7F) == 0x7F)  # no NaN codes
    assert torch.all(x.k_scale > 0) and torch.all(x.v_scale > 0)


def test_poisoned_tails():
    w = inputs.DecodeWorkload("tp", B=2, h_q=2, n_kv=1, d_h=64, S_max=16, q_dtype="bf16", kv_dtype="bf16",
                              lens=(3, 16), seed=5)
    x = inputs.make_decode_inputs(w, seq_lens=[3, 16], poison_tail=True)
    assert torch.isnan(x.k[0, :, 3:].float()).all() and not torch.isnan(x.k[0, :, :3].float()).any()
    assert not torch.isnan(x.v[1].float()).any()


@pytest.mark.parametrize("kind", ["int8", "int4"])
def test_int_cache_generator_shapes_and_poison(kind):
    wl = inputs.DecodeWorkload("q", B=2, h_q=8, n_kv=2, d_h=64, S_max=48, q_dtype="bf16", kv_dtype=kind,
                               lens=(1, 48), seed=9)
    inp = inputs.make_decode_inputs(wl, seq_lens=[48, 10], poison_tail=True)
    dc = 64 if kind == "int8" else 32
    want = torch.int8 if kind == "int8" else torch.uint8
    assert inp.k.shape == (2, 2, 48, dc) and inp.k.dtype == want and inp.v.dtype == want
    assert inp.k_scale.shape == (2, 2, 48) and inp.k_scale.dtype == torch.float32
    assert torch.isnan(inp.k_scale[1, :, 10:]).all() and torch.isfinite(inp.k_scale[1, :, :10]).all()
    assert torch.isfinite(inp.k_scale[0]).all()
    pc = inputs.POISON_CODE[kind]
    assert (inp.k[1, :, 10:].view(torch.uint8) == pc).all()
    pin = inputs.make_paged_decode_inputs(wl, 16, seq_lens=[48, 10])
    assert pin.k_pages.shape[-1] == dc and pin.k_pages.dtype == want
    spare = sorted(set(range(pin.num_pages)) - {int(x) for x in pin.block_table.flatten()})
    assert torch.isnan(pin.k_scale_pages[spare]).all()


def test_mla_inputs():
    wl = inputs.MlaWorkload("m", B=2, h_q=32, d_c=64, S_max=40, lens=(1, 40), seed=3)
    x = inputs.make_mla_inputs(wl, seq_lens=[40, 7], poison_tail=True)
    assert x.q.shape == (2, 32, 64) and x.c_kv.shape == (2, 40, 64) and x.c_kv.dtype == torch.bfloat16
    assert torch.isnan(x.c_kv[1, 7:]).all() and torch.isfinite(x.c_kv[1, :7]).all()
    y = inputs.make_mla_inputs(wl, seq_lens=[40, 7], poison_tail=True)
    assert torch.equal(x.q, y.q)
