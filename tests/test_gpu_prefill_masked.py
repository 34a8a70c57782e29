"""GPU parity of attn_prefill (general masks) against the fp64 oracle
oracle.prefill: causal or not, more keys than queries and the reverse, key
lengths with NaN padding, dense random and packed-document masks, and
sampled rows of the full-size workloads."""

import numpy as np
import pytest
import torch

import oracle
from oracle import masked as omasked
from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = pu.TOL["bf16"]


def wl(B, S_q, S_k, h_q, n_kv, d, causal, seed, mask=None, doc_lens=(512, 2048)):
    return inputs.MaskedPrefillWorkload("masked", B=B, S_q=S_q, S_k=S_k, h_q=h_q, n_kv=n_kv, d_h=d, causal=causal,
                                        seed=seed, mask=mask, doc_lens=doc_lens)


def run(inp):
    w = inp.wl
    return binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, causal=w.causal, kv_lens=inp.kv_lens, mask=inp.mask)


def oracle_full(inp):
    w = inp.wl
    return oracle.prefill(pu.to_f64(inp.q), pu.to_f64(inp.k), pu.to_f64(inp.v), w.scale, causal=w.causal,
                          kv_lens=None if inp.kv_lens is None else inp.kv_lens.cpu().numpy(),
                          mask=None if inp.mask is None else inp.mask.cpu().numpy())


def check(inp):
    w = inp.wl
    print(f"[prefill_masked] {w} kv_lens={None if inp.kv_lens is None else inp.kv_lens.tolist()} "
          f"mask={'none' if inp.mask is None else 'dense'}", flush=True)
    out = run(inp)
    pu.sync()
    err = pu.max_err(out, oracle_full(inp))
    assert err <= TOL, f"max abs err {err}"
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("h_q,n_kv", [(8, 8), (8, 4), (8, 2), (16, 2), (6, 2), (12, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_key_lengths_every_head_chunk(d, h_q, n_kv, causal):
    """Head chunks of 1, 2, 4 and 8 query heads (group sizes 1, 2, 4, 8, 3, 6);
    key lengths 200 (all), 1, 0 and 77, with NaN past each length."""
    inp = inputs.make_masked_prefill_inputs(wl(4, 200, 200, h_q, n_kv, d, causal, seed=400 + h_q + n_kv + d),
                                            device=DEV, kv_lens=[200, 1, 0, 77], poison_padding=True)
    out = check(inp)
    assert torch.count_nonzero(out[2]) == 0


@pytest.mark.parametrize("S_q,S_k", [(100, 333), (150, 40), (1, 257), (64, 64)])
def test_query_and_key_counts_differ(S_q, S_k):
    """End-aligned causal rule: cached keys ahead of the queries, and more
    queries than keys (the first S_q - S_k rows see nothing)."""
    inp = inputs.make_masked_prefill_inputs(wl(2, S_q, S_k, 8, 2, 128, True, seed=420 + S_q), device=DEV)
    out = check(inp)
    if S_q > S_k:
        assert torch.count_nonzero(out[:, :S_q - S_k]) == 0


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kind", ["random", "docs"])
def test_dense_masks(causal, kind):
    """A random mask and packed documents of 16..80 tokens (most 32 x 64 wave
    tiles fully hidden: the skip path), with key lengths, and three rows
    hidden completely."""
    w = wl(3, 260, 260, 8, 2, 128, causal, seed=430, mask=kind, doc_lens=(16, 80))
    m = inputs.draw_mask(kind, 3, 260, 260, 430, (16, 80))
    m[0, 5] = 0
    m[1, 200] = 0
    m[2, 259] = 0
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[260, 131, 64], mask=m, poison_padding=True)
    out = check(inp)
    assert torch.count_nonzero(out[0, 5]) == 0 and torch.count_nonzero(out[1, 200]) == 0


def test_mask_with_more_keys_than_queries_d64():
    w = wl(2, 96, 300, 4, 4, 64, True, seed=440, mask="random")
    check(inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[300, 250]))


def test_causal_without_masks_equals_causal_kernel():
    """With S_q = S_k, the causal rule and nothing else, the general kernel
    reproduces attn_prefill_causal bit for bit."""
    w = wl(2, 333, 333, 16, 4, 128, True, seed=450)
    inp = inputs.make_masked_prefill_inputs(w, device=DEV)
    a = run(inp)
    b = binding.attn_prefill_causal(inp.q, inp.k, inp.v, w.scale)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", sorted(inputs.MASKED_PREFILL_WORKLOADS))
def test_full_size_sampled(name):
    """The benchmarked workloads in their launch configuration, on sampled
    rows (first and last rows, rows at document and padding edges, random)."""
    w = inputs.MASKED_PREFILL_WORKLOADS[name]
    inp = inputs.make_masked_prefill_inputs(w, device=DEV)
    print(f"[prefill_masked] full size {w}", flush=True)
    out = run(inp)
    pu.sync()
    trip = pu.sample_rows(w.B, w.S_q, w.h_q, 48, seed=460)
    q, k, v = pu.to_f64(inp.q), pu.to_f64(inp.k), pu.to_f64(inp.v)
    lens = None if inp.kv_lens is None else inp.kv_lens.cpu().numpy()
    mask = None if inp.mask is None else inp.mask.cpu().numpy()
    ref = omasked.prefill_rows(q, k, v, w.scale, trip, causal=w.causal, kv_lens=lens, mask=mask)
    got = torch.stack([out[b, r, j] for b, r, j in trip])
    err = pu.max_err(got, ref)
    assert err <= TOL, f"max abs err {err}"
