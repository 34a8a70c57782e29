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


def wl(B, S_q, S_k, h_q, n_kv, d, causal, seed, mask=None, doc_lens=(512, 2048), dtype="bf16"):
    return inputs.MaskedPrefillWorkload("masked", B=B, S_q=S_q, S_k=S_k, h_q=h_q, n_kv=n_kv, d_h=d, causal=causal,
                                        seed=seed, mask=mask, doc_lens=doc_lens, dtype=dtype)


def run(inp):
    w = inp.wl
    return binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, causal=w.causal, kv_lens=inp.kv_lens, mask=inp.mask,
                                q_descale=inp.q_descale, k_descale=inp.k_descale, v_descale=inp.v_descale)


def _lens_mask(inp):
    return (None if inp.kv_lens is None else inp.kv_lens.cpu().numpy(),
            None if inp.mask is None else inp.mask.cpu().numpy())


def compare(inp, out, triples=None):
    """bf16: max-abs error <= 2e-2 against the oracle.  fp8: every element
    within the arithmetic's bound (parity_utils.fp8_prefill_bound) and the
    relative RMS error below 0.1 (a wrong key or head mapping gives ~1)."""
    w = inp.wl
    q, k, v = pu.masked_prefill_values(inp)
    lens, mask = _lens_mask(inp)
    if triples is None:
        ref = oracle.prefill(q, k, v, w.scale, causal=w.causal, kv_lens=lens, mask=mask)
        got = out
    else:
        ref = omasked.prefill_rows(q, k, v, w.scale, triples, causal=w.causal, kv_lens=lens, mask=mask)
        got = torch.stack([out[b, r, j] for b, r, j in triples])
    if w.dtype != "fp8":
        err = pu.max_err(got, ref)
        assert err <= TOL, f"max abs err {err}"
        return
    g = got.detach().float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    if triples is None:
        triples = [(b, r, j) for b in range(w.B) for r in range(w.S_q) for j in range(w.h_q)]
        g = g.reshape(-1, w.d_h)
        ref = ref.reshape(-1, w.d_h)
    bound = pu.fp8_prefill_bound(q, k, v, w.scale, triples, w.causal, lens, mask)
    excess = np.abs(g - ref) - bound
    assert np.all(excess <= 0), f"fp8 bound exceeded by {excess.max()} at row {triples[int(np.argmax(excess.max(1)))]}"
    rel = np.sqrt(np.mean((g - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    assert rel <= 0.1, f"relative rms error {rel}"


def check(inp):
    w = inp.wl
    print(f"[prefill_masked] {w} kv_lens={None if inp.kv_lens is None else inp.kv_lens.tolist()} "
          f"mask={'none' if inp.mask is None else 'dense'}", flush=True)
    out = run(inp)
    pu.sync()
    compare(inp, out)
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


def test_all_ones_mask_equals_causal_kernel():
    """Every tile of an all-ones mask is fully visible, so the general kernel
    skips the mask tiles and must reproduce attn_prefill_causal bit for bit."""
    w = wl(2, 332, 332, 16, 4, 128, True, seed=452)  # a dense mask needs S_k % 4 == 0
    inp = inputs.make_masked_prefill_inputs(w, device=DEV,
                                            mask=torch.ones((2, 332, 332), dtype=torch.uint8))
    a = run(inp)
    b = binding.attn_prefill_causal(inp.q, inp.k, inp.v, w.scale)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("causal", [True, False])
def test_documents_with_full_tiles(causal):
    """Documents of 96..300 tokens: row blocks see tiles that are hidden,
    fully visible (no per-element mask) and partly visible, and the rows of a
    block that starts a new document see nothing for several tiles."""
    w = wl(2, 700, 700, 8, 2, 128, causal, seed=455, mask="docs", doc_lens=(96, 300))
    check(inputs.make_masked_prefill_inputs(w, device=DEV))


@pytest.mark.parametrize("name", sorted(inputs.MASKED_PREFILL_WORKLOADS))
def test_full_size_sampled(name):
    """The benchmarked workloads in their launch configuration, on sampled
    rows (first and last rows, rows at document and padding edges, random)."""
    w = inputs.MASKED_PREFILL_WORKLOADS[name]
    inp = inputs.make_masked_prefill_inputs(w, device=DEV)
    print(f"[prefill_masked] full size {w}", flush=True)
    out = run(inp)
    pu.sync()
    compare(inp, out, pu.sample_rows(w.B, w.S_q, w.h_q, 48, seed=460))


@pytest.mark.parametrize("h_q,n_kv", [(8, 8), (8, 4), (8, 2), (16, 2), (6, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_head_chunks_and_lengths(h_q, n_kv, causal):
    """fp8 operands over every head-chunk size, key lengths 200, 1, 0 and 77
    (NaN codes past each length)."""
    inp = inputs.make_masked_prefill_inputs(wl(4, 200, 200, h_q, n_kv, 128, causal, seed=470 + h_q + n_kv,
                                               dtype="fp8"), device=DEV, kv_lens=[200, 1, 0, 77],
                                            poison_padding=True)
    out = check(inp)
    assert torch.count_nonzero(out[2]) == 0


@pytest.mark.parametrize("kind", ["random", "docs"])
def test_fp8_masks_and_key_counts(kind):
    w = wl(2, 150, 300, 8, 2, 128, True, seed=480, mask=kind, doc_lens=(16, 80), dtype="fp8")
    m = inputs.draw_mask(kind, 2, 150, 300, 480, (16, 80)) if kind == "random" else None
    if kind == "docs":  # documents over the keys; the queries are the last 150 positions
        full = inputs.draw_mask("docs", 2, 300, 300, 480, (16, 80))
        m = full[:, 150:, :].contiguous()
    check(inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[300, 222], mask=m))
