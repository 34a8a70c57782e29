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
    """bf16: max-abs error <= 2e-2 against the oracle.  fp8: max-abs error
    <= 5e-2 (the fp8 bar) element by element against the oracle on the
    dequantised values, and relative RMS error <= 0.03 over all compared
    elements (a wrong key or head mapping gives ~1)."""
    w = inp.wl
    q, k, v = pu.masked_prefill_values(inp)
    lens, mask = _lens_mask(inp)
    if triples is None:
        ref = oracle.prefill(q, k, v, w.scale, causal=w.causal, kv_lens=lens, mask=mask)
        got = out
    else:
        ref = pu.masked_rows(q, k, v, w.scale, triples, w.causal, lens, mask)
        idx = torch.tensor(triples, device=out.device)
        got = out[idx[:, 0], idx[:, 1], idx[:, 2]]
    if w.dtype != "fp8":
        err = pu.max_err(got, ref)
        print(f"[prefill_masked] max abs err {err:.3e}", flush=True)
        assert err <= TOL, f"max abs err {err}"
        return
    err, rel = pu.check_fp8_prefill(got, ref)
    print(f"[prefill_masked] fp8 max abs err {err:.3e}, relative rms {rel:.3e}", flush=True)


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


def test_more_key_tiles_than_the_bitmaps_hold():
    """524,588 keys (8,197 tiles of 64, more than the 8,192 the key-tile
    bitmaps hold): both entry points then visit every tile with the
    per-element mask.  Each row sees eight scattered keys, one of them in the
    last 300 (past the bitmaps' range), so the outputs are averages of a few
    value rows and a dropped or misplaced tile shows."""
    S_q, S_k = 40, 8192 * 64 + 300
    w = wl(1, S_q, S_k, 2, 1, 64, True, seed=445)
    g = torch.Generator().manual_seed(445)
    m = torch.zeros((1, S_q, S_k), dtype=torch.uint8)
    cols = torch.randint(0, S_k - 300, (S_q, 7), generator=g)
    m[0, torch.arange(S_q)[:, None], cols] = 1
    m[0, torch.arange(S_q), S_k - 300 + torch.randint(0, 300 - S_q, (S_q,), generator=g)] = 1
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, mask=m)
    print(f"[prefill_masked] {w} (scattered visible keys)", flush=True)
    a = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, causal=True, mask=inp.mask)
    b = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, causal=True, mask=inp.mask, mask_prepass=False)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert float(a.float().abs().mean()) > 0.1  # averages of a few rows, not of many
    compare(inp, a)


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
def test_full_size_every_block(name):
    """The benchmarked workloads in their launch configuration: one random
    (head, row) in every workgroup block, plus the first and last rows of
    every head, against the oracle row by row."""
    w = inputs.MASKED_PREFILL_WORKLOADS[name]
    inp = inputs.make_masked_prefill_inputs(w, device=DEV)
    print(f"[prefill_masked] full size {w}", flush=True)
    out = run(inp)
    pu.sync()
    trip = pu.prefill_block_samples(w.B, w.S_q, w.h_q, w.n_kv, seed=460)
    trip += [(b, r, j) for b in range(w.B) for j in range(w.h_q) for r in (0, w.S_q - 1)]
    compare(inp, out, trip)


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_fp8_zero_descale(which):
    """An all-zero head quantised by absmax has descale 0.  A zero Q or K
    descale makes every visible score 0 (equal weights: the mean of the
    visible V rows); a zero V descale makes the output 0.  Hidden keys must
    stay hidden (no NaN from 0 * -inf)."""
    w = wl(2, 150, 150, 8, 2, 128, True, seed=490, dtype="fp8")
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[150, 97], poison_padding=True)
    if which == "q":
        inp.q[1, :, 5] = 0
        inp.q_descale[1, 5] = 0.0
    elif which == "k":
        inp.k[0, :, 1] = 0
        inp.k_descale[0, 1] = 0.0
    else:
        inp.v[1, :, 0] = 0
        inp.v_descale[1, 0] = 0.0
    out = check(inp)
    if which == "v":
        assert torch.count_nonzero(out[1, :, 0:4]) == 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("h_q,n_kv", [(8, 8), (8, 4), (8, 2), (16, 2), (6, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_head_chunks_and_lengths(h_q, n_kv, causal, d):
    """fp8 operands over every head-chunk size and both head dims, key
    lengths 200, 1, 0 and 77 (NaN codes past each length)."""
    inp = inputs.make_masked_prefill_inputs(wl(4, 200, 200, h_q, n_kv, d, causal, seed=470 + h_q + n_kv + d,
                                               dtype="fp8"), device=DEV, kv_lens=[200, 1, 0, 77],
                                            poison_padding=True)
    out = check(inp)
    assert torch.count_nonzero(out[2]) == 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["random", "docs"])
def test_fp8_masks_and_key_counts(kind, d):
    w = wl(2, 150, 300, 8, 2, d, True, seed=480 + d, mask=kind, doc_lens=(16, 80), dtype="fp8")
    m = inputs.draw_mask(kind, 2, 150, 300, 480, (16, 80)) if kind == "random" else None
    if kind == "docs":  # documents over the keys; the queries are the last 150 positions
        full = inputs.draw_mask("docs", 2, 300, 300, 480, (16, 80))
        m = full[:, 150:, :].contiguous()
    check(inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[300, 222], mask=m))


def test_fp8_head_dim_64_long_causal():
    """fp8 at d = 64 over several row blocks and key tiles per workgroup (a
    1,000-token causal prompt, GQA with 4 query heads per K/V head), every
    output element against the oracle."""
    w = wl(1, 1000, 1000, 8, 2, 64, True, seed=495, dtype="fp8")
    check(inputs.make_masked_prefill_inputs(w, device=DEV))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_scale_gives_the_mean_of_visible_values(dtype):
    """scale = 0: each row weighs its visible keys equally (key lengths, the
    end-aligned causal rule and a dense mask combined), so it returns the
    mean of their V rows; rows that see no key are zero."""
    w = wl(2, 150, 232, 8, 2, 128, True, seed=77, mask="random", dtype=dtype)
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[232, 101])
    out = binding.attn_prefill(inp.q, inp.k, inp.v, 0.0, causal=True, kv_lens=inp.kv_lens, mask=inp.mask,
                               q_descale=inp.q_descale, k_descale=inp.k_descale, v_descale=inp.v_descale)
    pu.sync()
    q, k, v = pu.masked_prefill_values(inp)
    lens, mask = _lens_mask(inp)
    ref = oracle.prefill(q, k, v, 0.0, causal=True, kv_lens=lens, mask=mask)
    if dtype == "fp8":
        pu.check_fp8_prefill(out, ref)
    else:
        assert pu.max_err(out, ref) <= TOL


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("h_q,n_kv", [(8, 8), (8, 4), (8, 2), (16, 2)])
@pytest.mark.parametrize("kind", ["random", "docs"])
def test_mask_prepass_equals_in_kernel_scan(dtype, h_q, n_kv, kind):
    """The pass that forms every row block's key-tile bitmaps once
    (attn_prefill_ws) and the workgroups' own scans (attn_prefill) classify
    the same tiles, so the outputs agree bit for bit; row blocks of 256, 128,
    64 and 32 rows, key lengths, more keys than queries, and a workspace that
    starts full of stale words (every word the kernel reads is rewritten)."""
    w = wl(3, 300, 520, h_q, n_kv, 128, True, seed=500 + h_q + n_kv, mask=kind, doc_lens=(16, 120), dtype=dtype)
    if kind == "docs":  # documents over the keys; the queries are the last 300 positions
        m = inputs.draw_mask("docs", 3, 520, 520, w.seed, (16, 120))[:, 220:, :].contiguous()
    else:
        m = inputs.draw_mask("random", 3, 300, 520, w.seed)
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=[520, 333, 0], mask=m)
    args = dict(causal=True, kv_lens=inp.kv_lens, mask=inp.mask, q_descale=inp.q_descale,
                k_descale=inp.k_descale, v_descale=inp.v_descale)
    desc = binding._attn_desc(inp.q, inp.k, inp.v, torch.empty(inp.q.shape, dtype=torch.bfloat16, device=DEV),
                              True, inp.kv_lens, inp.mask)
    nbytes = binding.attn_prefill_workspace_bytes(desc)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    a = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, workspace=ws, **args)
    b = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, mask_prepass=False, **args)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    compare(inp, a)


@pytest.mark.parametrize("name", sorted(n for n, w in inputs.MASKED_PREFILL_WORKLOADS.items() if w.mask))
def test_full_size_mask_prepass_equals_in_kernel_scan(name):
    """The benchmarked workloads with a dense mask: both ways of classifying
    key tiles give the same bits over the whole output."""
    w = inputs.MASKED_PREFILL_WORKLOADS[name]
    inp = inputs.make_masked_prefill_inputs(w, device=DEV)
    args = dict(causal=w.causal, kv_lens=inp.kv_lens, mask=inp.mask, q_descale=inp.q_descale,
                k_descale=inp.k_descale, v_descale=inp.v_descale)
    a = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, **args)
    b = binding.attn_prefill(inp.q, inp.k, inp.v, w.scale, mask_prepass=False, **args)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp8", 128), ("fp8", 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_workgroups_take_several_row_blocks(dtype, d, causal):
    """Without a dense mask a workgroup takes several row blocks (512 here,
    more than the compute units) and starts the next one's loads early; key
    lengths include zeros, so blocks with no visible key sit between blocks
    that have keys in a workgroup's list, and more keys than queries."""
    B = 128
    lens = np.random.default_rng(11).integers(0, 151, B)
    lens[::7] = 0
    w = wl(B, 70, 150, 8, 2, d, causal, seed=600 + d, dtype=dtype)
    inp = inputs.make_masked_prefill_inputs(w, device=DEV, kv_lens=lens.tolist(), poison_padding=True)
    out = check(inp)
    assert torch.count_nonzero(out[0]) == 0
