"""GPU parity of attn_decode_paged against the fp64 paged-decode oracle, and
equality with attn_decode on the same cache laid out contiguously."""

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"


def wl(B, h_q, n_kv, d, S, kd, lens=None, seed=200):
    qd = "f32" if kd == "f32" else "bf16"
    return inputs.DecodeWorkload("paged", B=B, h_q=h_q, n_kv=n_kv, d_h=d, S_max=S, q_dtype=qd, kv_dtype=kd,
                                 lens=lens or (1, S), seed=seed)


def pages_f64(pin):
    """Pool contents as float64 values [num_pages, n_kv, page_size, d] (the oracle's input)."""
    kind = pin.base.wl.kv_dtype
    if kind in inputs.QUANTIZED:
        return (pu.dequantize(kind, pin.k_pages, pin.k_scale_pages), pu.dequantize(kind, pin.v_pages, pin.v_scale_pages))
    return pu.to_f64(pin.k_pages), pu.to_f64(pin.v_pages)


def run_paged(pin, n_split=0, out=None, workspace=None):
    b = pin.base
    return binding.attn_decode_paged(b.q, pin.k_pages, pin.v_pages, pin.block_table, b.seq_lens, b.wl.scale,
                                     out=out, k_scale=pin.k_scale_pages, v_scale=pin.v_scale_pages,
                                     workspace=workspace, n_split=n_split)


def check(pin, n_split=0):
    w = pin.base.wl
    print(f"[paged] {w} page_size={pin.page_size} lens={pin.base.seq_lens.tolist()} n_split={n_split}", flush=True)
    out = run_paged(pin, n_split=n_split)
    pu.sync()
    kp, vp = pages_f64(pin)
    ref = oracle.decode_paged(pu.to_f64(pin.base.q), kp, vp, pin.block_table.cpu().numpy(),
                              pin.base.seq_lens.cpu().numpy(), w.scale, pin.page_size)
    err = pu.max_err(out, ref)
    assert err <= pu.TOL[w.kv_dtype], f"max abs err {err}"
    return out


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
@pytest.mark.parametrize("page_size", [32, 64, 128])
def test_paged_matches_oracle(kd, page_size):
    w = wl(B=4, h_q=16, n_kv=2, d=128, S=512, kd=kd, seed=201 + page_size)
    pin = inputs.make_paged_decode_inputs(w, page_size, device=DEV, seq_lens=[512, 1, 300, 0], poison_tail=True,
                                          junk_unused_entries=True)
    out = check(pin)
    assert torch.count_nonzero(out[3]) == 0


@pytest.mark.parametrize("G,d", [(1, 64), (8, 128), (32, 128), (64, 64)])
def test_paged_group_sizes(G, d):
    n_kv = 2 if G <= 32 else 1
    for kd in ("bf16", "fp8", "int8", "int4"):
        w = wl(B=3, h_q=G * n_kv, n_kv=n_kv, d=d, S=256, kd=kd, seed=G * 7 + d)
        pin = inputs.make_paged_decode_inputs(w, 32, device=DEV, seq_lens=[256, 77, 33], poison_tail=True)
        check(pin)


@pytest.mark.parametrize("kd", ["bf16", "fp8", "int8", "int4"])
def test_paged_shared_prefix_pages(kd):
    """Sequences 1 and 2 reuse sequence 0's first pages (a shared prompt
    prefix): several table rows name the same physical pages."""
    w = wl(B=4, h_q=32, n_kv=4, d=128, S=512, kd=kd, seed=233)
    pin = inputs.make_paged_decode_inputs(w, 32, device=DEV, seq_lens=[512, 400, 97, 250], poison_tail=True)
    pin.block_table[1, :5] = pin.block_table[0, :5]
    pin.block_table[2, :3] = pin.block_table[0, :3]
    check(pin)


@pytest.mark.parametrize("n_split", [1, 7, 10 ** 6])
def test_paged_forced_splits(n_split):
    w = wl(B=3, h_q=16, n_kv=2, d=128, S=384, kd="bf16", seed=211)
    pin = inputs.make_paged_decode_inputs(w, 64, device=DEV, seq_lens=[384, 200, 5], poison_tail=True)
    check(pin, n_split=n_split)


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8", "int8", "int4"])
def test_paged_equals_contiguous_bitwise(kd):
    """Same values, same plan: the paged call must reproduce attn_decode exactly.
    At this size every workgroup's key range holds fewer tiles than it has
    waves, so each wave reduces at most one tile and the summation order is
    fixed."""
    w = wl(B=5, h_q=32, n_kv=4, d=128, S=1024, kd=kd, lens=(100, 1024), seed=223)
    pin = inputs.make_paged_decode_inputs(w, 64, device=DEV)
    b = pin.base
    ref = binding.attn_decode(b.q, b.k, b.v, b.seq_lens, w.scale, k_scale=b.k_scale, v_scale=b.v_scale)
    out = run_paged(pin)
    pu.sync()
    assert torch.equal(out, ref)


# Two calls over the same keys but with different tile-to-wave assignments
# differ only in float32 summation order and in where each wave rounds its
# probabilities to bf16 (relative 2^-9 per weight, against that wave's own
# reference max).  At the full decode sizes that moves outputs by about 1e-3
# at most; a larger gap means the calls did not read the same keys.
SAME_KEYS_TOL = 4e-3


@pytest.mark.parametrize("page_size", [32, 64])
def test_paged_full_size_ragged_gqa(page_size):
    """The ragged GQA workload (B=16, h_q=64, n_kv=8, d=128) in pages: every
    output row against the oracle at the bf16 bar, and close to the contiguous
    call on the same values."""
    w = inputs.GQA_RAGGED_BF16
    pin = inputs.make_paged_decode_inputs(w, page_size, device=DEV)
    b = pin.base
    print(f"[paged-full] page_size={page_size} sumL={int(b.seq_lens.sum())}", flush=True)
    ref = binding.attn_decode(b.q, b.k, b.v, b.seq_lens, w.scale)
    out = run_paged(pin)
    pu.sync()
    assert (out.float() - ref.float()).abs().max().item() <= SAME_KEYS_TOL
    assert pu.max_err(out, pu.oracle_decode_full(b)) <= pu.TOL["bf16"]


def test_paged_prepared_call_and_workspace_reuse():
    w = wl(B=3, h_q=16, n_kv=2, d=128, S=256, kd="bf16", seed=227)
    pin = inputs.make_paged_decode_inputs(w, 32, device=DEV, seq_lens=[256, 3, 100])
    ref = run_paged(pin)
    desc = binding.paged_desc(pin.base.q, pin.k_pages, pin.block_table)
    ws = torch.full((binding.attn_decode_paged_workspace_bytes(desc),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(pin.base.q)
    call = binding.prepare_decode_paged(pin.base.q, pin.k_pages, pin.v_pages, pin.block_table, pin.base.seq_lens,
                                        w.scale, out, ws)
    for _ in range(2):
        out.fill_(float("nan"))
        call()
        pu.sync()
        assert torch.equal(out, ref)
