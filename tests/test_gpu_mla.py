"""GPU parity of attn_decode_mla (absorbed latent-attention decode) against
the fp64 oracle oracle.mla_decode, on small cases that span several tiles,
head chunks and ragged tails, and on sampled sequences of the full-size
workload."""

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = pu.TOL["bf16"]


def wl(B, h_q, d_c, S, lens=None, seed=300):
    return inputs.MlaWorkload("mla", B=B, h_q=h_q, d_c=d_c, S_max=S, lens=lens or (1, S), seed=seed)


def oracle_rows(inp, bs):
    """Oracle output of sequences bs, [len(bs), h_q, d_c]."""
    w = inp.wl
    q = pu.to_f64(inp.q[bs])
    c = pu.to_f64(inp.c_kv[bs])
    return oracle.mla_decode(q, c, inp.seq_lens.cpu().numpy()[bs], w.scale)


def check(inp, n_split=0, workspace=None):
    w = inp.wl
    print(f"[mla] {w} lens={inp.seq_lens.tolist()} n_split={n_split}", flush=True)
    out = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, w.scale, workspace=workspace, n_split=n_split)
    pu.sync()
    ref = oracle_rows(inp, list(range(w.B)))
    err = pu.max_err(out, ref)
    assert err <= TOL, f"max abs err {err}"
    return out


@pytest.mark.parametrize("d_c", [256, 512])
@pytest.mark.parametrize("h_q", [16, 32, 64, 96])
def test_mla_matches_oracle(d_c, h_q):
    """Heads below one 32-head block (16), one block, two blocks, and two
    64-head chunks of which the second is partial (96); lengths 0, 1, a
    ragged tail and several tiles; the cache past each length holds NaN."""
    inp = inputs.make_mla_inputs(wl(B=4, h_q=h_q, d_c=d_c, S=300, seed=301 + h_q + d_c), device=DEV,
                                 seq_lens=[300, 1, 33, 0], poison_tail=True)
    out = check(inp)
    assert torch.count_nonzero(out[3]) == 0


@pytest.mark.parametrize("h_q,d_c", [(32, 512), (64, 256), (64, 512)])
@pytest.mark.parametrize("n_split", [1, 2, 5, 7, 31, 10 ** 6])
def test_mla_split_counts(n_split, h_q, d_c):
    """Ranges that cross sequence boundaries at every position of the kernel's
    rotation of in-flight tiles (few splits of 51 tiles), and ranges of at
    most one tile (more splits than tiles)."""
    inp = inputs.make_mla_inputs(wl(B=3, h_q=h_q, d_c=d_c, S=1000, seed=310), device=DEV,
                                 seq_lens=[1000, 517, 64], poison_tail=True)
    check(inp, n_split=n_split)


def test_mla_many_sequences():
    """B > 64: the schedule scans the lengths 64 at a time."""
    w = wl(B=70, h_q=32, d_c=256, S=96, lens=(0, 96), seed=320)
    inp = inputs.make_mla_inputs(w, device=DEV, poison_tail=True)
    check(inp)
    check(inp, n_split=37)


def test_mla_long_sequence_128_heads():
    """One long sequence, 128 heads in two 64-head passes over the cache."""
    inp = inputs.make_mla_inputs(wl(B=1, h_q=128, d_c=512, S=8192, seed=330), device=DEV, seq_lens=[8191])
    check(inp)


def test_mla_all_empty_and_dirty_workspace():
    """Every length 0 gives zero rows; a workspace full of NaN from an
    earlier use does not leak into a later result."""
    w = wl(B=3, h_q=32, d_c=512, S=128, seed=340)
    inp = inputs.make_mla_inputs(w, device=DEV, seq_lens=[0, 0, 0])
    desc = binding.mla_desc(inp.q, inp.c_kv)
    ws = torch.full((binding.attn_decode_mla_workspace_bytes(desc) // 4,), float("nan"), device=DEV)
    out = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, w.scale, workspace=ws)
    pu.sync()
    assert torch.count_nonzero(out) == 0
    inp2 = inputs.make_mla_inputs(w, device=DEV, seq_lens=[128, 5, 77])
    check(inp2, workspace=ws)


def test_mla_repeat_is_bitwise():
    """Every wave of a workgroup works on the same tile in a fixed order, so
    two identical calls agree bit for bit."""
    inp = inputs.make_mla_inputs(wl(B=5, h_q=64, d_c=512, S=700, seed=350), device=DEV)
    a = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, inp.wl.scale)
    b = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, inp.wl.scale)
    pu.sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mla_full_size_sampled():
    """The benchmarked workload, in its launch configuration: every head of
    a sample of sequences (the shortest, the longest and random ones) against
    the oracle."""
    w = inputs.MLA_DECODE_BF16
    inp = inputs.make_mla_inputs(w, device=DEV)
    print(f"[mla] full size {w}", flush=True)
    out = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, w.scale)
    pu.sync()
    lens = inp.seq_lens.cpu().numpy()
    rng = np.random.default_rng(360)
    bs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, w.B - 1, *rng.integers(0, w.B, 3).tolist()})
    err = pu.max_err(out[bs], oracle_rows(inp, bs))
    assert err <= TOL, f"max abs err {err}"


def test_mla_zero_scale_gives_the_mean_of_visible_rows():
    """scale = 0: every head returns the mean of the sequence's visible latent
    rows (the oracle at scale 0); a sequence of length 0 gives zeros."""
    inp = inputs.make_mla_inputs(wl(B=3, h_q=32, d_c=512, S=300, seed=330), device=DEV, seq_lens=[300, 1, 0],
                                 poison_tail=True)
    out = binding.attn_decode_mla(inp.q, inp.c_kv, inp.seq_lens, 0.0)
    pu.sync()
    ref = oracle.mla_decode(pu.to_f64(inp.q), pu.to_f64(inp.c_kv), inp.seq_lens.cpu().numpy(), 0.0)
    assert pu.max_err(out, ref) <= TOL

