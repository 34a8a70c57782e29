"""The entry points inside a captured HIP graph (the way a serving loop calls
them with no host work per step): the graph is captured once over static
buffers, then replayed several times with new contents copied into those
buffers before each replay, eager library calls sharing the workspace and
device synchronisations between replays.  Every replay must give the bits
of an eager call on the same contents (decode in its deterministic mode;
prefill is deterministic), and the eager results are held to the oracle.
The library records no memory fill into a graph: every kernel writes all
the words it reads later in the same call."""

import pytest
import torch

import oracle
from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 4


def capture(fn):
    """A graph of fn() captured on a side stream (after one warm-up call)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def decode_wl(kd, B=6, h_q=16, n_kv=2, S=700, seed=610):
    return inputs.DecodeWorkload("graph", B=B, h_q=h_q, n_kv=n_kv, d_h=128, S_max=S, q_dtype="bf16", kv_dtype=kd,
                                 lens=(1, S), seed=seed)


@pytest.mark.parametrize("kd", ["bf16", "fp8", "int4"])
@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays(kd, noalloc):
    w = decode_wl(kd)
    static = inputs.make_decode_inputs(w, device=DEV)
    out = torch.empty_like(static.q)
    ws = torch.empty(binding.attn_decode_workspace_bytes(binding.decode_desc(static.q, static.k, 0, True)),
                     dtype=torch.uint8, device=DEV)

    def call():
        if noalloc:
            binding.attn_decode_noalloc(static.q, static.k, static.v, static.seq_lens, w.scale, out,
                                        k_scale=static.k_scale, v_scale=static.v_scale, deterministic=True)
        else:
            binding.attn_decode(static.q, static.k, static.v, static.seq_lens, w.scale, out=out,
                                k_scale=static.k_scale, v_scale=static.v_scale, workspace=ws, deterministic=True)

    g = capture(call)
    for r in range(REPLAYS):
        step = inputs.make_decode_inputs(w, device=DEV, seed=w.seed + 1 + r)
        print(f"[graph-decode] {kd} noalloc={noalloc} replay {r} lens={step.seq_lens.tolist()}", flush=True)
        for name in ("q", "k", "v", "k_scale", "v_scale", "seq_lens"):
            src = getattr(step, name)
            if src is not None:
                getattr(static, name).copy_(src)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # an eager call with other lengths through the same workspace / scratch
        other = inputs.make_decode_inputs(w, device=DEV, seed=w.seed + 50 + r)
        if noalloc:
            binding.attn_decode_noalloc(other.q, other.k, other.v, other.seq_lens, w.scale, torch.empty_like(other.q),
                                        k_scale=other.k_scale, v_scale=other.v_scale, deterministic=True)
        else:
            binding.attn_decode(other.q, other.k, other.v, other.seq_lens, w.scale, k_scale=other.k_scale,
                                v_scale=other.v_scale, workspace=ws, deterministic=True)
        ref = binding.attn_decode(step.q, step.k, step.v, step.seq_lens, w.scale, k_scale=step.k_scale,
                                  v_scale=step.v_scale, deterministic=True)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"replay {r} differs from the eager call"
        if r == 0:
            err = pu.max_err(got, pu.oracle_decode_full(step))
            assert err <= pu.TOL[kd], f"max abs err {err}"


def test_paged_decode_graph_replays():
    w = decode_wl("bf16", S=704, seed=640)
    static = inputs.make_paged_decode_inputs(w, 64, device=DEV)
    b = static.base
    desc = binding.paged_desc(b.q, static.k_pages, static.block_table, 0, True)
    ws = torch.empty(binding.attn_decode_paged_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(b.q)

    def call():
        binding.attn_decode_paged(b.q, static.k_pages, static.v_pages, static.block_table, b.seq_lens, w.scale,
                                  out=out, workspace=ws, deterministic=True)

    g = capture(call)
    for r in range(REPLAYS):
        # the same pool shape, pages in another seeded order
        step = inputs.make_paged_decode_inputs(w, 64, device=DEV, seed=w.seed + 1 + r)
        print(f"[graph-paged] replay {r}", flush=True)
        for name in ("k_pages", "v_pages", "block_table"):
            getattr(static, name).copy_(getattr(step, name))
        for name in ("q", "seq_lens"):
            getattr(b, name).copy_(getattr(step.base, name))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = binding.attn_decode_paged(step.base.q, step.k_pages, step.v_pages, step.block_table,
                                        step.base.seq_lens, w.scale, deterministic=True)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"replay {r} differs from the eager call"
        if r == 0:
            assert pu.max_err(got, pu.oracle_decode_full(step.base)) <= pu.TOL["bf16"]


def test_mla_decode_graph_replays():
    w = inputs.MlaWorkload("graph", B=5, h_q=32, d_c=512, S_max=500, lens=(1, 500), seed=645)
    static = inputs.make_mla_inputs(w, device=DEV)
    ws = torch.empty(binding.attn_decode_mla_workspace_bytes(binding.mla_desc(static.q, static.c_kv, 0)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(static.q)

    def call():
        binding.attn_decode_mla(static.q, static.c_kv, static.seq_lens, w.scale, out=out, workspace=ws)

    g = capture(call)
    for r in range(REPLAYS):
        step = inputs.make_mla_inputs(w, device=DEV, seed=w.seed + 1 + r)
        print(f"[graph-mla] replay {r} lens={step.seq_lens.tolist()}", flush=True)
        for name in ("q", "c_kv", "seq_lens"):
            getattr(static, name).copy_(getattr(step, name))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = binding.attn_decode_mla(step.q, step.c_kv, step.seq_lens, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"replay {r} differs from the eager call"
        if r == 0:
            want = oracle.mla_decode(pu.to_f64(step.q), pu.to_f64(step.c_kv), step.seq_lens.cpu().numpy(), w.scale)
            assert pu.max_err(got, want) <= pu.TOL["bf16"]


def test_causal_prefill_graph_replays():
    w = inputs.PrefillWorkload("graph", B=2, S=700, h_q=16, n_kv=4, d_h=128, seed=650)
    static = inputs.make_prefill_inputs(w, device=DEV)
    out = torch.empty_like(static.q)

    def call():
        binding.attn_prefill_causal(static.q, static.k, static.v, w.scale, out=out)

    g = capture(call)
    for r in range(REPLAYS):
        step = inputs.make_prefill_inputs(w, device=DEV, seed=w.seed + 1 + r)
        print(f"[graph-prefill] replay {r}", flush=True)
        for name in ("q", "k", "v"):
            getattr(static, name).copy_(getattr(step, name))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = binding.attn_prefill_causal(step.q, step.k, step.v, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"replay {r} differs from the eager call"
        if r == 0:
            q, k, v = pu.prefill_f64(step)
            assert pu.max_err(got, oracle.prefill_causal(q, k, v, w.scale)) <= pu.TOL["bf16"]


def test_masked_prefill_with_bitmap_pass_graph_replays():
    """attn_prefill_ws (the bitmap pass, then the attention kernel) in one
    graph; each replay gets another packed-document mask, so the pass must
    rewrite every bitmap word the kernel reads."""
    w = inputs.MaskedPrefillWorkload("graph", B=2, S_q=600, S_k=600, h_q=16, n_kv=4, d_h=128, causal=True,
                                     seed=660, mask="docs", doc_lens=(40, 300))
    static = inputs.make_masked_prefill_inputs(w, device=DEV)
    out = torch.empty(static.q.shape, dtype=torch.bfloat16, device=DEV)
    desc = binding._attn_desc(static.q, static.k, static.v, out, True, None, static.mask)
    ws = torch.empty(binding.attn_prefill_workspace_bytes(desc), dtype=torch.uint8, device=DEV)

    def call():
        binding.attn_prefill(static.q, static.k, static.v, w.scale, causal=True, mask=static.mask, out=out,
                             workspace=ws)

    g = capture(call)
    for r in range(REPLAYS):
        kind = "docs" if r % 2 == 0 else "random"
        step = inputs.make_masked_prefill_inputs(
            w, device=DEV, seed=w.seed + 1 + r,
            mask=inputs.draw_mask(kind, w.B, w.S_q, w.S_k, w.seed + 1 + r, w.doc_lens).to(DEV))
        print(f"[graph-masked] replay {r} mask={kind}", flush=True)
        for name in ("q", "k", "v", "mask"):
            getattr(static, name).copy_(getattr(step, name))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = binding.attn_prefill(step.q, step.k, step.v, w.scale, causal=True, mask=step.mask,
                                   mask_prepass=False)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"replay {r} differs from the eager call"
        if r < 2:
            q, k, v = pu.to_f64(step.q), pu.to_f64(step.k), pu.to_f64(step.v)
            want = oracle.prefill(q, k, v, w.scale, causal=True, mask=step.mask.cpu().numpy())
            assert pu.max_err(got, want) <= pu.TOL["bf16"]
