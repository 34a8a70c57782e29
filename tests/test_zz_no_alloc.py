"""attn_decode_noalloc (partials in the library's static device scratch, no
allocation) against attn_decode, the entry point it is a variant of, on two
calls in a row -- the second with a smaller input -- and against the oracle."""

import pytest
import torch

from transformer_attention_gqa_amd import binding, inputs
import parity_utils as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(name, B, h_q, n_kv, S, kd, lens, seed):
    w = inputs.DecodeWorkload(name, B=B, h_q=h_q, n_kv=n_kv, d_h=128, S_max=S, q_dtype="bf16", kv_dtype=kd,
                              lens=(1, S), seed=seed)
    return inputs.make_decode_inputs(w, device=DEV, seq_lens=lens, poison_tail=True)


@pytest.mark.parametrize("kd", ["bf16", "fp8"])
def test_noalloc_equals_attn_decode_on_two_calls(kd):
    cases = [_case("noalloc-big", 16, 64, 8, 4096, kd, [4096, 1, 3000, 2048, 17, 4095, 1024, 999] * 2, 81),
             _case("noalloc-small", 3, 16, 2, 300, kd, [300, 5, 0], 82)]
    for inp in cases:
        w = inp.wl
        print(f"[noalloc] {w.name} {kd} lens={inp.seq_lens.tolist()}", flush=True)
        desc = binding.decode_desc(inp.q, inp.k)
        assert binding.attn_decode_workspace_bytes(desc) <= binding.attn_decode_noalloc_max_scratch_bytes()
        ref = binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, k_scale=inp.k_scale,
                                  v_scale=inp.v_scale, deterministic=True)
        out = torch.full_like(inp.q, float("nan"))
        binding.attn_decode_noalloc(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, out, k_scale=inp.k_scale,
                                    v_scale=inp.v_scale, deterministic=True)
        pu.sync()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        # default (dynamic) tile order: within the bar of the oracle
        out2 = torch.full_like(inp.q, float("nan"))
        binding.attn_decode_noalloc(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, out2, k_scale=inp.k_scale,
                                    v_scale=inp.v_scale)
        pu.sync()
        oracle_out = pu.oracle_decode_full(inp)
        assert pu.max_err(out2, oracle_out) <= pu.TOL[kd]
        assert pu.max_err(ref, oracle_out) <= pu.TOL[kd]
        assert torch.count_nonzero(out[inp.seq_lens.cpu() == 0]) == 0


def test_noalloc_rejects_oversized_calls():
    w = inputs.DecodeWorkload("noalloc-huge", B=64, h_q=64, n_kv=64, d_h=128, S_max=64, q_dtype="bf16",
                              kv_dtype="bf16", lens=(1, 64), seed=83)
    inp = inputs.make_decode_inputs(w, device=DEV)
    desc = binding.decode_desc(inp.q, inp.k, n_split=4096)
    assert binding.attn_decode_workspace_bytes(desc) > binding.attn_decode_noalloc_max_scratch_bytes()
    out = torch.zeros_like(inp.q)
    with pytest.raises(binding.GqaError) as e:
        binding.attn_decode_noalloc(inp.q, inp.k, inp.v, inp.seq_lens, w.scale, out, n_split=4096)
    assert e.value.status == 8
    pu.sync()
    assert torch.count_nonzero(out) == 0
