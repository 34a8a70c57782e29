"""Seeded random sweeps over the decode, paged decode, MLA decode and general
prefill entry points, each case compared with the oracle by the same checks
as the directed tests (shapes, cache formats, lengths including 0 and past
the cache, forced key-range counts, key lengths, dense random and packed
document masks, bf16 and fp8 prefill).  The cases are drawn from fixed seeds,
so a failure names a reproducible case (it is printed before it runs)."""

import random

import pytest

from transformer_attention_gqa_amd import inputs

import test_gpu_decode as td
import test_gpu_mla as tm
import test_gpu_paged as tpg
import test_gpu_prefill_masked as tp

pytestmark = pytest.mark.gpu

CASES = 100


def test_random_decode():
    rng = random.Random(1101)
    for _ in range(CASES):
        kd = rng.choice(["f32", "bf16", "fp8", "int8", "int4"])
        n_kv = rng.choice([1, 2, 4])
        G = rng.choice([1, 2, 4, 8, 16, 32])
        d = rng.choice([64, 128])
        S = rng.randint(1, 600)
        B = rng.randint(1, 80)
        while B * G * n_kv * S > 1_000_000:
            B, S = max(1, B // 2), max(1, S // 2)
        lens = [rng.choice([0, S, S + 7, rng.randint(0, S), rng.randint(S // 2, S)]) for _ in range(B)]
        w = td.wl("sweep", B=B, h_q=G * n_kv, n_kv=n_kv, d=d, S=S, qd="f32" if kd == "f32" else "bf16", kd=kd,
                  seed=rng.randint(0, 10 ** 6))
        inp = inputs.make_decode_inputs(w, device=td.DEV, seq_lens=lens, poison_tail=True)
        td.check_full(inp, n_split=rng.choice([0, 0, rng.randint(1, 300), 10 ** 6]))


def test_random_paged_decode():
    rng = random.Random(1102)
    for _ in range(CASES):
        kd = rng.choice(["f32", "bf16", "fp8", "int8", "int4"])
        n_kv = rng.choice([1, 2])
        G = rng.choice([1, 4, 8, 16, 32])
        page = rng.choice([32, 64, 128])
        S = page * rng.randint(1, 6)
        B = rng.randint(1, 6)
        lens = [rng.choice([0, S, rng.randint(0, S)]) for _ in range(B)]
        w = tpg.wl(B=B, h_q=G * n_kv, n_kv=n_kv, d=rng.choice([64, 128]), S=S, kd=kd, seed=rng.randint(0, 10 ** 6))
        pin = inputs.make_paged_decode_inputs(w, page, device=tpg.DEV, seq_lens=lens, poison_tail=True)
        tpg.check(pin, n_split=rng.choice([0, rng.randint(1, 50), 10 ** 6]))


def test_random_mla_decode():
    rng = random.Random(1103)
    for _ in range(CASES):
        d_c = rng.choice([256, 512])
        h_q = rng.choice([16, 32, 48, 64, 96, 128])
        S = rng.randint(1, 300)
        B = rng.randint(1, 70)
        while B * h_q * S * d_c > 200_000_000:
            B = max(1, B // 2)
        lens = [rng.choice([0, S, rng.randint(0, S)]) for _ in range(B)]
        w = tm.wl(B=B, h_q=h_q, d_c=d_c, S=S, seed=rng.randint(0, 10 ** 6))
        inp = inputs.make_mla_inputs(w, device=tm.DEV, seq_lens=lens, poison_tail=True)
        tm.check(inp, n_split=rng.choice([0, rng.randint(1, 100), 10 ** 6]))


def test_random_prefill():
    rng = random.Random(1104)
    for _ in range(CASES):
        dtype = rng.choice(["bf16", "bf16", "fp8"])
        h_q, n_kv = rng.choice([(8, 2), (16, 4), (6, 2), (8, 8), (4, 1), (16, 2)])
        d = 128 if dtype == "fp8" else rng.choice([64, 128])
        kind = rng.choice([None, "random", "docs", "docs"])
        S_q = rng.randint(1, 200)
        S_k = S_q if kind == "docs" else rng.randint(1, 200)
        if kind is not None:  # a dense mask needs S_k % 4 == 0; documents need S_q == S_k
            S_k = max(4, (S_k + 3) // 4 * 4)
            if kind == "docs":
                S_q = S_k
        B = rng.randint(1, 3)
        kv_lens = [rng.randint(0, S_k) for _ in range(B)] if rng.random() < 0.4 else None
        docs = (rng.randint(8, 40), rng.randint(41, 200))
        w = tp.wl(B, S_q, S_k, h_q, n_kv, d, rng.random() < 0.6, seed=rng.randint(0, 10 ** 6), mask=kind,
                  doc_lens=docs, dtype=dtype)
        mask = inputs.draw_mask(kind, B, S_q, S_k, w.seed, docs) if kind else None
        tp.check(inputs.make_masked_prefill_inputs(w, device=tp.DEV, kv_lens=kv_lens, mask=mask,
                                                   poison_padding=kv_lens is not None))
