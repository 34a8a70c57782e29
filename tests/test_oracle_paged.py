"""Pins of the paged-decode oracle (oracle/paged.py) against the contiguous
decode it must reduce to, hand-built index cases and invariants."""

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_gqa_amd import inputs


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def _cut(cache, page_size, order):
    """[B, n_kv, S, d] -> pool in the given page order + block table."""
    B, n_kv, S, d = cache.shape
    mp = S // page_size
    pool = np.full((B * mp + 2, n_kv, page_size, d), np.nan)
    table = np.zeros((B, mp), dtype=np.int64)
    for b in range(B):
        for i in range(mp):
            p = order[b * mp + i]
            pool[p] = cache[b, :, i * page_size:(i + 1) * page_size]
            table[b, i] = p
    return pool, table


@pytest.mark.parametrize("page_size", [1, 2, 4, 8])
def test_pages_in_order_equal_contiguous_decode(page_size):
    B, h_q, n_kv, S, d = 3, 4, 2, 8, 5
    q, k, v = _rand(B, h_q, d, seed=1), _rand(B, n_kv, S, d, seed=2), _rand(B, n_kv, S, d, seed=3)
    lens = [8, 3, 0]
    kp, table = _cut(k, page_size, list(range(B * S // page_size)))
    vp, _ = _cut(v, page_size, list(range(B * S // page_size)))
    got = oracle.decode_paged(q, kp, vp, table, lens, 0.4, page_size)
    assert np.array_equal(got, oracle.decode(q, k, v, lens, 0.4))


def test_page_order_does_not_matter():
    B, h_q, n_kv, S, d, ps = 2, 6, 3, 12, 4, 4
    q, k, v = _rand(B, h_q, d, seed=4), _rand(B, n_kv, S, d, seed=5), _rand(B, n_kv, S, d, seed=6)
    lens = [12, 7]
    order = list(np.random.default_rng(7).permutation(B * S // ps + 2)[:B * S // ps])
    kp, table = _cut(k, ps, order)
    vp, _ = _cut(v, ps, order)
    got = oracle.decode_paged(q, kp, vp, table, lens, 0.3, ps)
    np.testing.assert_allclose(got, oracle.decode(q, k, v, lens, 0.3), rtol=0, atol=1e-14)


def test_block_table_picks_the_logical_token():
    """One key dominates; V rows are one-hot in the logical token index, so the
    output names which stored slot the block table mapped that token to."""
    ps, n_pages, d = 2, 3, 6
    # logical tokens 0..5 of one sequence; logical page i lives in physical page table[i]
    table = np.array([[2, 0, 1]])
    kp = np.zeros((n_pages, 1, ps, d))
    vp = np.zeros((n_pages, 1, ps, d))
    for t in range(6):
        p, s = table[0, t // ps], t % ps
        vp[p, 0, s, t] = 1.0
    star = 3
    p, s = table[0, star // ps], star % ps
    kp[p, 0, s, 0] = 200.0
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    out = oracle.decode_paged(q, kp, vp, table, [6], 1.0, ps)
    assert np.argmax(out[0, 0]) == star and out[0, 0, star] > 1 - 1e-12


def test_slots_past_the_length_and_unused_entries_are_not_read():
    ps, d = 4, 3
    q = _rand(1, 2, d, seed=8)
    kp = _rand(3, 1, ps, d, seed=9)
    vp = _rand(3, 1, ps, d, seed=10)
    clean = oracle.decode_paged(q, kp, vp, np.array([[1, 0, 2]]), [5], 0.7, ps)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[0, :, 1:], vp2[0, :, 1:] = np.nan, np.nan   # tokens 5..7 of the sequence (page 2 of the table is unused)
    kp2[2], vp2[2] = np.nan, np.nan
    got = oracle.decode_paged(q, kp2, vp2, np.array([[1, 0, -9]]), [5], 0.7, ps)
    assert np.array_equal(got, clean)


def test_a_used_entry_outside_the_pool_is_an_error():
    with pytest.raises(ValueError):
        oracle.decode_paged(np.zeros((1, 1, 2)), np.zeros((2, 1, 2, 2)), np.zeros((2, 1, 2, 2)),
                            np.array([[0, 5]]), [3], 1.0, 2)


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8"])
def test_paged_input_generator_scatters_the_contiguous_cache(kd):
    qd = "f32" if kd == "f32" else "bf16"
    wl = inputs.DecodeWorkload("pg", B=3, h_q=8, n_kv=2, d_h=64, S_max=128, q_dtype=qd, kv_dtype=kd,
                               lens=(1, 128), seed=11)
    pin = inputs.make_paged_decode_inputs(wl, 32, junk_unused_entries=True)
    base = pin.base
    lens = base.seq_lens.tolist()
    for b in range(wl.B):
        used = (lens[b] + 31) // 32
        for i in range(4):
            p = int(pin.block_table[b, i])
            if i >= used:
                assert p == -1
                continue
            assert torch.equal(pin.k_pages[p], base.k[b, :, 32 * i:32 * (i + 1)])
            assert torch.equal(pin.v_pages[p], base.v[b, :, 32 * i:32 * (i + 1)])
            if kd == "fp8":
                assert torch.equal(pin.k_scale_pages[p], base.k_scale[b, :, 32 * i:32 * (i + 1)])
    used_pages = {int(x) for x in pin.block_table.flatten() if x >= 0}
    assert len(used_pages) == sum((n + 31) // 32 for n in lens)


def test_sequences_sharing_a_prefix_page_read_it_each():
    """Two sequences whose tables name the same first page (a shared prompt
    prefix) each attend to it: equal to contiguous caches that both hold a copy."""
    ps, n_kv, d = 4, 2, 3
    shared_k, shared_v = _rand(n_kv, ps, d, seed=12), _rand(n_kv, ps, d, seed=13)
    tail_k, tail_v = _rand(2, n_kv, ps, d, seed=14), _rand(2, n_kv, ps, d, seed=15)
    kp = np.stack([shared_k, tail_k[0], tail_k[1]])
    vp = np.stack([shared_v, tail_v[0], tail_v[1]])
    table = np.array([[0, 1], [0, 2]])
    q = _rand(2, 4, d, seed=16)
    lens = [7, 6]
    k = np.stack([np.concatenate([shared_k, tail_k[b]], axis=1) for b in range(2)])
    v = np.stack([np.concatenate([shared_v, tail_v[b]], axis=1) for b in range(2)])
    got = oracle.decode_paged(q, kp, vp, table, lens, 0.5, ps)
    assert np.array_equal(got, oracle.decode(q, k, v, lens, 0.5))
