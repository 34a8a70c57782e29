"""Pins of the general-mask prefill oracle (oracle/masked.py) and of the
per-head fp8 dequantiser: hand-built visibility, the pages' module code and
torch SDPA as library routines (with masks built independently of the
oracle), the causal and decode oracles as special cases, invariants and
brute force."""

from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask_torch(B, S_q, S_k, causal, kv_lens, dense):
    """The combined mask built with torch primitives only (tril with an offset
    for the end-aligned causal rule, an arange comparison for the lengths)."""
    m = torch.ones(B, S_q, S_k, dtype=torch.bool)
    if causal:
        m &= torch.ones(S_q, S_k, dtype=torch.bool).tril(diagonal=S_k - S_q)
    if kv_lens is not None:
        m &= torch.arange(S_k)[None, None, :] < torch.as_tensor(kv_lens)[:, None, None]
    if dense is not None:
        m &= torch.from_numpy(np.asarray(dense)) != 0
    return m


def test_visible_keys_hand_built():
    # 2 queries at the end of 5 keys: row 0 is key position 3, row 1 position 4
    assert oracle.visible_keys(2, 5, True).astype(int).tolist() == [[1, 1, 1, 1, 0], [1, 1, 1, 1, 1]]
    # more queries than keys: the first row sees nothing
    assert oracle.visible_keys(3, 2, True).astype(int).tolist() == [[0, 0], [1, 0], [1, 1]]
    # key padding, no causal rule
    assert oracle.visible_keys(2, 5, False, kv_len=3).astype(int).tolist() == [[1, 1, 1, 0, 0]] * 2
    # any nonzero mask value keeps the key; all three combine by AND
    dense = np.array([[7, 0, 1, 1], [1, 1, 0, 255]], dtype=np.uint8)
    assert oracle.visible_keys(2, 4, True, kv_len=3, mask_b=dense).astype(int).tolist() == \
        [[1, 0, 1, 0], [1, 1, 0, 0]]


def _module_attention(q, k, v, scale, attention_mask):
    """Masked grouped-query attention written from the definition, in torch
    float64 on the CPU: query head j reads K/V head j // G (contiguous groups,
    the head order of "GQA Implementation" in "Evolution of AI Attention
    Mechanisms"); for every (batch, head) the scores are scale * Q K^T, a key
    the mask hides scores -inf, each row is soft-maxed and multiplies V.
    q [B,S_q,h,d], k/v [B,S_k,n_kv,d], attention_mask [B,S_q,S_k] bool ->
    [B,S_q,h,d]."""
    B, S_q, h, d = q.shape
    G = h // k.shape[2]
    kv_head = np.arange(h) // G
    out = np.zeros_like(q)
    for b in range(B):
        hidden = ~attention_mask[b].numpy()
        for j in range(h):
            kk = torch.from_numpy(k[b, :, kv_head[j], :])
            vv = torch.from_numpy(v[b, :, kv_head[j], :])
            s = (torch.from_numpy(q[b, :, j, :]) @ kk.T) * scale
            s[torch.from_numpy(hidden)] = float("-inf")
            out[b, :, j, :] = (torch.softmax(s, dim=-1) @ vv).numpy()
    return out


CASES = [
    # (B, S_q, S_k, h_q, n_kv, causal, kv_lens, with dense mask)
    (2, 7, 7, 4, 2, True, None, False),
    (2, 5, 9, 4, 1, True, None, False),
    (2, 6, 6, 2, 2, False, [6, 3], False),
    (3, 4, 11, 6, 3, True, [11, 8, 5], True),
    (2, 8, 8, 4, 4, False, None, True),
]


@pytest.mark.parametrize("B,S_q,S_k,h_q,n_kv,causal,kv_lens,dense", CASES)
def test_matches_module_code_and_sdpa(B, S_q, S_k, h_q, n_kv, causal, kv_lens, dense):
    d = 8
    q, k, v = _rand(B, S_q, h_q, d, seed=1), _rand(B, S_k, n_kv, d, seed=2), _rand(B, S_k, n_kv, d, seed=3)
    dm = (np.random.default_rng(4).random((B, S_q, S_k)) < 0.7).astype(np.uint8) * 3 if dense else None
    got = oracle.prefill(q, k, v, 0.3, causal=causal, kv_lens=kv_lens, mask=dm)
    m = _mask_torch(B, S_q, S_k, causal, kv_lens, dm)
    has = m.any(-1).numpy()                                  # [B, S_q] rows with a visible key
    mod = _module_attention(q, k, v, 0.3, m)
    sd = F.scaled_dot_product_attention(*(torch.from_numpy(x).transpose(1, 2) for x in (q, k, v)),
                                        attn_mask=m[:, None], scale=0.3, enable_gqa=True).transpose(1, 2).numpy()
    np.testing.assert_allclose(got[has], mod[has], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[has], sd[has], rtol=0, atol=1e-13)
    assert np.all(got[~has] == 0)


def test_causal_square_equals_causal_oracle():
    q, k, v = _rand(2, 9, 4, 8, seed=5), _rand(2, 9, 2, 8, seed=6), _rand(2, 9, 2, 8, seed=7)
    np.testing.assert_allclose(oracle.prefill(q, k, v, 0.4, causal=True), oracle.prefill_causal(q, k, v, 0.4),
                               rtol=0, atol=1e-15)


def test_unmasked_rows_equal_decode_rows():
    """Without any mask every query row is one decode step over all keys."""
    q, k, v = _rand(2, 5, 4, 8, seed=8), _rand(2, 7, 2, 8, seed=9), _rand(2, 7, 2, 8, seed=10)
    got = oracle.prefill(q, k, v, 0.25)
    for r in range(5):
        ref = oracle.decode(q[:, r], k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3), [7, 7], 0.25)
        np.testing.assert_allclose(got[:, r], ref, rtol=0, atol=1e-14)


def test_key_lengths_truncate_and_never_read_the_tail():
    q, k, v = _rand(1, 4, 2, 8, seed=11), _rand(1, 10, 1, 8, seed=12), _rand(1, 10, 1, 8, seed=13)
    ref = oracle.prefill(q, k[:, :6], v[:, :6], 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[:, 6:] = np.nan
    v2[:, 6:] = np.nan
    np.testing.assert_array_equal(oracle.prefill(q, k2, v2, 0.5, kv_lens=[6]), ref)
    # lengths are clamped to [0, S_k]; zero gives zero rows
    np.testing.assert_array_equal(oracle.prefill(q, k, v, 0.5, kv_lens=[99]), oracle.prefill(q, k, v, 0.5))
    assert np.all(oracle.prefill(q, k, v, 0.5, kv_lens=[0]) == 0)


def test_joint_permutation_of_keys_and_mask_columns():
    q, k, v = _rand(1, 6, 2, 8, seed=14), _rand(1, 9, 2, 8, seed=15), _rand(1, 9, 2, 8, seed=16)
    dm = (np.random.default_rng(17).random((1, 6, 9)) < 0.6).astype(np.uint8)
    perm = np.random.default_rng(18).permutation(9)
    a = oracle.prefill(q, k, v, 0.7, mask=dm)
    b = oracle.prefill(q, k[:, perm], v[:, perm], 0.7, mask=dm[:, :, perm])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_single_visible_key_returns_its_value_row():
    q, k, v = _rand(1, 3, 1, 4, seed=19), _rand(1, 5, 1, 4, seed=20), _rand(1, 5, 1, 4, seed=21)
    dm = np.zeros((1, 3, 5), dtype=np.uint8)
    dm[0, 0, 2] = dm[0, 1, 4] = 1
    out = oracle.prefill(q, k, v, 1.3, mask=dm)
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 2, 0])
    np.testing.assert_array_equal(out[0, 1, 0], v[0, 4, 0])
    assert np.all(out[0, 2] == 0)


def test_brute_force_tiny_decimal():
    getcontext().prec = 50
    q, k, v = _rand(1, 3, 2, 3, seed=22), _rand(1, 5, 1, 3, seed=23), _rand(1, 5, 1, 3, seed=24)
    dm = np.array([[[1, 0, 1, 1, 0], [0, 1, 1, 0, 1], [1, 1, 1, 1, 1]]], dtype=np.uint8)
    out = oracle.prefill(q, k, v, 0.9, causal=True, mask=dm)   # row r sees keys <= r + 2
    for r in range(3):
        keys = [c for c in range(5) if c <= r + 2 and dm[0, r, c]]
        for j in range(2):
            s = [Decimal(0.9) * sum(Decimal(q[0, r, j, i]) * Decimal(k[0, c, 0, i]) for i in range(3)) for c in keys]
            e = [x.exp() for x in s]
            z = sum(e)
            ref = [float(sum(e[t] * Decimal(v[0, c, 0, i]) for t, c in enumerate(keys)) / z) for i in range(3)]
            np.testing.assert_allclose(out[0, r, j], ref, rtol=0, atol=1e-14)


def test_rows_function_matches_full():
    q, k, v = _rand(2, 6, 4, 8, seed=25), _rand(2, 9, 2, 8, seed=26), _rand(2, 9, 2, 8, seed=27)
    dm = (np.random.default_rng(28).random((2, 6, 9)) < 0.5).astype(np.uint8)
    full = oracle.prefill(q, k, v, 0.3, causal=True, kv_lens=[9, 4], mask=dm)
    trip = [(0, 0, 0), (1, 5, 3), (1, 2, 1), (0, 3, 2)]
    rows = oracle.masked.prefill_rows(q, k, v, 0.3, trip, causal=True, kv_lens=[9, 4], mask=dm)
    for i, (b, r, j) in enumerate(trip):
        np.testing.assert_allclose(rows[i], full[b, r, j], rtol=0, atol=1e-14)


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((1, 2, 2, 4)), np.zeros((1, 3, 1, 4)), np.zeros((1, 3, 1, 5)), 1.0)
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((1, 2, 2, 4)), np.zeros((1, 3, 1, 4)), np.zeros((1, 3, 1, 4)), 1.0,
                       mask=np.ones((1, 3, 2)))


def test_fp8_per_head_dequantisation():
    codes = np.array([[[[0x38, 0xB8]], [[0x7E, 0x01]]]], dtype=np.uint8)  # [1, 2, 1, 2]: 1, -1, 448, 2^-9
    out = oracle.dequantize_fp8_heads(codes, np.array([[0.5]], dtype=np.float32))
    np.testing.assert_array_equal(out[0, :, 0], [[0.5, -0.5], [224.0, 2.0 ** -10]])
    with pytest.raises(TypeError):
        oracle.dequantize_fp8_heads(codes, np.array([[0.5]]))
    with pytest.raises(ValueError):
        oracle.dequantize_fp8_heads(codes, np.ones((1, 2), dtype=np.float32))


def test_zero_descale_head_gives_the_mean_of_visible_values():
    """An all-zero head quantised by absmax has descale 0: its values decode
    to exactly 0, so every visible score of a zero query head is 0 and the
    softmax weights are equal -- each output row is the mean of the V rows it
    sees (closed form), never NaN."""
    rng = np.random.default_rng(11)
    B, S, h, n_kv, d = 1, 6, 2, 1, 8
    codes = rng.integers(0, 0x7F, size=(B, S, h, d), dtype=np.uint8)   # finite codes only
    qv = oracle.dequantize_fp8_heads(codes, np.array([[0.0, 0.25]], dtype=np.float32))
    assert np.all(qv[:, :, 0] == 0.0)
    k, v = _rand(B, S, n_kv, d, seed=5), _rand(B, S, n_kv, d, seed=6)
    out = oracle.prefill(qv, k, v, 0.3, causal=True, kv_lens=[5])
    for r in range(S):
        n = min(r + 1, 5)
        np.testing.assert_allclose(out[0, r, 0], v[0, :n, 0].mean(axis=0), rtol=0, atol=1e-15)
    assert np.all(np.isfinite(out))
