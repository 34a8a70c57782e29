"""Pins for the fp64 oracle: closed forms, invariants the pages fix, a library
routine computing the same definition, and brute force on tiny inputs.

Each test is chosen so that a plausible slip in the oracle (dropped scale,
wrong softmax axis, wrong head map, mask off by one, missing max shift,
transposed operand) fails at least one of them.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20261203)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_its_value_row():
    # softmax over one key is 1 -> output is exactly that V row
    q = _rand(1, 4, 8)
    k = _rand(1, 2, 5, 8)
    v = _rand(1, 2, 5, 8)
    out = oracle.decode(q, k, v, [1], 0.3)
    for j in range(4):
        assert np.array_equal(out[0, j], v[0, j // 2, 0])


def test_identical_keys_give_mean_of_values():
    q = _rand(2, 2, 6)
    k = np.broadcast_to(_rand(2, 1, 1, 6), (2, 1, 7, 6)).copy()
    v = _rand(2, 1, 7, 6)
    out = oracle.decode(q, k, v, [7, 4], 0.9)
    np.testing.assert_allclose(out[0, 0], v[0, 0, :7].mean(0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1, 1], v[1, 0, :4].mean(0), rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_uniform_weights_give_mean(mode):
    q = np.zeros((1, 3, 4)) if mode == "zero_q" else _rand(1, 3, 4)
    scale = 0.5 if mode == "zero_q" else 0.0
    k, v = _rand(1, 3, 9, 4), _rand(1, 3, 9, 4)
    out = oracle.decode(q, k, v, [6], scale)
    for j in range(3):
        np.testing.assert_allclose(out[0, j], v[0, j, :6].mean(0), rtol=0, atol=1e-15)


def test_two_keys_logistic_weight():
    # p1 = 1 / (1 + exp(s2 - s1)), s_t = scale * q . k_t
    q, k, v = _rand(1, 1, 5), _rand(1, 1, 2, 5), _rand(1, 1, 2, 5)
    scale = 0.37
    s1, s2 = scale * q[0, 0] @ k[0, 0, 0], scale * q[0, 0] @ k[0, 0, 1]
    p1 = 1.0 / (1.0 + math.exp(s2 - s1))
    expect = p1 * v[0, 0, 0] + (1 - p1) * v[0, 0, 1]
    np.testing.assert_allclose(oracle.decode(q, k, v, [2], scale)[0, 0], expect, rtol=0, atol=1e-15)


def test_head_map_is_contiguous_groups():
    # n_kv = 4, G = 2; V of K/V head g is the constant g + 1, so query head j
    # must return j // G + 1 exactly (j % n_kv would give a different pattern).
    B, h_q, n_kv, S, d = 1, 8, 4, 5, 3
    q, k = _rand(B, h_q, d), _rand(B, n_kv, S, d)
    v = np.zeros((B, n_kv, S, d))
    for g in range(n_kv):
        v[:, g] = g + 1.0
    out = oracle.decode(q, k, v, [S], 0.4)
    for j in range(h_q):
        np.testing.assert_allclose(out[0, j], np.full(d, j // 2 + 1.0), rtol=0, atol=1e-14)
    # same for prefill
    qp, kp = _rand(1, 3, h_q, d), _rand(1, 3, n_kv, d)
    vp = np.zeros((1, 3, n_kv, d))
    for g in range(n_kv):
        vp[:, :, g] = g + 1.0
    outp = oracle.prefill_causal(qp, kp, vp, 0.4)
    for j in range(h_q):
        np.testing.assert_allclose(outp[0, :, j], np.full((3, d), j // 2 + 1.0), rtol=0, atol=1e-14)


def test_hard_max_limit_and_stability():
    # With huge scores the softmax is one-hot on the largest score; the
    # max-shifted form must not overflow (exp(2000) is inf in float64).
    q = np.zeros((1, 1, 2))
    q[0, 0] = [1.0, 0.0]
    k = np.zeros((1, 1, 4, 2))
    k[0, 0, :, 0] = [1.0, 3.0, 2.0, -1.0]
    v = _rand(1, 1, 4, 2)
    out = oracle.decode(q, k, v, [4], 1000.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0, 0], v[0, 0, 1], rtol=0, atol=1e-15)
    # prefill: query row r picks the largest visible key
    qp = np.zeros((1, 4, 1, 2))
    qp[0, :, 0] = [1.0, 0.0]
    kp = k.transpose(0, 2, 1, 3)
    vp = v.transpose(0, 2, 1, 3)
    outp = oracle.prefill_causal(qp, kp, vp, 1000.0)
    assert np.all(np.isfinite(outp))
    for r, best in enumerate([0, 1, 1, 1]):
        np.testing.assert_allclose(outp[0, r, 0], vp[0, best, 0], rtol=0, atol=1e-15)


# ------------------------------------------------------------------ invariants

def test_weights_sum_to_one_via_constant_values():
    # V = 1 everywhere -> output 1 everywhere (rows of p sum to 1), p >= 0 by
    # construction checked through a one-hot V column
    q, k = _rand(2, 4, 8), _rand(2, 2, 11, 8)
    out = oracle.decode(q, k, np.ones((2, 2, 11, 8)), [11, 3], 0.35)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    vpos = np.zeros((2, 2, 11, 8))
    vpos[..., 0] = 1.0
    vpos[:, :, 5, 1] = 1.0
    w = oracle.decode(q, k, vpos, [11, 11], 0.35)
    assert np.all(w[..., 1] >= 0) and np.all(w[..., 1] <= 1)


def test_scale_moves_between_query_and_scale():
    q, k, v = _rand(1, 4, 8), _rand(1, 2, 9, 8), _rand(1, 2, 9, 8)
    a = oracle.decode(q, k, v, [9], 0.25)
    b = oracle.decode(4.0 * q, k, v, [9], 0.0625)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    c = oracle.decode(q, k, v, [9], 0.5)
    assert np.max(np.abs(a - c)) > 1e-3  # the scale does matter


def test_linear_in_values_and_permutation_invariant():
    q, k = _rand(1, 2, 6), _rand(1, 1, 10, 6)
    v1, v2 = _rand(1, 1, 10, 6), _rand(1, 1, 10, 6)
    lhs = oracle.decode(q, k, 2.0 * v1 - 3.0 * v2, [10], 0.4)
    rhs = 2.0 * oracle.decode(q, k, v1, [10], 0.4) - 3.0 * oracle.decode(q, k, v2, [10], 0.4)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)
    perm = RNG.permutation(10)
    np.testing.assert_allclose(oracle.decode(q, k[:, :, perm], v1[:, :, perm], [10], 0.4),
                               oracle.decode(q, k, v1, [10], 0.4), rtol=0, atol=1e-14)


def test_tail_beyond_length_is_never_read():
    q, k, v = _rand(2, 2, 4), _rand(2, 1, 8, 4), _rand(2, 1, 8, 4)
    kp, vp = k.copy(), v.copy()
    kp[0, :, 5:] = np.nan
    vp[0, :, 5:] = np.nan
    kp[1, :, 2:] = np.nan
    vp[1, :, 2:] = np.nan
    a = oracle.decode(q, kp, vp, [5, 2], 0.5)
    b = oracle.decode(q, k[:, :, :5], v[:, :, :5], [5, 2], 0.5)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)


def test_empty_and_overlong_lengths():
    q, k, v = _rand(3, 2, 4), _rand(3, 2, 6, 4), _rand(3, 2, 6, 4)
    out = oracle.decode(q, k, v, [0, 99, -3], 0.5)
    assert np.array_equal(out[0], np.zeros((2, 4)))
    assert np.array_equal(out[2], np.zeros((2, 4)))
    np.testing.assert_array_equal(out[1], oracle.decode(q, k, v, [0, 6, 0], 0.5)[1])


def test_prefill_first_row_is_first_value_row():
    q, k, v = _rand(2, 7, 4, 8), _rand(2, 7, 2, 8), _rand(2, 7, 2, 8)
    out = oracle.prefill_causal(q, k, v, 0.3)
    for b in range(2):
        for j in range(4):
            assert np.array_equal(out[b, 0, j], v[b, 0, j // 2])


def test_prefill_causal_perturbation():
    q, k, v = _rand(1, 9, 2, 4), _rand(1, 9, 1, 4), _rand(1, 9, 1, 4)
    base = oracle.prefill_causal(q, k, v, 0.5)
    for c in (0, 4, 8):
        k2, v2 = k.copy(), v.copy()
        k2[0, c] += 5.0
        v2[0, c] -= 7.0
        out = oracle.prefill_causal(q, k2, v2, 0.5)
        np.testing.assert_array_equal(out[0, :c], base[0, :c])
        assert np.max(np.abs(out[0, c:] - base[0, c:])) > 1e-6


def test_decode_equals_last_prefill_row():
    # cache-then-attend: the decode step over L cached tokens is row L-1 of the
    # causal product over the same K/V
    S, h_q, n_kv, d = 12, 4, 2, 8
    q, k, v = _rand(1, S, h_q, d), _rand(1, S, n_kv, d), _rand(1, S, n_kv, d)
    pre = oracle.prefill_causal(q, k, v, 0.3)
    for L in (1, 5, 12):
        dec = oracle.decode(q[:, L - 1], k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3), [L], 0.3)
        np.testing.assert_allclose(dec[0], pre[0, L - 1], rtol=0, atol=1e-14)


def test_row_helpers_match_full_forms():
    q, k, v = _rand(2, 4, 4, 8), _rand(2, 4, 2, 8), _rand(2, 4, 2, 8)
    full = oracle.prefill_causal(q, k, v, 0.2)
    trip = [(0, 0, 0), (1, 3, 3), (1, 2, 1)]
    rows = oracle.prefill_rows(q, k, v, 0.2, trip)
    for i, (b, r, j) in enumerate(trip):
        np.testing.assert_allclose(rows[i], full[b, r, j], rtol=0, atol=1e-14)
    qd, kd, vd = _rand(2, 4, 8), _rand(2, 2, 6, 8), _rand(2, 2, 6, 8)
    fd = oracle.decode(qd, kd, vd, [6, 3], 0.2)
    rd = oracle.decode_rows(qd, kd, vd, [6, 3], 0.2, [(1, 3), (0, 1)])
    np.testing.assert_allclose(rd[0], fd[1, 3], rtol=0, atol=1e-15)
    np.testing.assert_allclose(rd[1], fd[0, 1], rtol=0, atol=1e-15)


# ------------------------------------------------- spectrum and head repetition

def _repeat_kv_heads(x, n_rep, axis):
    """Each K/V head repeated n_rep times in place along `axis`, so head j of
    the result is K/V head j // n_rep: the contiguous query groups of GQA
    ("GQA Implementation" in "Evolution of AI Attention Mechanisms"), giving
    an MHA problem with one K/V head per query head."""
    return np.repeat(x, n_rep, axis=axis)


@pytest.mark.parametrize("h_q,n_kv", [(8, 8), (8, 4), (8, 2), (8, 1)])
def test_gqa_equals_mha_on_repeated_kv(h_q, n_kv):
    B, S, d = 2, 10, 8
    q, k, v = _rand(B, h_q, d), _rand(B, n_kv, S, d), _rand(B, n_kv, S, d)
    kr = _repeat_kv_heads(k, h_q // n_kv, axis=1)
    vr = _repeat_kv_heads(v, h_q // n_kv, axis=1)
    lens = [10, 7]
    np.testing.assert_allclose(oracle.decode(q, k, v, lens, 0.3), oracle.decode(q, kr, vr, lens, 0.3),
                               rtol=0, atol=1e-15)
    qp, kp, vp = _rand(B, S, h_q, d), _rand(B, S, n_kv, d), _rand(B, S, n_kv, d)
    kpr = _repeat_kv_heads(kp, h_q // n_kv, axis=2)
    vpr = _repeat_kv_heads(vp, h_q // n_kv, axis=2)
    np.testing.assert_allclose(oracle.prefill_causal(qp, kp, vp, 0.3), oracle.prefill_causal(qp, kpr, vpr, 0.3),
                               rtol=0, atol=1e-15)


def test_mqa_is_one_shared_head_and_mha_is_independent_heads():
    B, h, S, d = 1, 4, 9, 8
    q, k, v = _rand(B, h, d), _rand(B, 1, S, d), _rand(B, 1, S, d)
    # MQA decoding step: softmax(Q_all K^T * scale) V with one shared K, V
    scores = 0.4 * (q[0] @ k[0, 0].T)
    p = np.exp(scores - scores.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(oracle.decode(q, k, v, [S], 0.4)[0], p @ v[0, 0], rtol=0, atol=1e-14)
    # MHA: each head alone equals a 1-head problem on its own K/V head
    km, vm = _rand(B, h, S, d), _rand(B, h, S, d)
    full = oracle.decode(q, km, vm, [S], 0.4)
    for j in range(h):
        one = oracle.decode(q[:, j:j + 1], km[:, j:j + 1], vm[:, j:j + 1], [S], 0.4)
        np.testing.assert_array_equal(full[:, j], one[:, 0])


# ------------------------------------------------------ a library routine pin

@pytest.mark.parametrize("h_q,n_kv", [(8, 2), (6, 6), (4, 1)])
def test_matches_torch_sdpa_float64(h_q, n_kv):
    import torch.nn.functional as F
    B, S, d = 2, 13, 16
    qp, kp, vp = _rand(B, S, h_q, d), _rand(B, S, n_kv, d), _rand(B, S, n_kv, d)
    tq, tk, tv = (torch.from_numpy(x).transpose(1, 2) for x in (qp, kp, vp))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.21, enable_gqa=True)
    np.testing.assert_allclose(oracle.prefill_causal(qp, kp, vp, 0.21), ref.transpose(1, 2).numpy(),
                               rtol=0, atol=1e-13)
    # decode with ragged lengths via a boolean key mask
    q, k, v = _rand(B, h_q, d), _rand(B, n_kv, S, d), _rand(B, n_kv, S, d)
    lens = [13, 5]
    mask = torch.zeros(B, 1, 1, S, dtype=torch.bool)
    for b, n in enumerate(lens):
        mask[b, ..., :n] = True
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None], torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=mask, scale=0.21, enable_gqa=True)[:, :, 0]
    np.testing.assert_allclose(oracle.decode(q, k, v, lens, 0.21), ref.numpy(), rtol=0, atol=1e-13)


# ------------------------------------------------------------- brute force

def _brute_force_decimal(q, K, V, scale):
    getcontext().prec = 50
    s = [Decimal(scale) * sum(Decimal(q[i]) * Decimal(K[t][i]) for i in range(len(q))) for t in range(len(K))]
    e = [x.exp() for x in s]  # no max shift: 50 digits absorb the range here
    z = sum(e)
    return [float(sum(e[t] * Decimal(V[t][i]) for t in range(len(K))) / z) for i in range(len(V[0]))]


def test_brute_force_tiny_decimal():
    q, k, v = _rand(2, 4, 3), _rand(2, 2, 5, 3), _rand(2, 2, 5, 3)
    lens = [5, 3]
    out = oracle.decode(q, k, v, lens, 0.7)
    for b in range(2):
        for j in range(4):
            g = j // 2
            ref = _brute_force_decimal(q[b, j].tolist(), k[b, g, :lens[b]].tolist(), v[b, g, :lens[b]].tolist(), 0.7)
            np.testing.assert_allclose(out[b, j], ref, rtol=0, atol=1e-14)
    qp, kp, vp = _rand(1, 4, 2, 3), _rand(1, 4, 1, 3), _rand(1, 4, 1, 3)
    outp = oracle.prefill_causal(qp, kp, vp, 0.7)
    for r in range(4):
        for j in range(2):
            ref = _brute_force_decimal(qp[0, r, j].tolist(), kp[0, :r + 1, 0].tolist(), vp[0, :r + 1, 0].tolist(), 0.7)
            np.testing.assert_allclose(outp[0, r, j], ref, rtol=0, atol=1e-14)


def test_rejects_non_divisible_heads():
    with pytest.raises(ValueError):
        oracle.decode(_rand(1, 6, 4), _rand(1, 4, 3, 4), _rand(1, 4, 3, 4), [3], 1.0)
