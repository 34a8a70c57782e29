"""Pins of the absorbed-MLA decode oracle (oracle/mla.py): the explicit
per-head attention it stands for, the MQA decode it reduces to, and closed
forms."""

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_absorbed_form_equals_explicit_per_head_attention():
    """With random up-projections, attending with explicit K_h = c W_k,h^T and
    V_h = c W_v,h^T equals the absorbed form followed by W_v,h."""
    r = _rng(1)
    B, h, hd, d_c, S = 2, 3, 4, 6, 9
    W_k = r.standard_normal((h * hd, d_c))  # k_up_proj weight [hidden, d_c]
    W_v = r.standard_normal((h * hd, d_c))
    q = r.standard_normal((B, h, hd))
    c = r.standard_normal((B, S, d_c))
    lens = [9, 5]
    scale = 0.3
    q_abs = np.stack([np.stack([W_k[j * hd:(j + 1) * hd].T @ q[b, j] for j in range(h)]) for b in range(B)])
    o_c = oracle.mla_decode(q_abs, c, lens, scale)
    for b in range(B):
        for j in range(h):
            K = c[b, :lens[b]] @ W_k[j * hd:(j + 1) * hd].T  # [n, hd]
            V = c[b, :lens[b]] @ W_v[j * hd:(j + 1) * hd].T
            explicit = oracle.attend_one_row(q[b, j], K, V, scale)
            np.testing.assert_allclose(W_v[j * hd:(j + 1) * hd] @ o_c[b, j], explicit, rtol=1e-12, atol=1e-12)


def test_equals_mqa_decode_with_the_latent_as_keys_and_values():
    r = _rng(2)
    B, h, d_c, S = 3, 4, 8, 10
    q_abs, c = r.standard_normal((B, h, d_c)), r.standard_normal((B, S, d_c))
    lens = [10, 1, 6]
    got = oracle.mla_decode(q_abs, c, lens, 0.25)
    ref = oracle.decode(q_abs, c[:, None], c[:, None], lens, 0.25)  # one K/V head shared by all h
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_closed_forms():
    r = _rng(3)
    c = r.standard_normal((1, 5, 4))
    q = r.standard_normal((1, 2, 4))
    # a single visible token returns its latent row for every head
    assert np.allclose(oracle.mla_decode(q, c, [1], 0.7)[0], np.tile(c[0, 0], (2, 1)))
    # scale 0: the mean of the visible latent rows
    assert np.allclose(oracle.mla_decode(q, c, [4], 0.0)[0, 1], c[0, :4].mean(0))
    # L = 0: zero rows; tokens past L are never read
    assert np.all(oracle.mla_decode(q, c, [0], 1.0) == 0)
    c2 = c.copy()
    c2[0, 3:] = np.nan
    assert np.array_equal(oracle.mla_decode(q, c2, [3], 0.4), oracle.mla_decode(q, c, [3], 0.4))


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.mla_decode(np.zeros((1, 2, 4)), np.zeros((1, 3, 5)), [1], 1.0)
