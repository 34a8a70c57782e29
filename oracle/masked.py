"""Prefill attention with general masks, float64 -- the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:
  * "Evolution of AI Attention Mechanisms", section "MHA Implementation": the
    module forms scale * q k^T, sets every score whose attention_mask entry
    is 0 to -inf, soft-maxes over the keys and multiplies by V; K and V may
    hold cached keys ahead of the new ones (the module concatenates past_kv
    first), so there can be more keys than queries.
  * Same page, section "Flash Attention Usage": flash_attn_func with
    causal=True / False.
  * Same page, "GQA Implementation": query head j reads K/V head j // G.

Readings taken where the pages leave a step open:
  * causal with S_k keys and S_q queries is aligned at the end: query row r
    sits at position r + S_k - S_q of the key sequence and sees keys
    c <= r + S_k - S_q (with S_q = S_k this is the usual c <= r);
  * kv_lens[b] (optional) makes keys c >= kv_lens[b] invisible to every query
    row of sequence b (padding of a ragged batch);
  * mask[b, r, c] (optional, shared by all heads) makes key c invisible to row
    r where it is 0; any nonzero value keeps it, as with the module's
    `attention_mask == 0` test;
  * the three conditions combine by AND, and a row with no visible key gives
    a zero output row (the module's code would give NaN);
  * keys at or past kv_lens[b] are never read (their rows may hold anything,
    NaN included); keys hidden only by the causal rule or by the mask are
    multiplied by a zero weight, so their values must be finite.
"""

import numpy as np

from .attention import _check_group


def visible_keys(S_q, S_k, causal, kv_len=None, mask_b=None):
    """bool [S_q, S_k]: which keys each query row of one sequence may see."""
    vis = np.ones((S_q, S_k), dtype=bool)
    if causal:
        r = np.arange(S_q)[:, None]
        c = np.arange(S_k)[None, :]
        vis &= c <= r + (S_k - S_q)
    if kv_len is not None:
        vis[:, int(min(max(int(kv_len), 0), S_k)):] = False
    if mask_b is not None:
        vis &= np.asarray(mask_b) != 0
    return vis


def prefill(q, k, v, scale, causal=False, kv_lens=None, mask=None):
    """q [B, S_q, h_q, d]; k, v [B, S_k, n_kv, d] (float64 values);
    kv_lens [B] or None; mask [B, S_q, S_k] or None -> [B, S_q, h_q, d].

    For each batch entry and query head the full S_q x S_k score matrix is
    formed, invisible entries are set to -inf, rows with a visible key are
    soft-maxed (max-shifted) and multiply V; other rows are zero."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S_q, h_q, d = q.shape
    S_k, n_kv = k.shape[1], k.shape[2]
    if k.shape != (B, S_k, n_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, S_k, n_kv, d] matching q [B, S_q, h_q, d]")
    if mask is not None and np.shape(mask) != (B, S_q, S_k):
        raise ValueError("mask must be [B, S_q, S_k]")
    G = _check_group(h_q, n_kv)
    out = np.zeros((B, S_q, h_q, d), dtype=np.float64)
    for b in range(B):
        n = S_k if kv_lens is None else int(min(max(int(kv_lens[b]), 0), S_k))
        vis = visible_keys(S_q, S_k, causal, None if kv_lens is None else kv_lens[b],
                           None if mask is None else mask[b])[:, :n]
        rows = vis.any(axis=1)
        if not rows.any():
            continue
        for j in range(h_q):
            g = j // G
            s = scale * (q[b, :, j, :] @ k[b, :n, g, :].T)  # [S_q, n], materialised
            s = np.where(vis, s, -np.inf)[rows]
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            out[b, rows, j, :] = p @ v[b, :n, g, :]
    return out


def prefill_rows(q, k, v, scale, triples, causal=False, kv_lens=None, mask=None):
    """prefill() evaluated only at the listed (b, r, j) query rows -> [len, d]."""
    B, S_q, h_q, d = q.shape
    S_k, n_kv = k.shape[1], k.shape[2]
    G = _check_group(h_q, n_kv)
    rows = []
    for b, r, j in triples:
        vis = visible_keys(S_q, S_k, causal, None if kv_lens is None else kv_lens[b],
                           None if mask is None else mask[b])[r]
        if not vis.any():
            rows.append(np.zeros(d))
            continue
        g = j // G
        kk = np.asarray(k[b, :, g, :], dtype=np.float64)[vis]
        vv = np.asarray(v[b, :, g, :], dtype=np.float64)[vis]
        s = scale * (kk @ np.asarray(q[b, r, j, :], dtype=np.float64))
        e = np.exp(s - s.max())
        rows.append((e / e.sum()) @ vv)
    return np.stack(rows)
