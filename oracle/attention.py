"""Exact grouped-query attention in float64, scores materialised -- the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ("Evolution of AI Attention Mechanisms", sections
"MHA Mathematical Formulation", "MHA Implementation", "GQA Implementation";
"Multi-query attention", section "Formulation"):

    for query head j, with G = h_q / n_kv and K/V head g = j // G,
        scores = scale * q_j . k_t            for every visible key t
        p      = softmax(scores)              (over the visible keys)
        out_j  = sum_t p_t * v_t

* Head map.  The GQA module repeats each K/V head n_rep = G times with an
  expand over a new axis placed right after the K/V-head axis followed by a
  reshape to h_q heads, so repeated copy number r of K/V head g lands at query
  head g * G + r; query head j therefore reads K/V head j // G.
* Scale.  The modules multiply q K^T by head_dim ** -0.5 after the dot
  product; here `scale` is an argument (the callers pass 1/sqrt(d_h)).
* Visibility.  Decode: the new token's K/V is concatenated onto the cache
  before attention, so all L_b cached positions (the new one included) are
  visible.  Prefill: causal, query row r sees keys 0..r (S_q == S_k, diagonal
  kept), the `causal=True` mode of the library call in "Flash Attention Usage".
  Masked scores are set to -inf before the softmax, as the modules'
  masked_fill does.
* Softmax is evaluated in the max-subtracted form exp(s - max s) / sum, which
  is the same function as the modules' torch.softmax.
* A row with no visible key (L_b = 0) is defined here as an all-zero output;
  the pages leave it undefined (their code would produce NaN).

Layouts: decode q [B, h_q, d], caches [B, n_kv, S_max, d] (the cache layout
after the modules' view(B, S, n_kv, d).transpose(1, 2)); prefill q/k/v/out
[B, S, H, d] (the layout handed to flash_attn_func).
"""

import numpy as np


def _check_group(h_q, n_kv):
    if n_kv <= 0 or h_q % n_kv != 0:
        raise ValueError(f"h_q={h_q} is not a multiple of n_kv={n_kv}")
    return h_q // n_kv


def attend_one_row(q_vec, keys, values, scale):
    """softmax(scale * keys @ q_vec) @ values for one query row (float64).

    keys/values: [n, d]; n == 0 gives a zero row.
    """
    q_vec = np.asarray(q_vec, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    scores = scale * (keys @ q_vec)
    shifted = np.exp(scores - scores.max())
    p = shifted / shifted.sum()
    return p @ values


def decode(q, k_cache, v_cache, seq_lens, scale):
    """One decode step for a batch of sequences.

    q [B, h_q, d]; k_cache, v_cache [B, n_kv, S_max, d] (float64 values);
    seq_lens [B] (number of cached tokens, the current one included; values
    above S_max are clamped to S_max, values below 0 to 0).  Returns
    [B, h_q, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, h_q, d = q.shape
    _, n_kv, s_max, _ = k_cache.shape
    G = _check_group(h_q, n_kv)
    out = np.zeros((B, h_q, d), dtype=np.float64)
    for b in range(B):
        n = int(min(max(int(seq_lens[b]), 0), s_max))
        for j in range(h_q):
            g = j // G
            out[b, j] = attend_one_row(q[b, j], k_cache[b, g, :n], v_cache[b, g, :n], scale)
    return out


def decode_rows(q, k_cache, v_cache, seq_lens, scale, pairs):
    """decode() evaluated only for the listed (b, j) pairs -> [len(pairs), d]."""
    q = np.asarray(q, dtype=np.float64)
    B, h_q, d = q.shape
    n_kv, s_max = k_cache.shape[1], k_cache.shape[2]
    G = _check_group(h_q, n_kv)
    rows = []
    for b, j in pairs:
        n = int(min(max(int(seq_lens[b]), 0), s_max))
        g = j // G
        rows.append(attend_one_row(q[b, j], k_cache[b, g, :n], v_cache[b, g, :n], scale))
    return np.stack(rows) if rows else np.zeros((0, d))


def prefill_causal(q, k, v, scale):
    """Causal self-attention over a whole prompt, scores materialised.

    q [B, S, h_q, d]; k, v [B, S, n_kv, d] (float64 values).  For each batch
    entry and query head the full S x S score matrix is formed, entries with
    key index > query index are set to -inf, each row is soft-maxed and the
    result multiplies V.  Returns [B, S, h_q, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, h_q, d = q.shape
    n_kv = k.shape[2]
    G = _check_group(h_q, n_kv)
    out = np.zeros((B, S, h_q, d), dtype=np.float64)
    if S == 0:
        return out
    future = np.triu(np.ones((S, S), dtype=bool), k=1)  # key index > query index
    for b in range(B):
        for j in range(h_q):
            g = j // G
            scores = scale * (q[b, :, j, :] @ k[b, :, g, :].T)
            scores[future] = -np.inf
            shifted = np.exp(scores - scores.max(axis=1, keepdims=True))
            p = shifted / shifted.sum(axis=1, keepdims=True)
            out[b, :, j, :] = p @ v[b, :, g, :]
    return out


def prefill_rows(q, k, v, scale, triples):
    """prefill_causal() evaluated only at the listed (b, r, j) query rows.

    Row r of the causal product attends to keys 0..r of its K/V head.
    Returns [len(triples), d] float64.
    """
    B, S, h_q, d = q.shape
    n_kv = k.shape[2]
    G = _check_group(h_q, n_kv)
    rows = []
    for b, r, j in triples:
        g = j // G
        rows.append(attend_one_row(q[b, r, j], k[b, : r + 1, g], v[b, : r + 1, g], scale))
    return np.stack(rows) if rows else np.zeros((0, d))
