"""Absorbed multi-head latent attention decode, float64 -- the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ("Evolution of AI Attention Mechanisms", section
"Generation 3: MLA Multi-Head Latent Attention", "MLA Core Idea" and "MLA
Implementation"): the cache holds one latent vector c_kv (d_c values) per
token.  K and V of head h would be up-projections of it, K_h = c_kv W_k,h^T
and V_h = c_kv W_v,h^T; with the absorption step the query is moved into the
latent space instead, q_abs,h = W_k,h^T q_h, so that

    scores_h = scale * q_abs,h . c_kv[t]       (t over the visible tokens)
    o_c,h    = softmax(scores_h) @ c_kv        (the page's attn_to_c)

and the up-projection W_v,h is applied to o_c,h afterwards (outside this
function, like the page's v_up_proj and o_proj).  The latent cache thus
serves as both keys and values of one head shared by every query head.

Reading taken where the page's code is garbled: it multiplies each head's
query (head_dim values) by the whole k_up_proj weight; the absorption
identity it states needs each head's own rows W_k,h of that weight, which is
the reading pinned in the tests (explicit per-head attention with random
up-projections equals the absorbed form followed by W_v,h).
"""

import numpy as np


def mla_decode(q_abs, c_kv, seq_lens, scale):
    """q_abs [B, h, d_c], c_kv [B, S_max, d_c] float64, seq_lens [B] ->
    o_c [B, h, d_c].  A row with L_b = 0 is zero."""
    q_abs = np.asarray(q_abs, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    B, h, d_c = q_abs.shape
    if c_kv.shape[0] != B or c_kv.shape[2] != d_c:
        raise ValueError("c_kv must be [B, S_max, d_c] matching q_abs [B, h, d_c]")
    out = np.zeros((B, h, d_c), dtype=np.float64)
    for b in range(B):
        n = int(min(max(int(seq_lens[b]), 0), c_kv.shape[1]))
        if n == 0:
            continue
        c = c_kv[b, :n]                       # [n, d_c]
        s = scale * (q_abs[b] @ c.T)          # [h, n] scores, materialised
        s = s - s.max(axis=1, keepdims=True)  # stable softmax over the tokens
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[b] = p @ c                        # weights times the latent rows
    return out
