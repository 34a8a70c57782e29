"""Decode over a paged KV cache, float64 -- the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ("Multi-Query Attention (MQA)" glossary, section
"PagedAttention"): the cache of every sequence is cut into fixed-size pages
that may lie anywhere in memory.  Reading taken here (the plainest one the
section supports): a pool of pages [num_pages, n_kv, page_size, d], page p
holding page_size consecutive tokens of all K/V heads of one sequence, and a
block table [B, max_pages] whose entry (b, i) names the page that holds
tokens i*page_size .. (i+1)*page_size - 1 of sequence b.  The attention itself
is the decode step of `attention.decode` over the L_b logical tokens.

The oracle first gathers each sequence's logical cache through its block
table (the definition of the paging), then runs the plain decode.
"""

import numpy as np

from .attention import decode


def gather_logical_cache(pages, block_table, seq_lens, page_size):
    """pages [num_pages, n_kv, page_size, d] -> logical cache [B, n_kv, S, d]
    with S = max_pages * page_size; positions at or beyond L_b are zero (they
    are never read by the decode)."""
    pages = np.asarray(pages)
    block_table = np.asarray(block_table)
    num_pages, n_kv, ps, d = pages.shape
    if ps != page_size:
        raise ValueError(f"pages hold {ps} tokens, page_size is {page_size}")
    B, max_pages = block_table.shape
    s_cap = max_pages * page_size
    out = np.zeros((B, n_kv, s_cap, d), dtype=pages.dtype)
    for b in range(B):
        n = int(min(max(int(seq_lens[b]), 0), s_cap))
        for i in range((n + page_size - 1) // page_size):
            p = int(block_table[b, i])
            if not 0 <= p < num_pages:
                raise ValueError(f"block_table[{b}, {i}] = {p} is not a page of the pool")
            out[b, :, i * page_size:(i + 1) * page_size] = pages[p]
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, page_size):
    """One decode step over a paged cache -> [B, h_q, d] float64.

    seq_lens values are clamped to [0, max_pages * page_size]."""
    k = gather_logical_cache(k_pages, block_table, seq_lens, page_size)
    v = gather_logical_cache(v_pages, block_table, seq_lens, page_size)
    return decode(q, k, v, seq_lens, scale)
