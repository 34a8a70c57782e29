"""Algorithmic work of the two calls, and the MI355X peaks they are priced against.

KV bytes ("Multi-query attention", section "Why this is a bandwidth argument,
not a FLOP argument"): one decode step reads

    KV bytes = 2 * b * L * n_kv * d_h * S * B

(b bytes per element, L layers, n_kv K/V heads, S context, B batch).  For
ragged batches the S * B product is the sum of the per-sequence lengths.  The
same page states that decode FLOPs are Theta(h * d_h * S) per step whatever
n_kv is: 2 * d_h multiply-adds per (query head, key) for the scores and
2 * d_h for the weighted sum of V, i.e. 4 * h_q * d_h * S flops per sequence.

Per-layer KV-cache size ("Evolution of AI Attention Mechanisms", section
"MHA Mathematical Formulation"): 2 * S * h * d_h * sizeof(dtype), with MQA
keeping one K/V head and GQA keeping g of them ("MQA (Multi-Query
Attention)" and "GQA (Grouped-Query Attention)" sections).

Latent attention ("Evolution of AI Attention Mechanisms", section
"Generation 3: MLA"): the cache keeps one latent vector of d_c values per
token instead of per-head keys and values; in the absorbed decode that row is
both key and value of every head, so a step reads it once:
2 * d_c * sum L bytes in bf16, for 4 * h_q * d_c flops per token.

Causal prefill FLOPs count only the key/query pairs the causal mask keeps:
S (S + 1) / 2 pairs per (batch, query head), 4 * d_h flops each.
"""

ELEMENT_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}
QUANTIZED = ("fp8", "int8", "int4")  # caches with per-(token, kv-head) float32 scales

# MI355X published peaks (dense).
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0, "f32": 157.3, "f64": 78.6}


def kv_cache_bytes(bytes_per_elem, layers, n_kv, d_h, S, B):
    """2 * b * L * n_kv * d_h * S * B."""
    return 2 * bytes_per_elem * layers * n_kv * d_h * S * B


def mha_kv_cache_bytes_per_layer(S, h, d_h, bytes_per_elem):
    """2 * S * h * d_h * sizeof(dtype) for one layer of a full-head cache."""
    return 2 * S * h * d_h * bytes_per_elem


def kv_fraction_of_mha(n_kv, h):
    """Cache size of an n_kv-head layer relative to the h-head MHA layer."""
    return n_kv / h


def decode_kv_bytes(kv_dtype, n_kv, d_h, seq_lens):
    """KV bytes one decode call must read (L = 1 layer, sum over ragged lengths)."""
    total = sum(int(x) for x in seq_lens)
    return int(kv_cache_bytes(ELEMENT_BYTES[kv_dtype], 1, n_kv, d_h, total, 1))


def decode_scale_bytes(kv_dtype, n_kv, seq_lens):
    """Quantized caches only: the float32 per-(token, kv-head) scales of K and V."""
    if kv_dtype not in QUANTIZED:
        return 0
    return 2 * 4 * n_kv * sum(int(x) for x in seq_lens)


def decode_flops(h_q, d_h, seq_lens):
    return 4 * h_q * d_h * sum(int(x) for x in seq_lens)


def mla_latent_bytes(d_c, seq_lens, bytes_per_elem=2):
    """Latent-cache bytes one absorbed decode step must read."""
    return int(bytes_per_elem * d_c * sum(int(x) for x in seq_lens))


def mla_flops(h_q, d_c, seq_lens):
    """Scores and weighted sum over the latent rows: 4 * h_q * d_c per token."""
    return 4 * h_q * d_c * sum(int(x) for x in seq_lens)


def prefill_causal_flops(B, S, h_q, d_h):
    return 4 * B * h_q * d_h * S * (S + 1) // 2


def visible_pairs(B, S_q, S_k, causal, kv_lens=None, mask=None):
    """Number of (batch, query row, key) pairs a general-mask prefill must
    compute: the causal rule (end-aligned), key lengths and dense mask
    combined.  Host-side accounting with torch (CPU)."""
    import torch
    r = torch.arange(S_q)[:, None]
    c = torch.arange(S_k)[None, :]
    vis = (c <= r + (S_k - S_q)) if causal else torch.ones(S_q, S_k, dtype=torch.bool)
    vis = vis[None].expand(B, S_q, S_k)
    if kv_lens is not None:
        vis = vis & (c[None] < torch.as_tensor(kv_lens).reshape(B, 1, 1).cpu())
    if mask is not None:
        vis = vis & (mask.cpu() != 0)
    return int(vis.sum())


def prefill_masked_flops(h_q, d_h, pairs):
    """4 * d_h flops per visible (query, key) pair and query head."""
    return 4 * h_q * d_h * int(pairs)


def prefill_io_bytes(B, S, h_q, n_kv, d_h, bytes_per_elem=2):
    """Compulsory HBM traffic of causal prefill: read Q, K, V once, write O once."""
    return bytes_per_elem * B * S * d_h * (2 * h_q + 2 * n_kv)
