"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare element by element."""

import numpy as np
import torch

import oracle
from transformer_attention_gqa_amd import binding, inputs

# max-abs-error bars, by the K/V element type the path reads
# (int8 / int4 caches take the quantized-cache bar: the oracle sees the exact
# dequantized values, and the kernel's arithmetic is that of the fp8 path with
# an exact code -> bf16 conversion)
TOL = {"f32": 1e-3, "bf16": 2e-2, "fp8": 5e-2, "int8": 5e-2, "int4": 5e-2}


def to_f64(t):
    """Stored tensor -> exact float64 numpy values (via the oracle's decoders)."""
    arr = inputs.stored_numpy(t)
    if arr.dtype == np.uint16:
        return oracle.bf16_bits_to_f64(arr)
    if arr.dtype == np.float32:
        return arr.astype(np.float64)
    raise TypeError(arr.dtype)


def dequantize(kind, codes, scales):
    """Stored codes and scales of a quantized cache -> float64 values (oracle decoders)."""
    c, sc = inputs.stored_numpy(codes), inputs.stored_numpy(scales)
    if kind == "fp8":
        return oracle.dequantize_fp8_cache(c, sc)
    return oracle.dequantize_int_cache(c, sc, 8 if kind == "int8" else 4)


def cache_f64(inp, b, g):
    """K/V slab (b, g) of a decode input as float64 values [S_max, d] each."""
    kind = inp.wl.kv_dtype
    if kind in inputs.QUANTIZED:
        return (dequantize(kind, inp.k[b, g], inp.k_scale[b, g]), dequantize(kind, inp.v[b, g], inp.v_scale[b, g]))
    return to_f64(inp.k[b, g]), to_f64(inp.v[b, g])


def run_decode(inp, n_split=0, out=None, workspace=None):
    wl = inp.wl
    return binding.attn_decode(inp.q, inp.k, inp.v, inp.seq_lens, wl.scale, out=out, k_scale=inp.k_scale,
                               v_scale=inp.v_scale, workspace=workspace, n_split=n_split)


def oracle_decode_pairs(inp, pairs):
    """Oracle outputs for the (b, j) pairs, building float64 slabs only as needed."""
    wl = inp.wl
    q = to_f64(inp.q)
    lens = inp.seq_lens.cpu().tolist()
    G = wl.G
    cache = {}
    rows = []
    for b, j in pairs:
        g = j // G
        if (b, g) not in cache:
            cache[(b, g)] = cache_f64(inp, b, g)
        k, v = cache[(b, g)]
        n = int(min(max(lens[b], 0), wl.S_max))
        rows.append(oracle.attend_one_row(q[b, j], k[:n], v[:n], wl.scale))
    return np.stack(rows)


def oracle_decode_full(inp):
    wl = inp.wl
    pairs = [(b, j) for b in range(wl.B) for j in range(wl.h_q)]
    return oracle_decode_pairs(inp, pairs).reshape(wl.B, wl.h_q, wl.d_h)


def max_err(gpu_out, ref):
    got = gpu_out.detach().float().cpu().double().numpy()
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


def prefill_f64(inp):
    return to_f64(inp.q), to_f64(inp.k), to_f64(inp.v)


def sample_pairs(B, h_q, n, seed):
    rng = np.random.default_rng(seed)
    pairs = {(b, int(rng.integers(h_q))) for b in range(B)}
    pairs |= {(0, 0), (B - 1, h_q - 1)}
    while len(pairs) < n:
        pairs.add((int(rng.integers(B)), int(rng.integers(h_q))))
    return sorted(pairs)


def sample_rows(B, S, h_q, n, seed):
    rng = np.random.default_rng(seed)
    trip = {(0, 0, 0), (B - 1, S - 1, h_q - 1), (0, S - 1, 0), (B - 1, 63, h_q // 2), (0, 64, 1 % h_q)}
    while len(trip) < n:
        trip.add((int(rng.integers(B)), int(rng.integers(S)), int(rng.integers(h_q))))
    return sorted(trip)


def sync():
    torch.cuda.synchronize()


def masked_prefill_values(inp):
    """q, k, v of a masked-prefill input as float64 values (fp8 codes through
    the oracle's per-head dequantiser)."""
    if inp.wl.dtype == "fp8":
        return tuple(oracle.dequantize_fp8_heads(inputs.stored_numpy(t), inputs.stored_numpy(d))
                     for t, d in ((inp.q, inp.q_descale), (inp.k, inp.k_descale), (inp.v, inp.v_descale)))
    return to_f64(inp.q), to_f64(inp.k), to_f64(inp.v)


def fp8_prefill_bound(q, k, v, scale, triples, causal, kv_lens, mask):
    """Per-element error bound of the fp8 prefill at the (b, r, j) rows, from
    the arithmetic: the weights are rounded to e4m3 (relative error <= 2^-4 in
    the normal range, absolute <= 2^-10 below 2^-6, in units where the largest
    weight is at least 1), the output to bf16 (2^-8 relative), plus 2^-7 for
    float32 accumulation.  With exact weights w_i = p_i / l:
        |dO_d| <= 2^-4 sum_i w_i |v_id| + 2^-10 sum_{p_i < 2^-6} |v_id| / l
                  + 2^-8 |O_d| + 2^-7."""
    out = []
    S_q, S_k = q.shape[1], k.shape[1]
    G = q.shape[2] // k.shape[2]
    for b, r, j in triples:
        vis = oracle.visible_keys(S_q, S_k, causal, None if kv_lens is None else kv_lens[b],
                                  None if mask is None else mask[b])[r]
        if not vis.any():
            out.append(np.full(q.shape[3], 2.0 ** -7))
            continue
        kk, vv = k[b, vis, j // G], v[b, vis, j // G]
        s = scale * (kk @ q[b, r, j])
        p = np.exp(s - s.max())
        lsum = p.sum()
        o = (p / lsum) @ vv
        small = p < 2.0 ** -6
        out.append(2.0 ** -4 * ((p / lsum) @ np.abs(vv)) + 2.0 ** -10 * np.abs(vv[small]).sum(0) / lsum
                   + 2.0 ** -8 * np.abs(o) + 2.0 ** -7)
    return np.stack(out)
