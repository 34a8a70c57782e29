"""Seeded synthetic inputs for the decode and causal-prefill workloads.

This module only draws random numbers and stores them in the element formats
the library consumes.  It holds none of the attention arithmetic, and it is the
one piece the GPU path, the tests and the CPU oracle all share.

Recipe (every workload is synthetic):
  * values: standard normal float32 draws from a `torch.Generator` seeded per
    workload, drawn on the device that will hold the tensor;
  * bf16 tensors: round-to-nearest-even of those draws (torch's float32 ->
    bfloat16 cast);
  * fp8 KV cache: per (batch, kv-head, token) row, scale = max|x| / 448 in
    float32 (1.0 for an all-zero row), code = e4m3fn(clamp(x / scale, +-448))
    via torch's round-to-nearest-even cast -- the "quantization-aware scaling
    factors" reading of the KV-cache quantisation passage of the
    "Multi-Query Attention (MQA)" glossary page;
  * int8 / int4 KV caches (the same passage's INT8 / INT4 caches): the same
    per-row granularity, scale = max|x| / 127 (int8) or / 7 (int4), code =
    round-half-to-even(x / scale) clamped to the symmetric range; int4 codes
    are packed two per byte, element 2i in the low nibble;
  * ragged lengths: integers drawn uniformly from [lo, hi] inclusive from a CPU
    generator, so a workload's lengths are the same whichever device holds the
    tensors;
  * optional tail poisoning: cache rows at positions >= L_b set to NaN, so a
    kernel that reads past a sequence's end is caught.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

DTYPES = ("f32", "bf16", "fp8", "int8", "int4")
FP8_MAX = 448.0
INT8_MAX = 127  # symmetric codes: -127 .. 127
INT4_MAX = 7    # symmetric codes: -7 .. 7
QUANTIZED = ("fp8", "int8", "int4")


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    h_q: int
    n_kv: int
    d_h: int
    S_max: int
    q_dtype: str  # "f32" | "bf16"
    kv_dtype: str  # "f32" | "bf16" | "fp8" | "int8" | "int4"
    lens: Tuple[int, int]  # inclusive range of L_b; (S, S) for fixed length
    seed: int

    @property
    def G(self):
        return self.h_q // self.n_kv

    @property
    def scale(self):
        return 1.0 / float(self.d_h) ** 0.5


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    S: int
    h_q: int
    n_kv: int
    d_h: int
    seed: int
    dtype: str = "bf16"

    @property
    def G(self):
        return self.h_q // self.n_kv

    @property
    def scale(self):
        return 1.0 / float(self.d_h) ** 0.5


# The five synthetic workloads the library is measured on.
MQA_TINY_F32 = DecodeWorkload("mqa_decode_tiny_f32", B=2, h_q=8, n_kv=1, d_h=64, S_max=128,
                              q_dtype="f32", kv_dtype="f32", lens=(128, 128), seed=1)
GQA_RAGGED_BF16 = DecodeWorkload("gqa_decode_ragged_bf16", B=16, h_q=64, n_kv=8, d_h=128, S_max=4096,
                                 q_dtype="bf16", kv_dtype="bf16", lens=(1024, 4096), seed=2)
MQA_LONG_BF16 = DecodeWorkload("mqa_decode_long_bf16", B=64, h_q=32, n_kv=1, d_h=128, S_max=8192,
                               q_dtype="bf16", kv_dtype="bf16", lens=(8192, 8192), seed=3)
GQA_PREFILL_BF16 = PrefillWorkload("gqa_prefill_causal_bf16", B=4, S=4096, h_q=32, n_kv=8, d_h=128, seed=4)
GQA_FP8KV = DecodeWorkload("gqa_decode_fp8kv", B=32, h_q=64, n_kv=8, d_h=128, S_max=32768,
                           q_dtype="bf16", kv_dtype="fp8", lens=(32768, 32768), seed=5)

DECODE_WORKLOADS = {w.name: w for w in (MQA_TINY_F32, GQA_RAGGED_BF16, MQA_LONG_BF16, GQA_FP8KV)}

# The fp8-cache workload's shape with int8 and packed int4 caches.
GQA_INT8KV = DecodeWorkload("gqa_decode_int8kv", B=32, h_q=64, n_kv=8, d_h=128, S_max=32768,
                            q_dtype="bf16", kv_dtype="int8", lens=(32768, 32768), seed=6)
GQA_INT4KV = DecodeWorkload("gqa_decode_int4kv", B=32, h_q=64, n_kv=8, d_h=128, S_max=32768,
                            q_dtype="bf16", kv_dtype="int4", lens=(32768, 32768), seed=7)
QUANT_DECODE_WORKLOADS = {w.name: w for w in (GQA_INT8KV, GQA_INT4KV)}
PREFILL_WORKLOADS = {GQA_PREFILL_BF16.name: GQA_PREFILL_BF16}


@dataclass(frozen=True)
class MlaWorkload:
    """Absorbed multi-head latent attention decode: h query heads (already
    moved into the latent space) over one latent cache row of d_c values per
    token, which serves as both keys and values."""
    name: str
    B: int
    h_q: int
    d_c: int
    S_max: int
    lens: Tuple[int, int]
    seed: int

    @property
    def scale(self):
        return 1.0 / float(self.d_c) ** 0.5  # the latent dimension, as in the absorbed form's code


# 32 heads over a 512-value latent (the MLA module's defaults), ragged lengths.
MLA_DECODE_BF16 = MlaWorkload("mla_decode_bf16", B=32, h_q=32, d_c=512, S_max=16384, lens=(4096, 16384), seed=8)
MLA_WORKLOADS = {MLA_DECODE_BF16.name: MLA_DECODE_BF16}


@dataclass
class MlaInputs:
    wl: MlaWorkload
    q: torch.Tensor         # [B, h_q, d_c] bf16 (absorbed queries)
    c_kv: torch.Tensor      # [B, S_max, d_c] bf16 latent cache
    seq_lens: torch.Tensor  # [B] int32


def make_mla_inputs(wl, device="cpu", seq_lens=None, poison_tail=False, seed=None):
    seed = wl.seed if seed is None else seed
    g = _gen(device, seed)
    if seq_lens is None:
        lens = draw_lengths(wl.B, wl.lens[0], wl.lens[1], seed)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).reshape(wl.B)
    q = torch.randn((wl.B, wl.h_q, wl.d_c), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((wl.B, wl.S_max, wl.d_c), dtype=torch.bfloat16, device=device)
    for b in range(wl.B):
        c[b] = torch.randn((wl.S_max, wl.d_c), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    if poison_tail:
        for b in range(wl.B):
            n = int(min(max(int(lens[b]), 0), wl.S_max))
            c[b, n:] = float("nan")
    return MlaInputs(wl, q, c, lens.to(device))


@dataclass(frozen=True)
class PagedDecodeWorkload:
    """A decode workload whose cache lives in a pool of fixed-size pages."""
    name: str
    base: DecodeWorkload
    page_size: int


# The ragged GQA decode with its cache in 64-token pages scattered over the pool.
GQA_RAGGED_BF16_PAGED64 = PagedDecodeWorkload("gqa_decode_ragged_bf16_paged64", GQA_RAGGED_BF16, 64)
PAGED_WORKLOADS = {GQA_RAGGED_BF16_PAGED64.name: GQA_RAGGED_BF16_PAGED64}


def _torch_dtype(tag):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[tag]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_lengths(B, lo, hi, seed):
    """Ragged lengths, uniform integers in [lo, hi], from a CPU generator."""
    g = _gen("cpu", seed * 7919 + 17)
    if lo == hi:
        return torch.full((B,), lo, dtype=torch.int32)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def quantize_e4m3_rows(x):
    """float32 [..., d] -> (uint8 codes [..., d], float32 scales [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).float()
    y = (x / scale[..., None]).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def quantize_int_rows(x, qmax):
    """float32 [..., d] -> (int8 codes [..., d] in [-qmax, qmax], float32 scales
    [...]): symmetric absmax per row, round half to even."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / qmax, torch.ones_like(amax)).float()
    codes = torch.round(x / scale[..., None]).clamp(-qmax, qmax).to(torch.int8)
    return codes, scale


def pack_int4(codes):
    """int8 codes [..., d] in [-8, 7] -> uint8 [..., d/2]: element 2i in the low
    nibble of byte i, element 2i + 1 in the high nibble (two's complement)."""
    c = codes.to(torch.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).to(torch.uint8)


def quantize_rows(x, kind):
    """float32 [..., d] -> (stored codes, float32 scales) for a quantized cache kind."""
    if kind == "fp8":
        return quantize_e4m3_rows(x)
    if kind == "int8":
        return quantize_int_rows(x, INT8_MAX)
    if kind == "int4":
        codes, scale = quantize_int_rows(x, INT4_MAX)
        return pack_int4(codes), scale
    raise ValueError(kind)


def code_shape(kind, shape):
    """Shape and dtype of the stored codes of a quantized cache of `shape` [..., d]."""
    if kind == "int4":
        return tuple(shape[:-1]) + (shape[-1] // 2,), torch.uint8
    return tuple(shape), (torch.int8 if kind == "int8" else torch.uint8)


# Code patterns that fill cache rows which must never be read: NaN for fp8,
# the largest codes for the integer kinds (their scales are set to NaN).
POISON_CODE = {"fp8": 0x7F, "int8": 0x7F, "int4": 0x77}


@dataclass
class DecodeInputs:
    wl: DecodeWorkload
    q: torch.Tensor  # [B, h_q, d] f32/bf16
    k: torch.Tensor  # [B, n_kv, S_max, d] f32/bf16, uint8 fp8 / int8 codes, or [.., d/2] packed int4
    v: torch.Tensor
    seq_lens: torch.Tensor  # [B] int32, same device
    k_scale: Optional[torch.Tensor] = None  # [B, n_kv, S_max] f32 (quantized caches only)
    v_scale: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)


def make_decode_inputs(wl, device="cpu", seq_lens=None, poison_tail=False, seed=None):
    """Draw q, K/V cache (and scales of a quantized cache) for a decode workload.

    seq_lens overrides the workload's length rule (list/tensor of B ints).
    """
    seed = wl.seed if seed is None else seed
    g = _gen(device, seed)
    B, h_q, n_kv, d, S = wl.B, wl.h_q, wl.n_kv, wl.d_h, wl.S_max
    if seq_lens is None:
        lens = draw_lengths(B, wl.lens[0], wl.lens[1], seed)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).reshape(B)
    q = torch.randn((B, h_q, d), generator=g, device=device, dtype=torch.float32).to(_torch_dtype(wl.q_dtype))
    if wl.kv_dtype in QUANTIZED:
        shape, cdt = code_shape(wl.kv_dtype, (B, n_kv, S, d))
        k = torch.empty(shape, dtype=cdt, device=device)
        v = torch.empty(shape, dtype=cdt, device=device)
        ks = torch.empty((B, n_kv, S), dtype=torch.float32, device=device)
        vs = torch.empty((B, n_kv, S), dtype=torch.float32, device=device)
        for b in range(B):  # per batch entry to bound temporary memory
            xk = torch.randn((n_kv, S, d), generator=g, device=device, dtype=torch.float32)
            k[b], ks[b] = quantize_rows(xk, wl.kv_dtype)
            del xk
            xv = torch.randn((n_kv, S, d), generator=g, device=device, dtype=torch.float32)
            v[b], vs[b] = quantize_rows(xv, wl.kv_dtype)
            del xv
        inp = DecodeInputs(wl, q, k, v, lens.to(device), ks, vs)
    else:
        dt = _torch_dtype(wl.kv_dtype)
        k = torch.empty((B, n_kv, S, d), dtype=dt, device=device)
        v = torch.empty((B, n_kv, S, d), dtype=dt, device=device)
        for b in range(B):
            k[b] = torch.randn((n_kv, S, d), generator=g, device=device, dtype=torch.float32).to(dt)
            v[b] = torch.randn((n_kv, S, d), generator=g, device=device, dtype=torch.float32).to(dt)
        inp = DecodeInputs(wl, q, k, v, lens.to(device))
    if poison_tail:
        poison_cache_tails(inp)
    return inp


def poison_cache_tails(inp):
    """Fill cache rows at positions >= L_b with NaN (quantized caches: the
    POISON_CODE pattern and NaN scales)."""
    S = inp.wl.S_max
    for b in range(inp.wl.B):
        n = int(min(max(int(inp.seq_lens[b]), 0), S))
        if n >= S:
            continue
        if inp.wl.kv_dtype in QUANTIZED:
            pc = POISON_CODE[inp.wl.kv_dtype]
            inp.k[b, :, n:, :] = _as_code(pc, inp.k.dtype)
            inp.v[b, :, n:, :] = _as_code(pc, inp.v.dtype)
            inp.k_scale[b, :, n:] = float("nan")
            inp.v_scale[b, :, n:] = float("nan")
        else:
            inp.k[b, :, n:, :] = float("nan")
            inp.v[b, :, n:, :] = float("nan")


def _as_code(byte, dtype):
    """A byte pattern as a fill value of a code tensor's dtype."""
    return byte - 256 if dtype == torch.int8 and byte >= 128 else byte


@dataclass
class PagedDecodeInputs:
    """A decode workload's cache cut into pages and scattered over a pool."""
    base: DecodeInputs                 # q, seq_lens and the contiguous cache the pages were cut from
    page_size: int
    k_pages: torch.Tensor              # [num_pages, n_kv, page_size, d]
    v_pages: torch.Tensor
    k_scale_pages: Optional[torch.Tensor]  # [num_pages, n_kv, page_size] float32 (quantized caches only)
    v_scale_pages: Optional[torch.Tensor]
    block_table: torch.Tensor          # [B, max_pages] int32

    @property
    def num_pages(self):
        return self.k_pages.shape[0]


def make_paged_decode_inputs(wl, page_size, device="cpu", seq_lens=None, poison_tail=False, seed=None,
                             spare_pages=3, junk_unused_entries=False, keep_base=True):
    """Draw a decode workload (as make_decode_inputs) and scatter its cache into
    a pool of B * S_max / page_size + spare_pages pages in a seeded random
    order.  Spare pages hold NaN (quantized caches: POISON_CODE and NaN
    scales).  With
    junk_unused_entries, block-table entries past a sequence's last page are
    set to -1 (they must never be read)."""
    if wl.S_max % page_size:
        raise ValueError("S_max must be a multiple of page_size")
    seed = wl.seed if seed is None else seed
    base = make_decode_inputs(wl, device=device, seq_lens=seq_lens, poison_tail=poison_tail, seed=seed)
    B, n_kv, d, S = wl.B, wl.n_kv, wl.d_h, wl.S_max
    max_pages = S // page_size
    num_pages = B * max_pages + spare_pages
    g = torch.Generator(device="cpu").manual_seed(seed * 104729 + page_size)
    perm = torch.randperm(num_pages, generator=g)[:B * max_pages].to(torch.int32)
    table = perm.reshape(B, max_pages).clone()
    quant = wl.kv_dtype in QUANTIZED
    dc = base.k.shape[-1]  # stored elements per row (d / 2 for packed int4)
    kp = torch.empty((num_pages, n_kv, page_size, dc), dtype=base.k.dtype, device=device)
    vp = torch.empty_like(kp)
    fill = _as_code(POISON_CODE[wl.kv_dtype], kp.dtype) if quant else float("nan")
    kp.fill_(fill)
    vp.fill_(fill)
    ksp = vsp = None
    if quant:
        ksp = torch.full((num_pages, n_kv, page_size), float("nan"), dtype=torch.float32, device=device)
        vsp = torch.full_like(ksp, float("nan"))
    idx = table.to(device=device, dtype=torch.long)
    for b in range(B):
        kp[idx[b]] = base.k[b].reshape(n_kv, max_pages, page_size, dc).transpose(0, 1)
        vp[idx[b]] = base.v[b].reshape(n_kv, max_pages, page_size, dc).transpose(0, 1)
        if quant:
            ksp[idx[b]] = base.k_scale[b].reshape(n_kv, max_pages, page_size).transpose(0, 1)
            vsp[idx[b]] = base.v_scale[b].reshape(n_kv, max_pages, page_size).transpose(0, 1)
    if junk_unused_entries:
        lens = base.seq_lens.cpu().tolist()
        for b in range(B):
            used = (min(max(int(lens[b]), 0), S) + page_size - 1) // page_size
            table[b, used:] = -1
    if not keep_base:  # drop the contiguous cache (q and seq_lens stay)
        base = DecodeInputs(wl, base.q, base.k[:0], base.v[:0], base.seq_lens)
    return PagedDecodeInputs(base, page_size, kp, vp, ksp, vsp, table.to(device))


@dataclass
class PrefillInputs:
    wl: PrefillWorkload
    q: torch.Tensor  # [B, S, h_q, d] bf16
    k: torch.Tensor  # [B, S, n_kv, d] bf16
    v: torch.Tensor


def make_prefill_inputs(wl, device="cpu", seed=None):
    seed = wl.seed if seed is None else seed
    g = _gen(device, seed)
    dt = _torch_dtype(wl.dtype)
    q = torch.randn((wl.B, wl.S, wl.h_q, wl.d_h), generator=g, device=device, dtype=torch.float32).to(dt)
    k = torch.randn((wl.B, wl.S, wl.n_kv, wl.d_h), generator=g, device=device, dtype=torch.float32).to(dt)
    v = torch.randn((wl.B, wl.S, wl.n_kv, wl.d_h), generator=g, device=device, dtype=torch.float32).to(dt)
    return PrefillInputs(wl, q, k, v)


@dataclass(frozen=True)
class MaskedPrefillWorkload:
    """Prefill with general masks: S_q queries over S_k keys (cached keys come
    first), the causal rule optional, ragged key lengths (padding) and a dense
    mask shared by all heads.

    mask kinds: None; "random" (each byte 1 with probability 3/4, seeded);
    "docs" (packed documents: consecutive spans of random length in
    doc_lens, a row sees only keys of its own span)."""
    name: str
    B: int
    S_q: int
    S_k: int
    h_q: int
    n_kv: int
    d_h: int
    causal: bool
    seed: int
    kv_lens: Optional[Tuple[int, int]] = None
    mask: Optional[str] = None
    doc_lens: Tuple[int, int] = (512, 2048)
    dtype: str = "bf16"  # or "fp8": e4m3 codes with one descale factor per (batch, head)

    @property
    def G(self):
        return self.h_q // self.n_kv

    @property
    def scale(self):
        return 1.0 / float(self.d_h) ** 0.5


# c4's shape without the causal rule, padded to ragged key lengths
GQA_PREFILL_PADDED = MaskedPrefillWorkload("gqa_prefill_padded_bf16", B=4, S_q=4096, S_k=4096, h_q=32, n_kv=8,
                                           d_h=128, causal=False, seed=9, kv_lens=(2048, 4096))
# c4 with packed documents of 512..2048 tokens (dense block-diagonal mask on top of the causal rule)
GQA_PREFILL_DOCS = MaskedPrefillWorkload("gqa_prefill_docs_bf16", B=4, S_q=4096, S_k=4096, h_q=32, n_kv=8,
                                         d_h=128, causal=True, seed=10, mask="docs")
# c4 (causal, B=4, S=4096, 32 query / 8 K/V heads, d=128) on fp8 codes
GQA_PREFILL_FP8 = MaskedPrefillWorkload("gqa_prefill_causal_fp8", B=4, S_q=4096, S_k=4096, h_q=32, n_kv=8, d_h=128,
                                        causal=True, seed=11, dtype="fp8")
MASKED_PREFILL_WORKLOADS = {w.name: w for w in (GQA_PREFILL_PADDED, GQA_PREFILL_DOCS, GQA_PREFILL_FP8)}


@dataclass
class MaskedPrefillInputs:
    wl: MaskedPrefillWorkload
    q: torch.Tensor                  # [B, S_q, h_q, d] bf16 (fp8: uint8 e4m3 codes)
    k: torch.Tensor                  # [B, S_k, n_kv, d] bf16 (fp8: uint8 codes)
    v: torch.Tensor
    kv_lens: Optional[torch.Tensor]  # [B] int32
    mask: Optional[torch.Tensor]     # [B, S_q, S_k] uint8
    q_descale: Optional[torch.Tensor] = None  # [B, h_q] float32 (fp8 only)
    k_descale: Optional[torch.Tensor] = None  # [B, n_kv] float32
    v_descale: Optional[torch.Tensor] = None


def quantize_e4m3_heads(x):
    """float32 [B, S, H, d] -> (uint8 e4m3 codes, float32 descale [B, H]): one
    absmax factor per (batch, head), descale = amax / 448 (amax = 0 -> 1),
    code = RNE(x / descale)."""
    x = x.float()
    amax = x.abs().amax(dim=(1, 3))
    descale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).float()
    y = (x / descale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), descale


def draw_mask(kind, B, S_q, S_k, seed, doc_lens=(512, 2048)):
    """uint8 [B, S_q, S_k] from a CPU generator (1 = visible)."""
    g = _gen("cpu", seed * 7919 + 29)
    if kind == "random":
        return (torch.rand((B, S_q, S_k), generator=g) < 0.75).to(torch.uint8)
    if kind == "docs":
        if S_q != S_k:
            raise ValueError("document masks need S_q == S_k")
        doc = torch.empty((B, S_k), dtype=torch.int64)
        for b in range(B):
            pos, i = 0, 0
            while pos < S_k:
                n = int(torch.randint(doc_lens[0], doc_lens[1] + 1, (1,), generator=g))
                doc[b, pos:pos + n] = i
                pos, i = pos + n, i + 1
        return (doc[:, :, None] == doc[:, None, :]).to(torch.uint8)
    raise ValueError(f"unknown mask kind {kind}")


def make_masked_prefill_inputs(wl, device="cpu", kv_lens=None, mask=None, poison_padding=False, seed=None):
    """Seeded q/k/v (N(0,1) -> bf16), key lengths (given, drawn from wl.kv_lens, or
    none) and a mask (given, drawn by wl.mask's kind, or none).  poison_padding
    fills key/value rows at or past each key length with NaN."""
    seed = wl.seed if seed is None else seed
    g = _gen(device, seed)
    q = torch.randn((wl.B, wl.S_q, wl.h_q, wl.d_h), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((wl.B, wl.S_k, wl.n_kv, wl.d_h), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((wl.B, wl.S_k, wl.n_kv, wl.d_h), generator=g, device=device, dtype=torch.float32)
    descales = (None, None, None)
    if wl.dtype == "fp8":
        (q, dq), (k, dk), (v, dv) = quantize_e4m3_heads(q), quantize_e4m3_heads(k), quantize_e4m3_heads(v)
        descales = (dq, dk, dv)
    else:
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    if kv_lens is None and wl.kv_lens is not None:
        kv_lens = draw_lengths(wl.B, wl.kv_lens[0], wl.kv_lens[1], seed)
    if kv_lens is not None:
        kv_lens = torch.as_tensor(kv_lens, dtype=torch.int32).reshape(wl.B)
        if poison_padding:
            for b in range(wl.B):
                n = int(min(max(int(kv_lens[b]), 0), wl.S_k))
                if wl.dtype == "fp8":
                    k[b, n:] = POISON_CODE["fp8"]
                    v[b, n:] = POISON_CODE["fp8"]
                else:
                    k[b, n:] = float("nan")
                    v[b, n:] = float("nan")
        kv_lens = kv_lens.to(device)
    if mask is None and wl.mask is not None:
        mask = draw_mask(wl.mask, wl.B, wl.S_q, wl.S_k, seed, wl.doc_lens)
    if mask is not None:
        mask = torch.as_tensor(mask).to(torch.uint8).contiguous().to(device)
    return MaskedPrefillInputs(wl, q, k, v, kv_lens, mask, *descales)


def stored_numpy(t):
    """A tensor's stored encoding as a numpy array: bf16 -> uint16 bit patterns,
    fp8 and packed int4 codes stay uint8, int8 codes int8, float32/int32 as is.
    (Bit views, no arithmetic.)"""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
