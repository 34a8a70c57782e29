"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from transformer_attention_gqa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

ALIGNED = 0x10000          # fake, never dereferenced: validation fails first
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+|gqa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def dd(B=2, h_q=8, n_kv=2, S=64, d=128, qt=1, kt=1, ns=0, flags=0):
    return binding.gqa_decode_desc(B, h_q, n_kv, S, d, qt, kt, ns, flags)


def call_decode(lib, desc, q=ALIGNED, k=ALIGNED, v=ALIGNED, ks=None, vs=None, lens=ALIGNED, out=ALIGNED,
                ws=ALIGNED, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(ctypes.byref(desc)) if desc is not None else 0
    p = ctypes.byref(desc) if desc is not None else None
    return lib.attn_decode(p, q, k, v, ks, vs, lens, 1.0, out, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), 2), (dict(h_q=-1), 2), (dict(n_kv=0), 2), (dict(S=0), 2), (dict(d=96), 2), (dict(d=256), 2),
    (dict(h_q=12, n_kv=8), 2), (dict(ns=-1), 2),
    (dict(qt=0, kt=1), 3), (dict(qt=1, kt=0), 3), (dict(qt=0, kt=2), 3), (dict(qt=2, kt=2), 3), (dict(qt=7), 3),
])
def test_decode_descriptor_errors(lib, bad, code):
    desc = dd(**bad)
    assert call_decode(lib, desc) == code
    assert lib.attn_decode_workspace_bytes(ctypes.byref(desc)) == 0
    assert lib.attn_decode_num_splits(ctypes.byref(desc)) == -1


def test_decode_pointer_errors(lib):
    assert call_decode(lib, None) == 1
    assert call_decode(lib, dd(), q=None) == 1
    assert call_decode(lib, dd(), lens=None) == 1
    assert call_decode(lib, dd(), out=None) == 1
    assert call_decode(lib, dd(kt=2), ks=None, vs=ALIGNED) == 1   # fp8 cache needs scales
    assert call_decode(lib, dd(), k=MISALIGNED) == 4
    assert call_decode(lib, dd(), out=MISALIGNED) == 4
    assert call_decode(lib, dd(), lens=ALIGNED + 2) == 4
    assert call_decode(lib, dd(kt=2), ks=MISALIGNED, vs=ALIGNED) == 4


def test_decode_workspace_errors(lib):
    desc = dd()
    need = lib.attn_decode_workspace_bytes(ctypes.byref(desc))
    assert need > 0
    assert call_decode(lib, desc, ws=None) == 5
    assert call_decode(lib, desc, ws_bytes=need - 1) == 5
    assert call_decode(lib, desc, ws=MISALIGNED) == 4
    assert lib.attn_decode_partials(ctypes.byref(desc), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, 1.0,
                                    ALIGNED, need - 4, None) == 5
    assert lib.attn_decode_combine(ctypes.byref(desc), ALIGNED, ALIGNED, need - 4, ALIGNED, None) == 5
    assert lib.attn_decode_combine(ctypes.byref(desc), ALIGNED, ALIGNED, need, None, None) == 1


def test_split_plan_is_deterministic_and_honours_requests(lib):
    base = dd(B=16, h_q=64, n_kv=8, S=4096)
    a = lib.attn_decode_workspace_bytes(ctypes.byref(base))
    assert a == lib.attn_decode_workspace_bytes(ctypes.byref(base))
    # one workgroup per compute unit of the current device; with no device to
    # query (this host), the 256 of a whole MI355X
    assert lib.attn_decode_num_splits(ctypes.byref(base)) == 256
    n_slabs = 16 * 8  # G = 8 <= 16: one head chunk per K/V head
    max_tiles = n_slabs * (4096 // 32)
    for req in (1, 2, 7, 128, 100000):
        desc = dd(B=16, h_q=64, n_kv=8, S=4096, ns=req)
        ns = lib.attn_decode_num_splits(ctypes.byref(desc))
        assert ns == min(req, max_tiles, 65536)
        # one partial slot per (workgroup, slab) pair a balanced range can touch
        ws = lib.attn_decode_workspace_bytes(ctypes.byref(desc))
        assert ws >= (ns + n_slabs) * 16 * (128 + 2) * 4
    # the float32 path plans in 64-token tiles, the matrix-core paths in 32-token tiles
    tiny = dd(B=2, h_q=8, n_kv=1, S=128, d=64, qt=0, kt=0)
    assert lib.attn_decode_num_splits(ctypes.byref(tiny)) == 2 * 2
    big_g = dd(B=2, h_q=64, n_kv=1, S=64, qt=1, kt=1)  # G = 64 -> two chunks of 32 heads
    assert lib.attn_decode_num_splits(ctypes.byref(big_g)) == 2 * 2 * 2


def test_prefill_errors(lib):
    def pd(B=1, S=16, h_q=4, n_kv=2, d=128, dt=1):
        return binding.gqa_prefill_desc(B, S, h_q, n_kv, d, dt)

    def call(desc, q=ALIGNED, k=ALIGNED, v=ALIGNED, out=ALIGNED):
        return lib.attn_prefill_causal(ctypes.byref(desc) if desc is not None else None, q, k, v, 0.1, out, None)

    assert call(None) == 1
    assert call(pd(S=0)) == 2
    assert call(pd(h_q=6, n_kv=4)) == 2
    assert call(pd(d=80)) == 2
    assert call(pd(dt=0)) == 3
    assert call(pd(dt=2)) == 3
    assert call(pd(), v=None) == 1
    assert call(pd(), out=MISALIGNED) == 4


@pytest.mark.parametrize("scale", [-0.125, -1e-30, float("inf"), float("-inf"), float("nan")])
def test_scale_must_be_finite_and_non_negative(lib, scale):
    desc = dd()
    need = lib.attn_decode_workspace_bytes(ctypes.byref(desc))
    assert lib.attn_decode(ctypes.byref(desc), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, scale, ALIGNED,
                           ALIGNED, need, None) == 7
    assert lib.attn_decode_partials(ctypes.byref(desc), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, scale,
                                    ALIGNED, need, None) == 7
    pdesc = binding.gqa_prefill_desc(1, 16, 4, 2, 128, 1)
    assert lib.attn_prefill_causal(ctypes.byref(pdesc), ALIGNED, ALIGNED, ALIGNED, scale, ALIGNED, None) == 7


def test_status_strings(lib):
    for code, name in binding.STATUS.items():
        assert lib.gqa_status_string(code).decode().startswith(name)
    assert lib.gqa_last_hip_error().decode() == ""


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library.__wrapped__(str(tmp_path / "nope.so")) if hasattr(binding.load_library, "__wrapped__") \
            else _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = binding._lib
    binding._lib = None
    try:
        return binding.load_library(path)
    finally:
        binding._lib = saved


def pgd(B=2, h_q=8, n_kv=2, d=128, qt=1, kt=1, ps=64, pages=10, maxp=4, ns=0):
    return binding.gqa_paged_desc(B, h_q, n_kv, d, qt, kt, ps, pages, maxp, ns)


def call_paged(lib, desc, q=ALIGNED, kp=ALIGNED, vp=ALIGNED, ks=None, vs=None, table=ALIGNED, lens=ALIGNED,
               out=ALIGNED, ws=ALIGNED, ws_bytes=None, scale=1.0):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_paged_workspace_bytes(ctypes.byref(desc)) if desc is not None else 0
    p = ctypes.byref(desc) if desc is not None else None
    return lib.attn_decode_paged(p, q, kp, vp, ks, vs, table, lens, scale, out, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(ps=16), 2), (dict(ps=48), 2), (dict(ps=0), 2), (dict(pages=0), 2), (dict(maxp=0), 2),
    (dict(ps=1 << 21), 2), (dict(B=0), 2), (dict(h_q=12, n_kv=8), 2), (dict(d=96), 2), (dict(ns=-1), 2),
    (dict(qt=0, kt=1), 3), (dict(qt=1, kt=0), 3),
])
def test_paged_descriptor_errors(lib, bad, code):
    desc = pgd(**bad)
    assert call_paged(lib, desc) == code
    assert lib.attn_decode_paged_workspace_bytes(ctypes.byref(desc)) == 0
    assert lib.attn_decode_paged_num_splits(ctypes.byref(desc)) == -1


def test_paged_plan_matches_the_contiguous_plan(lib):
    """A paged call plans like a contiguous one with S_max = max_pages * page_size."""
    for ps, maxp, ns in ((32, 4, 0), (64, 64, 0), (128, 32, 7), (256, 16, 10 ** 6)):
        p = pgd(B=16, h_q=64, n_kv=8, ps=ps, pages=999, maxp=maxp, ns=ns)
        c = dd(B=16, h_q=64, n_kv=8, S=ps * maxp, ns=ns)
        assert lib.attn_decode_paged_num_splits(ctypes.byref(p)) == lib.attn_decode_num_splits(ctypes.byref(c))
        assert lib.attn_decode_paged_workspace_bytes(ctypes.byref(p)) == \
            lib.attn_decode_workspace_bytes(ctypes.byref(c))


def test_paged_pointer_and_value_errors(lib):
    desc = pgd()
    assert call_paged(lib, None) == 1
    assert call_paged(lib, desc, table=None) == 1
    assert call_paged(lib, desc, kp=None) == 1
    assert call_paged(lib, desc, out=None) == 1
    assert call_paged(lib, pgd(kt=2), ks=None, vs=None) == 1
    assert call_paged(lib, desc, table=ALIGNED + 2) == 4
    assert call_paged(lib, desc, vp=MISALIGNED) == 4
    assert call_paged(lib, desc, ws_bytes=16) == 5
    assert call_paged(lib, desc, scale=-1.0) == 7


@pytest.mark.parametrize("kt", [3, 4])
def test_int_caches_are_accepted_with_scales(lib, kt):
    """INT8 (3) and INT4 (4) caches take bf16 Q and per-row scales, like FP8."""
    desc = dd(kt=kt)
    assert lib.attn_decode_num_splits(ctypes.byref(desc)) > 0
    ws = lib.attn_decode_workspace_bytes(ctypes.byref(desc))
    assert ws > 0
    if kt == 3:  # int8 shares fp8's plan; int4 schedules 64-token tiles (fewer ranges on a short cache)
        assert ws == lib.attn_decode_workspace_bytes(ctypes.byref(dd(kt=2)))
    assert call_decode(lib, desc, ks=None, vs=ALIGNED) == 1
    assert call_decode(lib, desc, ks=ALIGNED, vs=MISALIGNED) == 4
    assert call_decode(lib, dd(qt=0, kt=kt)) == 3
    assert call_paged(lib, pgd(kt=kt), ks=None, vs=None) == 1


def mld(B=2, h_q=32, S=64, d_c=512, dt=1, ns=0):
    return binding.gqa_mla_desc(B, h_q, S, d_c, dt, ns)


def call_mla(lib, desc, q=ALIGNED, c=ALIGNED, lens=ALIGNED, out=ALIGNED, ws=ALIGNED, ws_bytes=None, scale=1.0):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_mla_workspace_bytes(ctypes.byref(desc)) if desc is not None else 0
    p = ctypes.byref(desc) if desc is not None else None
    return lib.attn_decode_mla(p, q, c, lens, scale, out, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), 2), (dict(h_q=0), 2), (dict(S=-3), 2), (dict(d_c=128), 2), (dict(d_c=576), 2), (dict(ns=-1), 2),
    (dict(dt=0), 3), (dict(dt=2), 3),
])
def test_mla_descriptor_errors(lib, bad, code):
    desc = mld(**bad)
    assert call_mla(lib, desc) == code
    assert lib.attn_decode_mla_workspace_bytes(ctypes.byref(desc)) == 0
    assert lib.attn_decode_mla_num_splits(ctypes.byref(desc)) == -1


def test_mla_pointer_and_value_errors(lib):
    desc = mld()
    assert call_mla(lib, None) == 1
    assert call_mla(lib, desc, q=None) == 1
    assert call_mla(lib, desc, c=None) == 1
    assert call_mla(lib, desc, lens=None) == 1
    assert call_mla(lib, desc, out=None) == 1
    assert call_mla(lib, desc, c=MISALIGNED) == 4
    assert call_mla(lib, desc, lens=ALIGNED + 2) == 4
    assert call_mla(lib, desc, ws=None) == 5
    assert call_mla(lib, desc, ws_bytes=16) == 5
    assert call_mla(lib, desc, scale=float("inf")) == 7


def test_mla_plan(lib):
    """Head chunks of up to 64 heads; the workspace holds (W + slabs) rows of
    d_c partial values per chunk head plus (m, l), like the decode workspace."""
    for B, h_q, S, d_c, ns in ((32, 32, 16384, 512, 0), (4, 16, 100, 256, 0), (3, 96, 1000, 512, 5),
                               (1, 128, 64, 512, 10 ** 6)):
        desc = mld(B=B, h_q=h_q, S=S, d_c=d_c, ns=ns)
        hpc = 64 if h_q > 32 else 32
        slabs = B * -(-h_q // hpc)
        W = min(ns or 256, slabs * -(-S // 32))
        assert lib.attn_decode_mla_num_splits(ctypes.byref(desc)) == W
        rows = (W + slabs) * hpc
        o_bytes = -(-rows * d_c * 4 // 256) * 256
        assert lib.attn_decode_mla_workspace_bytes(ctypes.byref(desc)) == o_bytes + rows * 8


def ad(B=2, S_q=64, S_k=64, h_q=8, n_kv=2, d=128, dt=1, causal=1):
    return binding.gqa_attn_desc(B, S_q, S_k, h_q, n_kv, d, dt, causal)


def call_prefill(lib, desc, q=ALIGNED, k=ALIGNED, v=ALIGNED, qd=None, kd=None, vd=None, lens=None, mask=None,
                 out=ALIGNED, scale=1.0):
    p = ctypes.byref(desc) if desc is not None else None
    return lib.attn_prefill(p, q, k, v, qd, kd, vd, lens, mask, scale, out, None)


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), 2), (dict(S_q=0), 2), (dict(S_k=-1), 2), (dict(h_q=12, n_kv=8), 2), (dict(d=96), 2),
    (dict(causal=2), 2), (dict(dt=0), 3), (dict(dt=3), 3), (dict(dt=2, d=96), 2),
])
def test_prefill_descriptor_errors(lib, bad, code):
    assert call_prefill(lib, ad(**bad)) == code


def test_prefill_fp8_needs_aligned_descale_factors(lib):
    """fp8 operands take three descale arrays; bf16 operands take none."""
    assert call_prefill(lib, ad(dt=2)) == 1
    assert call_prefill(lib, ad(dt=2, d=64)) == 1              # d = 64 passes the shape checks
    assert call_prefill(lib, ad(dt=2), qd=ALIGNED, kd=ALIGNED) == 1
    assert call_prefill(lib, ad(dt=2), qd=ALIGNED, kd=ALIGNED + 2, vd=ALIGNED) == 4
    assert call_prefill(lib, ad(dt=1), vd=ALIGNED) == 3


def test_prefill_pointer_mask_and_value_errors(lib):
    assert call_prefill(lib, None) == 1
    assert call_prefill(lib, ad(), k=None) == 1
    assert call_prefill(lib, ad(), out=None) == 1
    assert call_prefill(lib, ad(), v=MISALIGNED) == 4
    assert call_prefill(lib, ad(), mask=MISALIGNED) == 4
    assert call_prefill(lib, ad(), lens=ALIGNED + 2) == 4
    assert call_prefill(lib, ad(S_k=66), mask=ALIGNED) == 2   # mask rows are read 4 keys at a time
    assert call_prefill(lib, ad(), qd=ALIGNED) == 3            # descale factors only with fp8 operands
    assert call_prefill(lib, ad(), scale=-1.0) == 7


def call_prefill_ws(lib, desc, mask=ALIGNED, ws=ALIGNED, ws_bytes=None, **kw):
    if ws_bytes is None:
        ws_bytes = lib.attn_prefill_workspace_bytes(ctypes.byref(desc))
    a = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, qd=None, kd=None, vd=None, lens=None, out=ALIGNED, scale=1.0)
    a.update(kw)
    return lib.attn_prefill_ws(ctypes.byref(desc), a["q"], a["k"], a["v"], a["qd"], a["kd"], a["vd"], a["lens"],
                               mask, a["scale"], a["out"], ws, ws_bytes, None)


@pytest.mark.parametrize("B,S_q,S_k,h_q,n_kv", [(2, 64, 64, 8, 2), (4, 4096, 4096, 32, 8), (3, 1000, 70000, 8, 8),
                                              (1, 33, 600000, 16, 2), (2, 300, 300, 12, 4)])
def test_prefill_workspace_size(lib, B, S_q, S_k, h_q, n_kv):
    """Two bitmaps per (batch entry, row block), one bit per 64-key tile,
    at most 256 words each; a row block holds 32 rows for every wave of 8
    that a head chunk leaves over (chunk = gcd(group size, 8))."""
    G = h_q // n_kv
    hc = next(c for c in (8, 4, 2, 1) if G % c == 0)
    BM = 32 * (8 // hc)
    words = min(-(-S_k // (64 * 32)), 256)
    assert lib.attn_prefill_workspace_bytes(ctypes.byref(ad(B, S_q, S_k, h_q, n_kv))) == \
        B * -(-S_q // BM) * 2 * words * 4
    assert lib.attn_prefill_workspace_bytes(ctypes.byref(ad(B=0))) == 0
    assert lib.attn_prefill_workspace_bytes(None) == 0


def test_prefill_workspace_errors(lib):
    """attn_prefill_ws checks what attn_prefill checks, and with a mask a
    workspace of attn_prefill_workspace_bytes, 16-byte aligned."""
    desc = ad()
    need = lib.attn_prefill_workspace_bytes(ctypes.byref(desc))
    assert need > 0
    assert call_prefill_ws(lib, desc, ws=None) == 5
    assert call_prefill_ws(lib, desc, ws_bytes=need - 1) == 5
    assert call_prefill_ws(lib, desc, ws=MISALIGNED) == 4
    assert call_prefill_ws(lib, ad(S_k=66)) == 2
    assert call_prefill_ws(lib, desc, q=None) == 1
    assert call_prefill_ws(lib, desc, mask=MISALIGNED) == 4
    assert call_prefill_ws(lib, desc, scale=-1.0) == 7
    assert call_prefill_ws(lib, desc, scale=float("nan")) == 7
    assert call_prefill_ws(lib, ad(dt=2)) == 1
    # the workspace is checked before the scale: both are host checks
    assert call_prefill_ws(lib, desc, ws=None, scale=-1.0) == 5


@pytest.mark.parametrize("flags", [2, 4, -1, 1 << 30])
def test_unknown_decode_flags_are_rejected(lib, flags):
    desc = dd(flags=flags)
    assert call_decode(lib, desc) == 7
    assert lib.attn_decode_num_splits(ctypes.byref(desc)) == -1
    assert lib.attn_decode_workspace_bytes(ctypes.byref(desc)) == 0
    pdesc = binding.gqa_paged_desc(2, 8, 2, 128, 1, 1, 64, 10, 4, 0, flags)
    assert lib.attn_decode_paged_num_splits(ctypes.byref(pdesc)) == -1


def test_deterministic_flag_keeps_the_plan(lib):
    """The deterministic mode changes only the order inside a workgroup: the
    split count and the workspace are those of the default mode, and the
    call passes validation (then fails on the first missing pointer)."""
    a, b = dd(B=16, h_q=64, n_kv=8, S=4096), dd(B=16, h_q=64, n_kv=8, S=4096, flags=binding.GQA_DECODE_DETERMINISTIC)
    assert lib.attn_decode_num_splits(ctypes.byref(a)) == lib.attn_decode_num_splits(ctypes.byref(b))
    assert lib.attn_decode_workspace_bytes(ctypes.byref(a)) == lib.attn_decode_workspace_bytes(ctypes.byref(b))
    assert call_decode(lib, b, q=None) == 1
    assert lib.gqa_last_hip_error().decode() == ""



def test_noalloc_scratch_limit_is_checked_on_the_host(lib):
    """attn_decode_noalloc rejects, before any HIP call, a descriptor whose
    partials need more than the static scratch holds (here 64 x 64 slabs)."""
    assert lib.attn_decode_noalloc_max_scratch_bytes() == 16 << 20
    big = dd(B=64, h_q=64, n_kv=64, S=4096)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(big)) > lib.attn_decode_noalloc_max_scratch_bytes()
    assert lib.attn_decode_noalloc(ctypes.byref(big), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, 1.0,
                                   ALIGNED, None) == 8
    assert lib.attn_decode_noalloc(ctypes.byref(dd()), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, 1.0,
                                   None, None) == 1
    assert lib.attn_decode_noalloc(ctypes.byref(dd()), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, -1.0,
                                   ALIGNED, None) == 7
    assert lib.attn_decode_noalloc(ctypes.byref(dd(flags=2)), ALIGNED, ALIGNED, ALIGNED, None, None, ALIGNED, 1.0,
                                   ALIGNED, None) == 7
    assert lib.gqa_last_hip_error().decode() == ""


def test_stream_read_argument_errors(lib):
    assert lib.gqa_stream_read(None, 1024, ALIGNED, None) == 1
    assert lib.gqa_stream_read(ALIGNED, 1024, None, None) == 1
    assert lib.gqa_stream_read(ALIGNED, 0, ALIGNED, None) == 2
    assert lib.gqa_stream_read(ALIGNED, 1000, ALIGNED, None) == 2
    assert lib.gqa_stream_read(MISALIGNED, 1024, ALIGNED, None) == 4
    assert lib.gqa_stream_read(ALIGNED, 1024, ALIGNED + 2, None) == 4
