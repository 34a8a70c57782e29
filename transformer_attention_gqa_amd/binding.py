"""ctypes binding of libgqa_attn.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks tensor metadata, fills the descriptor struct,
passes raw device pointers and the current HIP stream, and raises GqaError on a
non-zero status.  PyTorch provides device memory and the stream.

The library is loaded from this package directory.  If it is missing the import
of the functions still works, but every call raises: there is no fallback path.
"""

import ctypes
import os

import torch

LIB_NAME = "libgqa_attn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

GQA_F32, GQA_BF16, GQA_FP8_E4M3, GQA_INT8, GQA_INT4 = 0, 1, 2, 3, 4
GQA_DECODE_DETERMINISTIC = 1
QUANTIZED_KV = (GQA_FP8_E4M3, GQA_INT8, GQA_INT4)
STATUS = {0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_SHAPE", 3: "GQA_ERR_DTYPE", 4: "GQA_ERR_ALIGN",
          5: "GQA_ERR_WORKSPACE", 6: "GQA_ERR_HIP", 7: "GQA_ERR_VALUE", 8: "GQA_ERR_SCRATCH"}
EXPORTED = ("attn_decode_num_splits", "attn_decode_workspace_bytes", "attn_decode", "attn_decode_partials",
            "attn_decode_combine", "attn_decode_paged_num_splits", "attn_decode_paged_workspace_bytes",
            "attn_decode_paged", "attn_decode_mla_num_splits", "attn_decode_mla_workspace_bytes",
            "attn_decode_mla", "attn_decode_mla_partials", "attn_decode_mla_combine", "attn_prefill_causal", "attn_prefill", "attn_prefill_ws", "attn_prefill_workspace_bytes",
            "gqa_status_string", "gqa_last_hip_error",
            "attn_decode_noalloc", "attn_decode_noalloc_max_scratch_bytes", "gqa_stream_read")


class GqaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class gqa_decode_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("S_max", ctypes.c_int32), ("d_h", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("n_split", ctypes.c_int32), ("flags", ctypes.c_int32)]


class gqa_paged_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("n_split", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class gqa_mla_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("h_q", ctypes.c_int32), ("S_max", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_split", ctypes.c_int32)]


class gqa_attn_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S_q", ctypes.c_int32), ("S_k", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("d_h", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32)]


class gqa_prefill_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("d_h", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load_library(path=LIB_PATH):
    """Load (once) and return the ctypes handle; raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{LIB_NAME} is not built ({path} missing); run "
                           "`python -m transformer_attention_gqa_amd.build` first")
    lib = ctypes.CDLL(path)
    vp, cp, i32, f32, sz = ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dd, pd = ctypes.POINTER(gqa_decode_desc), ctypes.POINTER(gqa_prefill_desc)
    lib.attn_decode_num_splits.argtypes, lib.attn_decode_num_splits.restype = [dd], i32
    lib.attn_decode_workspace_bytes.argtypes, lib.attn_decode_workspace_bytes.restype = [dd], sz
    lib.attn_decode.argtypes = [dd, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [dd, vp, vp, vp, vp, vp, vp, f32, vp, vp]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_noalloc_max_scratch_bytes.argtypes, lib.attn_decode_noalloc_max_scratch_bytes.restype = [], sz
    lib.attn_decode_partials.argtypes = [dd, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp]
    lib.attn_decode_partials.restype = ctypes.c_int
    lib.attn_decode_combine.argtypes = [dd, vp, vp, sz, vp, vp]
    lib.attn_decode_combine.restype = ctypes.c_int
    gd = ctypes.POINTER(gqa_paged_desc)
    lib.attn_decode_paged_num_splits.argtypes, lib.attn_decode_paged_num_splits.restype = [gd], i32
    lib.attn_decode_paged_workspace_bytes.argtypes, lib.attn_decode_paged_workspace_bytes.restype = [gd], sz
    lib.attn_decode_paged.argtypes = [gd, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp]
    lib.attn_decode_paged.restype = ctypes.c_int
    md = ctypes.POINTER(gqa_mla_desc)
    lib.attn_decode_mla_num_splits.argtypes, lib.attn_decode_mla_num_splits.restype = [md], i32
    lib.attn_decode_mla_workspace_bytes.argtypes, lib.attn_decode_mla_workspace_bytes.restype = [md], sz
    lib.attn_decode_mla.argtypes = [md, vp, vp, vp, f32, vp, vp, sz, vp]
    lib.attn_decode_mla.restype = ctypes.c_int
    lib.attn_decode_mla_partials.argtypes = [md, vp, vp, vp, f32, vp, sz, vp]
    lib.attn_decode_mla_partials.restype = ctypes.c_int
    lib.attn_decode_mla_combine.argtypes = [md, vp, vp, sz, vp, vp]
    lib.attn_decode_mla_combine.restype = ctypes.c_int
    lib.attn_prefill_causal.argtypes = [pd, vp, vp, vp, f32, vp, vp]
    ad = ctypes.POINTER(gqa_attn_desc)
    lib.attn_prefill.argtypes = [ad, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill_ws.argtypes = [ad, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp]
    lib.attn_prefill_ws.restype = ctypes.c_int
    lib.attn_prefill_workspace_bytes.argtypes, lib.attn_prefill_workspace_bytes.restype = [ad], sz
    lib.attn_prefill_causal.restype = ctypes.c_int
    lib.gqa_stream_read.argtypes, lib.gqa_stream_read.restype = [vp, sz, vp, vp], ctypes.c_int
    lib.gqa_status_string.argtypes, lib.gqa_status_string.restype = [ctypes.c_int], cp
    lib.gqa_last_hip_error.argtypes, lib.gqa_last_hip_error.restype = [], cp
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        lib = load_library()
        msg = lib.gqa_status_string(status).decode()
        if status == 6:
            msg += ": " + lib.gqa_last_hip_error().decode()
        raise GqaError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _temp_workspace(nbytes, device, stream):
    """A workspace the call allocates for itself, on the stream its kernels run
    on: the caching allocator then hands the block to another tensor only
    behind that stream's work, even when `stream` is not torch's current
    stream and the tensor is freed as soon as the call returns."""
    if stream is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return GQA_F32
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return GQA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _kv_code(cache, d):
    """Element type of a K/V cache (or page pool) read with head dim d: int8
    codes are INT8; byte codes are FP8 E4M3 when a row holds d of them and
    packed INT4 when it holds d / 2."""
    if cache.dtype == torch.int8:
        return GQA_INT8
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        if cache.shape[-1] == d:
            return GQA_FP8_E4M3
        if cache.dtype == torch.uint8 and 2 * cache.shape[-1] == d:
            return GQA_INT4
        raise ValueError(f"byte cache rows of {cache.shape[-1]} do not match head dim {d} (fp8) or {d}/2 (int4)")
    return _dtype_code(cache)


def _row_elems(cache, d):
    """Stored elements per cache row for head dim d."""
    return d // 2 if _kv_code(cache, d) == GQA_INT4 else d


def _require(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def decode_desc(q, k_cache, n_split=0, deterministic=False):
    """Descriptor for q [B, h_q, d] and cache [B, n_kv, S_max, d]."""
    B, h_q, d = q.shape
    n_kv, s_max = k_cache.shape[1], k_cache.shape[2]
    return gqa_decode_desc(B, h_q, n_kv, s_max, d, _dtype_code(q), _kv_code(k_cache, d), n_split,
                           GQA_DECODE_DETERMINISTIC if deterministic else 0)


def attn_decode_num_splits(desc):
    return load_library().attn_decode_num_splits(ctypes.byref(desc))


def attn_decode_workspace_bytes(desc):
    return load_library().attn_decode_workspace_bytes(ctypes.byref(desc))


def _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale):
    _require(q, "q", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same shape and dtype")
    if k_cache.shape[0] != q.shape[0] or k_cache.shape[3] != _row_elems(k_cache, q.shape[2]):
        raise ValueError("cache [B, n_kv, S_max, d] (packed int4: d/2 bytes) does not match q [B, h_q, d]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")
    if _kv_code(k_cache, q.shape[2]) in QUANTIZED_KV:
        for name, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None or s.dtype != torch.float32 or tuple(s.shape) != tuple(k_cache.shape[:3]) \
                    or not s.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 tensor of shape [B, n_kv, S_max]")


def _workspace(desc, device, workspace, stream):
    if workspace is None:
        workspace = _temp_workspace(attn_decode_workspace_bytes(desc), device, stream)
    return workspace, workspace.numel() * workspace.element_size()


def attn_decode(q, k_cache, v_cache, seq_lens, scale, out=None, k_scale=None, v_scale=None, workspace=None,
                n_split=0, stream=None, deterministic=False):
    """out[B, h_q, d] = GQA decode step (split + combine kernels).  With
    deterministic=True identical calls give identical bits."""
    _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale)
    desc = decode_desc(q, k_cache, n_split, deterministic)
    if out is None:
        out = torch.empty_like(q)
    workspace, ws_bytes = _workspace(desc, q.device, workspace, stream)
    _check(load_library().attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                      _ptr(v_scale), _ptr(seq_lens), float(scale), _ptr(out), _ptr(workspace),
                                      ws_bytes, _stream(stream)))
    return out


def attn_decode_noalloc_max_scratch_bytes():
    return load_library().attn_decode_noalloc_max_scratch_bytes()


def attn_decode_noalloc(q, k_cache, v_cache, seq_lens, scale, out, k_scale=None, v_scale=None, n_split=0,
                        stream=None, deterministic=False):
    """attn_decode with its partials in the library's static device scratch:
    allocates nothing (the caller passes `out`).  Calls that can overlap on
    one GPU race (see attn_decode_noalloc in gqa_attn.h)."""
    _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    desc = decode_desc(q, k_cache, n_split, deterministic)
    _check(load_library().attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens), float(scale), _ptr(out),
                                              _stream(stream)))
    return out


class PreparedCall:
    """A library call with its arguments checked and packed once.

    Calling it passes the same pointers again (one ctypes call, no per-call
    checks), so the tensors it was built from must stay alive and keep their
    storage.  The stream is the one given at preparation, or else torch's
    current stream at each call."""

    def __init__(self, fn, args, stream, result=None):
        self._fn = fn
        self._args = args
        self._stream = None if stream is None else _stream(stream)
        self.result = result

    def __call__(self):
        st = self._stream if self._stream is not None else ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        _check(self._fn(*self._args, st))
        return self.result


def prepare_decode(q, k_cache, v_cache, seq_lens, scale, out, workspace, k_scale=None, v_scale=None, n_split=0,
                   stream=None, deterministic=False):
    """PreparedCall of attn_decode (see attn_decode for the arguments)."""
    _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale)
    desc = decode_desc(q, k_cache, n_split, deterministic)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < attn_decode_workspace_bytes(desc):
        raise ValueError("workspace smaller than attn_decode_workspace_bytes")
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
            ctypes.c_float(scale), _ptr(out), _ptr(workspace), ctypes.c_size_t(ws_bytes))
    call = PreparedCall(lib.attn_decode, args, stream, out)
    call._keep = (desc,)
    return call


def prepare_decode_partials(q, k_cache, v_cache, seq_lens, scale, workspace, k_scale=None, v_scale=None, n_split=0,
                            stream=None, deterministic=False):
    """PreparedCall of attn_decode_partials."""
    _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale)
    desc = decode_desc(q, k_cache, n_split, deterministic)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
            ctypes.c_float(scale), _ptr(workspace), ctypes.c_size_t(ws_bytes))
    call = PreparedCall(lib.attn_decode_partials, args, stream)
    call._keep = (desc,)
    return call


def attn_decode_partials(q, k_cache, v_cache, seq_lens, scale, workspace, k_scale=None, v_scale=None, n_split=0,
                         stream=None, deterministic=False):
    """Split kernel only: per-chunk partials into `workspace`."""
    _decode_checks(q, k_cache, v_cache, seq_lens, k_scale, v_scale)
    desc = decode_desc(q, k_cache, n_split, deterministic)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().attn_decode_partials(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens), float(scale),
                                               _ptr(workspace), ws_bytes, _stream(stream)))


def attn_decode_combine(q, k_cache, seq_lens, workspace, out, n_split=0, stream=None):
    """Combine kernel only: partials in `workspace` -> out.  q/k_cache give shapes."""
    desc = decode_desc(q, k_cache, n_split)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().attn_decode_combine(ctypes.byref(desc), _ptr(seq_lens), _ptr(workspace), ws_bytes,
                                              _ptr(out), _stream(stream)))
    return out


def paged_desc(q, k_pages, block_table, n_split=0, deterministic=False):
    """Descriptor for q [B, h_q, d], pages [num_pages, n_kv, page_size, d] and block_table [B, max_pages]."""
    B, h_q, d = q.shape
    num_pages, n_kv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    return gqa_paged_desc(B, h_q, n_kv, d, _dtype_code(q), _kv_code(k_pages, d), page_size, num_pages,
                          block_table.shape[1], n_split, GQA_DECODE_DETERMINISTIC if deterministic else 0)


def attn_decode_paged_num_splits(desc):
    return load_library().attn_decode_paged_num_splits(ctypes.byref(desc))


def attn_decode_paged_workspace_bytes(desc):
    return load_library().attn_decode_paged_workspace_bytes(ctypes.byref(desc))


def _paged_checks(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale):
    _require(q, "q", 3)
    _require(k_pages, "k_pages", 4)
    _require(v_pages, "v_pages", 4)
    if k_pages.shape != v_pages.shape or k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must have the same shape and dtype")
    if k_pages.shape[3] != _row_elems(k_pages, q.shape[2]):
        raise ValueError("pages [num_pages, n_kv, page_size, d] (packed int4: d/2 bytes) do not match q [B, h_q, d]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != q.shape[0] \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 tensor of shape [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")
    if _kv_code(k_pages, q.shape[2]) in QUANTIZED_KV:
        for name, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None or s.dtype != torch.float32 or tuple(s.shape) != tuple(k_pages.shape[:3]) \
                    or not s.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 tensor of shape [num_pages, n_kv, page_size]")


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, out=None, k_scale=None, v_scale=None,
                      workspace=None, n_split=0, stream=None, deterministic=False):
    """out[B, h_q, d] = GQA decode step over a paged cache (see attn_decode_paged in gqa_attn.h)."""
    _paged_checks(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale)
    desc = paged_desc(q, k_pages, block_table, n_split, deterministic)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _temp_workspace(attn_decode_paged_workspace_bytes(desc), q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().attn_decode_paged(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                            _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
                                            float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def prepare_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, out, workspace, k_scale=None,
                         v_scale=None, n_split=0, stream=None):
    """PreparedCall of attn_decode_paged."""
    _paged_checks(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale)
    desc = paged_desc(q, k_pages, block_table, n_split)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < attn_decode_paged_workspace_bytes(desc):
        raise ValueError("workspace smaller than attn_decode_paged_workspace_bytes")
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), _ptr(seq_lens), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(ws_bytes))
    call = PreparedCall(lib.attn_decode_paged, args, stream, out)
    call._keep = (desc,)
    return call


def mla_desc(q_abs, c_kv, n_split=0):
    """Descriptor for q_abs [B, h_q, d_c] and c_kv [B, S_max, d_c]."""
    B, h_q, d_c = q_abs.shape
    return gqa_mla_desc(B, h_q, c_kv.shape[1], d_c, _dtype_code(q_abs), n_split)


def attn_decode_mla_num_splits(desc):
    return load_library().attn_decode_mla_num_splits(ctypes.byref(desc))


def attn_decode_mla_workspace_bytes(desc):
    return load_library().attn_decode_mla_workspace_bytes(ctypes.byref(desc))


def _mla_checks(q_abs, c_kv, seq_lens, out):
    _require(q_abs, "q_abs", 3)
    _require(c_kv, "c_kv", 3)
    if c_kv.dtype != q_abs.dtype or c_kv.shape[0] != q_abs.shape[0] or c_kv.shape[2] != q_abs.shape[2]:
        raise ValueError("c_kv must be [B, S_max, d_c] typed and sized like q_abs [B, h_q, d_c]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q_abs.shape[0],) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape [B]")
    if out.shape != q_abs.shape or out.dtype != q_abs.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q_abs")


def attn_decode_mla(q_abs, c_kv, seq_lens, scale, out=None, workspace=None, n_split=0, stream=None):
    """o_c[B, h_q, d_c] = absorbed latent-attention decode step (see attn_decode_mla in gqa_attn.h)."""
    if out is None:
        out = torch.empty_like(q_abs)
    _mla_checks(q_abs, c_kv, seq_lens, out)
    desc = mla_desc(q_abs, c_kv, n_split)
    if workspace is None:
        workspace = _temp_workspace(attn_decode_mla_workspace_bytes(desc), q_abs.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().attn_decode_mla(ctypes.byref(desc), _ptr(q_abs), _ptr(c_kv), _ptr(seq_lens),
                                          float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def prepare_decode_mla(q_abs, c_kv, seq_lens, scale, out, workspace, n_split=0, stream=None):
    """PreparedCall of attn_decode_mla."""
    _mla_checks(q_abs, c_kv, seq_lens, out)
    desc = mla_desc(q_abs, c_kv, n_split)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < attn_decode_mla_workspace_bytes(desc):
        raise ValueError("workspace smaller than attn_decode_mla_workspace_bytes")
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q_abs), _ptr(c_kv), _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), ctypes.c_size_t(ws_bytes))
    call = PreparedCall(lib.attn_decode_mla, args, stream, out)
    call._keep = (desc,)
    return call


def prepare_decode_mla_partials(q_abs, c_kv, seq_lens, scale, workspace, n_split=0, stream=None):
    """PreparedCall of attn_decode_mla_partials (split kernel only)."""
    _mla_checks(q_abs, c_kv, seq_lens, q_abs)
    desc = mla_desc(q_abs, c_kv, n_split)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q_abs), _ptr(c_kv), _ptr(seq_lens), ctypes.c_float(scale), _ptr(workspace),
            ctypes.c_size_t(ws_bytes))
    call = PreparedCall(lib.attn_decode_mla_partials, args, stream)
    call._keep = (desc,)
    return call


def _prefill_desc(q, k, v, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _require(t, name, 4)
    B, S, h_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != S or k.shape[3] != d:
        raise ValueError("k/v must be [B, S, n_kv, d] matching q [B, S, h_q, d]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be shaped and typed like q")
    return gqa_prefill_desc(B, S, h_q, k.shape[2], d, _dtype_code(q))


def attn_prefill_causal(q, k, v, scale, out=None, stream=None):
    """out[B, S, h_q, d] = causal GQA attention over q [B,S,h_q,d], k/v [B,S,n_kv,d] (bf16)."""
    if out is None:
        out = torch.empty_like(q)
    desc = _prefill_desc(q, k, v, out)
    _check(load_library().attn_prefill_causal(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), float(scale),
                                              _ptr(out), _stream(stream)))
    return out


def prepare_prefill_causal(q, k, v, scale, out, stream=None):
    """PreparedCall of attn_prefill_causal."""
    desc = _prefill_desc(q, k, v, out)
    lib = load_library()
    call = PreparedCall(lib.attn_prefill_causal, (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                                  ctypes.c_float(scale), _ptr(out)), stream, out)
    call._keep = (desc,)
    return call


def _attn_desc(q, k, v, out, causal, kv_lens, mask):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _require(t, name, 4)
    B, S_q, h_q, d = q.shape
    if k.shape != v.shape or k.dtype != v.dtype or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v must be [B, S_k, n_kv, d] matching q [B, S_q, h_q, d]")
    if out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be a bf16 tensor shaped like q")
    if q.dtype != k.dtype:
        raise ValueError("q and k/v must have the same dtype (bf16, or uint8 e4m3 codes)")
    S_k = k.shape[1]
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.shape != (B,) or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 tensor of shape [B]")
    if mask is not None and (mask.dtype not in (torch.uint8, torch.bool) or tuple(mask.shape) != (B, S_q, S_k)
                             or not mask.is_contiguous()):
        raise ValueError("mask must be a contiguous uint8/bool tensor of shape [B, S_q, S_k]")
    return gqa_attn_desc(B, S_q, S_k, h_q, k.shape[2], d, _dtype_code(q), 1 if causal else 0)


def _descale_checks(q, k, descales):
    if q.dtype != torch.uint8:
        if any(d is not None for d in descales):
            raise ValueError("descale factors go with fp8 (uint8 e4m3 code) operands only")
        return
    B, h_q, n_kv = q.shape[0], q.shape[2], k.shape[2]
    for name, d, H in zip(("q_descale", "k_descale", "v_descale"), descales, (h_q, n_kv, n_kv)):
        if d is None or d.dtype != torch.float32 or tuple(d.shape) != (B, H) or not d.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape [B, {H}]")


def attn_prefill_workspace_bytes(desc):
    """Bytes of workspace attn_prefill_ws needs for a masked call (the
    per-row-block key-tile bitmaps)."""
    return load_library().attn_prefill_workspace_bytes(ctypes.byref(desc))


def attn_prefill(q, k, v, scale, causal=True, kv_lens=None, mask=None, out=None, q_descale=None, k_descale=None,
                 v_descale=None, stream=None, workspace=None, mask_prepass=True):
    """out[B, S_q, h_q, d] (bf16) = attention of q [B,S_q,h_q,d] over k/v [B,S_k,n_kv,d] with the causal rule
    (end-aligned), key lengths and a dense [B, S_q, S_k] mask.  Operands are bf16, or uint8 e4m3 codes with
    per-(batch, head) descale factors (see attn_prefill in gqa_attn.h).

    With a mask and `mask_prepass` (the default) the call goes through
    attn_prefill_ws: one pass classifies every row block's key tiles into
    `workspace` (allocated on the call's stream when None) and the attention
    kernel reads those bitmaps.  `mask_prepass=False` calls attn_prefill,
    whose workgroups each scan their own mask rows; both give the same bits."""
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    desc = _attn_desc(q, k, v, out, causal, kv_lens, mask)
    _descale_checks(q, k, (q_descale, k_descale, v_descale))
    lib = load_library()
    head = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
            _ptr(kv_lens), _ptr(mask), float(scale), _ptr(out))
    if mask is None or not mask_prepass:
        if workspace is not None:
            raise ValueError("a workspace goes with a masked call through the pre-pass only")
        _check(lib.attn_prefill(*head, _stream(stream)))
        return out
    if workspace is None:
        workspace = _temp_workspace(attn_prefill_workspace_bytes(desc), q.device, stream)
    _check(lib.attn_prefill_ws(*head, _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)))
    return out


def prepare_prefill(q, k, v, scale, out, causal=True, kv_lens=None, mask=None, q_descale=None, k_descale=None,
                    v_descale=None, stream=None, workspace=None):
    """PreparedCall of attn_prefill, or of attn_prefill_ws when a workspace
    (at least attn_prefill_workspace_bytes) is given with a mask."""
    desc = _attn_desc(q, k, v, out, causal, kv_lens, mask)
    _descale_checks(q, k, (q_descale, k_descale, v_descale))
    lib = load_library()
    head = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
            _ptr(kv_lens), _ptr(mask), ctypes.c_float(scale), _ptr(out))
    if workspace is None:
        call = PreparedCall(lib.attn_prefill, head, stream, out)
    else:
        if mask is None:
            raise ValueError("a workspace goes with a masked call only")
        ws_bytes = workspace.numel() * workspace.element_size()
        if ws_bytes < attn_prefill_workspace_bytes(desc):
            raise ValueError("workspace smaller than attn_prefill_workspace_bytes")
        call = PreparedCall(lib.attn_prefill_ws, head + (_ptr(workspace), ctypes.c_size_t(ws_bytes)), stream, out)
        call._keep_ws = workspace
    call._keep = (desc,)
    return call


def gqa_stream_read(buf, sink, stream=None):
    """Read every byte of `buf` once on the GPU (the measured HBM read
    ceiling); `sink` is a one-element int32/uint32 device tensor."""
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().gqa_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
