"""Exact grouped-query attention for AMD MI355X (gfx950).

The compute path is libgqa_attn.so (hand-written HIP kernels behind a C ABI,
declared in include/gqa_attn.h); `binding` marshals torch tensors into it.
`inputs` draws the seeded synthetic workloads and `roofline` counts the
algorithmic bytes and flops the measurements are priced with.
"""

from . import inputs, roofline  # noqa: F401
from .binding import (  # noqa: F401
    GqaError,
    attn_decode,
    attn_decode_combine,
    attn_decode_mla,
    attn_decode_num_splits,
    attn_decode_partials,
    attn_decode_workspace_bytes,
    attn_prefill_causal,
    decode_desc,
    load_library,
)
