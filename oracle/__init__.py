"""fp64 CPU oracle for exact grouped-query attention -- TEST INFRASTRUCTURE ONLY.

This package is the correctness yardstick for the GPU library.  It is plain,
slow and materialising on purpose: every score row softmax(scale * q K^T) is
formed in full in float64 and multiplied by V with a library matmul, exactly as
the standard-attention formulation on the pages writes it.  It shares no code,
headers, tables or constants with the HIP path, and the HIP path never imports
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it.

Sources (page title, then section):
  * "Evolution of AI Attention Mechanisms: A Complete Guide from MHA to MLA and
    Flash Attention" -- "MHA Mathematical Formulation" (per-head softmax
    attention with 1/sqrt(d_h) scaling), "MHA Implementation" and
    "GQA Implementation" (scale after the dot product, mask -> -inf, softmax over
    keys, weights times V; K/V heads repeated so query head j reads K/V head
    j // (h_q / n_kv); the cache is concatenated before attention so the newest
    token sees itself), "Flash Attention Usage" (token-major [B, S, H, d]
    layout, causal=True, default scale).
  * "Multi-query attention" (learn.pranaymahendrakar.com) -- "Formulation"
    (O_i = softmax(Q_i K^T / sqrt(d_h)) V with one shared K/V head).
  * "Multi-Query Attention (MQA)" glossary (inferensys.com) -- "KV cache
    quantization" (FP8 / INT8 / INT4 cache with scaling factors).

Modules:
  codecs     -- stored-value decoders (bf16 bit patterns, OCP e4m3fn codes,
                int8 and packed int4 codes).
  attention  -- the decode and causal-prefill definitions.
  paged      -- decode over a paged cache ("Multi-Query Attention (MQA)"
                glossary, "PagedAttention").
  mla        -- absorbed multi-head latent attention decode ("Evolution of AI
                Attention Mechanisms", "Generation 3: MLA").
  masked     -- prefill with general masks: causal or not, key lengths, a
                dense attention mask ("MHA Implementation", "Flash Attention
                Usage").

Pinning: every function here is checked by `-m "not gpu"` tests against
closed forms, invariants the pages fix, a library routine that computes the
same definition, and brute force on tiny inputs.  No function is parity
unpinned.
"""

from . import attention, codecs, masked, mla, paged  # noqa: F401
from .attention import (  # noqa: F401
    attend_one_row,
    decode,
    decode_rows,
    prefill_causal,
    prefill_rows,
)
from .codecs import (  # noqa: F401
    bf16_bits_to_f64,
    dequantize_fp8_cache,
    dequantize_fp8_heads,
    dequantize_int_cache,
    e4m3fn_to_f64,
    int4_unpack,
    int8_to_f64,
)
from .masked import prefill, visible_keys  # noqa: F401
from .mla import mla_decode  # noqa: F401
from .paged import decode_paged, gather_logical_cache  # noqa: F401
