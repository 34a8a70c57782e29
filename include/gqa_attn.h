/*
 * gqa_attn.h -- exact grouped-query attention on AMD MI355X (gfx950).
 *
 * C ABI of libgqa_attn.so.  Plain pointers and sizes only.
 *
 * The operation ("Evolution of AI Attention Mechanisms: A Complete Guide from
 * MHA to MLA and Flash Attention", sections "MHA Mathematical Formulation" and
 * "GQA Implementation"; "Multi-query attention", section "Formulation"):
 * each of h_q query heads attends to one of n_kv shared K/V heads.  Query head
 * j uses K/V head j / G, where G = h_q / n_kv is the group size: the GQA module
 * repeats K/V head g for query heads g*G .. g*G+G-1.  G = 1 is MHA and
 * G = h_q is MQA.  For each query row,
 *
 *     out = softmax(scale * q . K^T) V        (over the visible keys)
 *
 * computed exactly (up to floating-point rounding order) with a running max
 * and running sum, so the score matrix is never written to memory ("Flash
 * Attention Principle" on the first page).
 *
 * Conventions shared by every call
 *  - Every tensor pointer is caller-owned device memory on the current HIP
 *    device, densely packed in the stated layout (innermost index last), and
 *    aligned to 16 bytes.  The library never allocates, frees or synchronises,
 *    and keeps no pointer after the call returns.
 *  - Work is enqueued on `stream` (NULL = the default stream) and runs
 *    asynchronously; the call returns once the kernels are enqueued.
 *  - Arguments are checked on the host before any HIP call.  A bad argument
 *    returns a status code and enqueues nothing.  A launch failure returns
 *    GQA_ERR_HIP (gqa_last_hip_error() gives the HIP message).  Faults inside
 *    a kernel surface at the caller's next synchronisation.
 *  - Calls are stateless and may run concurrently on different streams as
 *    long as each decode call has its own workspace.
 *  - `out` must not overlap any input or the workspace.
 *  - Supported head dimensions: d_h = 64 or 128.
 *  - `scale` multiplies q . k before the softmax (the modules use
 *    head_dim ** -0.5); it must be finite and >= 0 (GQA_ERR_VALUE otherwise).
 *    0 gives every visible key the same weight (the mean of their values).
 *    A scale whose product with log2(e) is below the smallest normal float
 *    is raised to it (the scores are then zero to float precision).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as in hip_runtime_api.h; repeating an identical typedef is
 * valid C11/C++, so this header stands alone for plain C callers. */
typedef struct ihipStream_t* hipStream_t;

/* Element types. */
enum {
  GQA_F32 = 0,       /* IEEE binary32                                        */
  GQA_BF16 = 1,      /* bfloat16 (upper half of binary32)                    */
  GQA_FP8_E4M3 = 2,  /* OCP 8-bit float E4M3 ("e4m3fn": bias 7, max 448,     */
                     /* no infinities, NaN = S.1111.111)                     */
  GQA_INT8 = 3,      /* signed 8-bit integer code                            */
  GQA_INT4 = 4       /* signed 4-bit integer code (two's complement), two    */
                     /* per byte: element 2i in bits 0..3 of byte i,         */
                     /* element 2i+1 in bits 4..7                            */
};

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  GQA_ERR_SHAPE = 2,     /* a dimension <= 0, h_q % n_kv != 0, bad d_h or
                            page_size, ...                                    */
  GQA_ERR_DTYPE = 3,     /* unsupported element-type combination              */
  GQA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                  */
  GQA_ERR_WORKSPACE = 5, /* workspace missing or smaller than required        */
  GQA_ERR_HIP = 6,       /* a HIP launch or query failed                      */
  GQA_ERR_VALUE = 7,     /* scale is not a finite number >= 0, or a flags
                            word holds unknown bits                           */
  GQA_ERR_SCRATCH = 8    /* attn_decode_noalloc: the call's partials need
                            more than attn_decode_noalloc_max_scratch_bytes() */
} gqa_status;

/* Decode flags (gqa_decode_desc.flags, gqa_paged_desc.flags). */
enum {
  /* Fixed tile order inside each workgroup, so that identical calls give
   * bitwise-identical outputs on every path (see "Sequence split" below).
   * Costs a few percent of decode time; without it the waves of a
   * workgroup take tiles as they free up. */
  GQA_DECODE_DETERMINISTIC = 1
};

/* ---------------------------------------------------------------- decode --
 * One autoregressive step over a KV cache.  The new token's K/V has already
 * been written into the cache, so it attends to itself: the GQA and MHA
 * modules concatenate the cache before attention ("GQA Implementation").
 * The decode step is softmax(Q_all K_shared^T) V_shared for the heads of a
 * group ("Multi-Query Attention (MQA)" glossary, "Kernel Optimization").
 *
 * Shapes (row-major, innermost last):
 *   q        [B, h_q, d_h]             q_dtype (F32 or BF16)
 *   k_cache  [B, n_kv, S_max, d_h]     kv_dtype -- the cache layout after the
 *   v_cache  [B, n_kv, S_max, d_h]     modules' view(B,S,n_kv,d).transpose(1,2)
 *                                      (INT4: [B, n_kv, S_max, d_h/2] bytes)
 *   k_scale  [B, n_kv, S_max] float32  FP8 / INT8 / INT4 caches only: one
 *   v_scale  [B, n_kv, S_max] float32  dequantisation factor per (token,
 *                                      kv-head) row; value = decode(code) *
 *                                      scale ("KV cache quantization" in the
 *                                      MQA glossary).  NULL for F32/BF16.
 *   seq_lens [B] int32 (device)        L_b = visible cache positions 0..L_b-1
 *                                      of sequence b.  Read on the device
 *                                      only: values are clamped to [0, S_max];
 *                                      L_b = 0 yields a zero output row.
 *   out      [B, h_q, d_h]             q_dtype
 * Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 * (BF16, INT8), (BF16, INT4).  Codes become bf16 exactly; the K scale
 * multiplies the score and the V scale the softmax weight.  Accumulation is
 * float32 throughout.
 *
 * Sequence split: the 32-token tiles (64 on the F32 path, and on the INT4
 * path when a K/V head serves at most 16 query heads) of every
 * (sequence, kv-head) are concatenated and cut into n_split equal ranges, one
 * per workgroup, so ragged lengths are balanced across the GPU.  Each range
 * leaves an unnormalised partial (O_s, m_s, l_s) per head for every
 * (sequence, kv-head) it touches, and a combine kernel merges them:
 *   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
 * By default, on the matrix-core paths the waves of a workgroup take the
 * tiles of its range as they become free, so the float32 summation order and
 * the point at which each wave rounds its softmax weights to bf16 can change
 * between two identical calls: results agree to about 1e-3, not bit for bit.
 * With GQA_DECODE_DETERMINISTIC in `flags` wave i of a workgroup takes tiles
 * i, i + 8, i + 16, ... of each segment, and identical calls (same
 * descriptor, same device) give identical bits.  The float32 path always has
 * a fixed order.
 */
typedef struct gqa_decode_desc {
  int32_t B, h_q, n_kv, S_max, d_h;
  int32_t q_dtype, kv_dtype; /* GQA_F32 / GQA_BF16 / GQA_FP8_E4M3 / ...     */
  int32_t n_split;           /* 0: one workgroup per compute unit of the
                                current device (queried once per device;
                                256 if no device can be queried).  > 0:
                                number of workgroups / key ranges.  Either is
                                capped at the number of tiles of a full cache
                                and at 65536 (the effective count is
                                attn_decode_num_splits()).                    */
  int32_t flags;             /* 0 or GQA_DECODE_DETERMINISTIC                 */
} gqa_decode_desc;

/* Effective number of key ranges (= decode workgroups) for this descriptor,
 * or -1 if the descriptor is invalid.  Host-only (with n_split = 0 it reads
 * the current device's compute-unit count, enqueuing nothing). */
int32_t attn_decode_num_splits(const gqa_decode_desc* d);

/* Bytes of device workspace attn_decode needs for this descriptor (0 if the
 * descriptor is invalid).  Host-only, as attn_decode_num_splits. */
size_t attn_decode_workspace_bytes(const gqa_decode_desc* d);

/* Full decode step: split kernel then combine kernel, both on `stream`.
 * workspace: caller-owned device memory of at least
 * attn_decode_workspace_bytes(d) bytes (any contents); it must stay untouched
 * until the stream reaches the end of this call's work. */
gqa_status attn_decode(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                       void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two halves of attn_decode, for callers that want to place other work
 * between them -- e.g. exchange partials between devices that each hold a
 * slice of a long sequence before combining.  attn_decode_partials writes the
 * per-chunk partials into `workspace`; attn_decode_combine reads them and
 * writes `out`.  Both take the same descriptor, seq_lens and workspace. */
gqa_status attn_decode_partials(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);
gqa_status attn_decode_combine(const gqa_decode_desc* d, const int32_t* seq_lens, const void* workspace,
                               size_t workspace_bytes, void* out, hipStream_t stream);

/* ------------------------------------------- decode without allocation --
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * step of attn_decode with the same arguments except the workspace.  The
 * partials live in a static device array of the library, 16 MiB per GPU,
 * which each GPU the library runs on holds until the process ends; its
 * device address is looked up once per device on the first call there.
 * The call allocates and frees nothing (no hipMalloc, no hipFree).
 * A descriptor whose workspace (attn_decode_workspace_bytes) exceeds
 * attn_decode_noalloc_max_scratch_bytes() returns GQA_ERR_SCRATCH and
 * enqueues nothing; the ragged GQA, long MQA and fp8 / int8 / int4 cache
 * workloads of this library's benchmark need at most 5.3 MiB.  All calls on
 * one GPU share its array: two calls whose work can overlap on that GPU
 * (different streams without ordering between them) race and give wrong
 * results; calls ordered on one stream are safe.  No contents need to carry
 * over between calls.  Results equal those of attn_decode with the same
 * descriptor (bit for bit with GQA_DECODE_DETERMINISTIC). */
size_t attn_decode_noalloc_max_scratch_bytes(void);
gqa_status attn_decode_noalloc(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                               void* out, hipStream_t stream);

/* ------------------------------------------------------ paged decode --
 * The decode step of attn_decode over a paged cache ("Multi-Query Attention
 * (MQA)" glossary, "PagedAttention": each sequence's cache is cut into
 * fixed-size pages that may lie anywhere in memory).
 *
 * Shapes (row-major, innermost last):
 *   q             [B, h_q, d_h]                     q_dtype
 *   k_pages       [num_pages, n_kv, page_size, d_h] kv_dtype (INT4: d_h/2
 *                                                   bytes per row) -- a pool of
 *   v_pages       [num_pages, n_kv, page_size, d_h] pages; page p holds
 *                                                   page_size consecutive
 *                                                   tokens of all K/V heads
 *                                                   of one sequence
 *   k_scale_pages [num_pages, n_kv, page_size] float32   FP8/INT8/INT4 only
 *   v_scale_pages [num_pages, n_kv, page_size] float32
 *   block_table   [B, max_pages_per_seq] int32 (device): entry (b, i) is the
 *                 page holding tokens i*page_size .. (i+1)*page_size - 1 of
 *                 sequence b.  Only the entries of the pages covering
 *                 positions 0 .. L_b-1 are read; an entry outside
 *                 [0, num_pages) is clamped into the pool (no fault; the
 *                 output is then unspecified).
 *   seq_lens      [B] int32 (device), clamped to [0, max_pages_per_seq *
 *                 page_size]; L_b = 0 yields a zero row.
 *   out           [B, h_q, d_h]                     q_dtype
 * page_size must be a power of two >= 32.  Element types, workspace and
 * results are those of attn_decode with S_max = max_pages_per_seq *
 * page_size: the same kernels run with one block-table lookup per 32-token
 * tile (the entries of a range are held in registers, 64 at a time).
 */
typedef struct gqa_paged_desc {
  int32_t B, h_q, n_kv, d_h;
  int32_t q_dtype, kv_dtype;
  int32_t page_size;         /* tokens per page: a power of two >= 32      */
  int32_t num_pages;         /* pages in the pool                          */
  int32_t max_pages_per_seq; /* columns of block_table                     */
  int32_t n_split;           /* as in gqa_decode_desc                      */
  int32_t flags;             /* as in gqa_decode_desc                      */
} gqa_paged_desc;

int32_t attn_decode_paged_num_splits(const gqa_paged_desc* d);
size_t attn_decode_paged_workspace_bytes(const gqa_paged_desc* d);
gqa_status attn_decode_paged(const gqa_paged_desc* d, const void* q, const void* k_pages, const void* v_pages,
                             const float* k_scale_pages, const float* v_scale_pages, const int32_t* block_table,
                             const int32_t* seq_lens, float scale, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- latent-attention decode --
 * One decode step of multi-head latent attention in its absorbed form
 * ("Evolution of AI Attention Mechanisms", section "Generation 3: MLA"): the
 * cache holds one latent vector c_kv of d_c values per token, and each head's
 * query has already been moved into the latent space (q_abs,h = W_k,h^T q_h,
 * with W_k,h the head's rows of the key up-projection).  Every head then
 * attends to the latent rows, which serve as its keys and its values:
 *
 *     o_c,h = softmax(scale * q_abs,h . c_kv^T) c_kv   (over the L_b tokens)
 *
 * The value up-projection W_v,h and the output projection are applied by the
 * caller afterwards.  This is MQA with one shared K = V head of width d_c.
 *
 * Shapes (row-major, innermost last):
 *   q_abs    [B, h_q, d_c]    bfloat16
 *   c_kv     [B, S_max, d_c]  bfloat16
 *   seq_lens [B] int32 (device), clamped to [0, S_max]; L_b = 0 gives a
 *            zero row
 *   out      [B, h_q, d_c]    bfloat16
 * d_c = 256 or 512; dtype must be GQA_BF16.  Products on bf16 matrix cores
 * with float32 accumulation; each latent row is read from memory once for
 * both products and for all heads (up to 64 heads per pass over the cache;
 * h_q > 64 takes ceil(h_q / 64) passes).  Split, workspace and
 * reproducibility are those of attn_decode, with slabs (sequence, chunk of
 * up to 64 heads) and 32-token tiles.
 */
typedef struct gqa_mla_desc {
  int32_t B, h_q, S_max, d_c;
  int32_t dtype;   /* GQA_BF16 */
  int32_t n_split; /* as in gqa_decode_desc */
} gqa_mla_desc;

int32_t attn_decode_mla_num_splits(const gqa_mla_desc* d);
size_t attn_decode_mla_workspace_bytes(const gqa_mla_desc* d);
gqa_status attn_decode_mla(const gqa_mla_desc* d, const void* q_abs, const void* c_kv, const int32_t* seq_lens,
                           float scale, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);
/* The two halves of attn_decode_mla (split kernel, then combine kernel),
 * with the same roles and arguments as attn_decode_partials and
 * attn_decode_combine. */
gqa_status attn_decode_mla_partials(const gqa_mla_desc* d, const void* q_abs, const void* c_kv,
                                    const int32_t* seq_lens, float scale, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);
gqa_status attn_decode_mla_combine(const gqa_mla_desc* d, const int32_t* seq_lens, const void* workspace,
                                   size_t workspace_bytes, void* out, hipStream_t stream);

/* ------------------------------------------------------- causal prefill --
 * Causal self-attention over whole prompts, the mode of the library call
 * flash_attn_func(q, k, v, causal=True, softmax_scale=...) in "Flash
 * Attention Usage": query row r sees keys 0..r (diagonal included).
 *
 * Shapes (token-major, the layout handed to flash_attn_func):
 *   q, out   [B, S, h_q, d_h]   bfloat16
 *   k, v     [B, S, n_kv, d_h]  bfloat16
 * dtype must be GQA_BF16.  QK^T and PV run on bf16 matrix cores with float32
 * accumulation; the running max and sum are float32; out is rounded to bf16.
 */
typedef struct gqa_prefill_desc {
  int32_t B, S, h_q, n_kv, d_h;
  int32_t dtype; /* GQA_BF16 */
} gqa_prefill_desc;

gqa_status attn_prefill_causal(const gqa_prefill_desc* d, const void* q, const void* k, const void* v, float scale,
                               void* out, hipStream_t stream);

/* --------------------------------------------- prefill, general masks --
 * Prefill attention with the masks of the pages' interfaces: the module's
 * attention_mask (scores where the mask is 0 become -inf before the softmax;
 * "Evolution of AI Attention Mechanisms", "MHA Implementation") and
 * flash_attn_func's causal flag ("Flash Attention Usage").  The module
 * concatenates cached keys ahead of the new ones, so S_k may exceed S_q.
 *
 * Shapes (token-major):
 *   q, out   [B, S_q, h_q, d_h]   bfloat16
 *   k, v     [B, S_k, n_kv, d_h]  bfloat16
 *   kv_lens  [B] int32 (device) or NULL: keys c >= kv_lens[b] (clamped to
 *            [0, S_k]) are invisible to every row of sequence b and are
 *            never read, so padding may hold anything
 *   mask     [B, S_q, S_k] uint8 (device) or NULL, shared by all heads: key c
 *            is invisible to query row r where mask[b][r][c] == 0 (any
 *            nonzero byte keeps it); needs S_k % 4 == 0
 * causal = 1 adds the causal rule aligned at the end of the keys: query row
 * r sees keys c <= r + S_k - S_q (c <= r when S_q = S_k).  The conditions
 * combine by AND.  A query row that sees no key gets a zero output row.
 * Keys hidden only by the causal rule or the mask are read and multiplied
 * by a zero weight, so their values must be finite.
 * dtype GQA_BF16: q/k/v bfloat16, q/k/v_descale NULL.  Products on bf16
 * matrix cores, float32 statistics, out rounded to bf16.
 * dtype GQA_FP8_E4M3 (the FP8 mode listed for FlashAttention-3 in "Flash
 * Attention 3 Features"): q/k/v hold OCP E4M3 codes (same shapes, one byte
 * per element) and the values are code * descale with float32 factors
 *   q_descale [B, h_q], k_descale [B, n_kv], v_descale [B, n_kv] (device),
 *   finite and >= 0 (an all-zero head quantised by absmax has descale 0;
 *   its scores are then 0, i.e. equal weights);
 * d_h = 64 or 128.  Both products run on fp8 matrix cores: the scores from
 * the codes (the descale factors fold into the score scale and the output),
 * and the weighted sum with each softmax weight split into two E4M3 terms,
 * hi = e4m3(p) and lo = e4m3(p - hi), two products per d tile (relative
 * error at most 2^-8 per weight, 2^-10 absolute for the smallest), float32
 * accumulation, out bf16.
 * Key tiles past every row's visible prefix are skipped, and a wave skips
 * the products of a tile the dense mask hides from all of its rows.
 */
typedef struct gqa_attn_desc {
  int32_t B, S_q, S_k, h_q, n_kv, d_h;
  int32_t dtype;  /* GQA_BF16 or GQA_FP8_E4M3 */
  int32_t causal; /* 0 or 1 */
} gqa_attn_desc;

gqa_status attn_prefill(const gqa_attn_desc* d, const void* q, const void* k, const void* v,
                        const float* q_descale, const float* k_descale, const float* v_descale,
                        const int32_t* kv_lens, const uint8_t* mask, float scale, void* out, hipStream_t stream);

/* attn_prefill with a caller-owned workspace for the dense mask's key-tile
 * bitmaps.  Without a workspace (attn_prefill) every workgroup scans the mask
 * rows of its row block to find the key tiles any row sees and those every
 * row sees, once per K/V-head workgroup; with one, a pass over the mask forms
 * them once per (batch entry, row block) before the attention kernel, on the
 * same stream.  The results are the same bits either way.
 *   workspace        device, 16-byte aligned, attn_prefill_workspace_bytes(d)
 *                    bytes or more (GQA_ERR_WORKSPACE otherwise); ignored and
 *                    may be NULL when mask is NULL
 * The workspace holds no state between calls; calls that may run
 * concurrently need their own. */
gqa_status attn_prefill_ws(const gqa_attn_desc* d, const void* q, const void* k, const void* v,
                           const float* q_descale, const float* k_descale, const float* v_descale,
                           const int32_t* kv_lens, const uint8_t* mask, float scale, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes attn_prefill_ws needs for a dense mask (host only): per
 * (batch entry, row block), two bitmaps of one bit per 64-key tile in 32-bit
 * words (at most 256 words each); 0 for an invalid descriptor. */
size_t attn_prefill_workspace_bytes(const gqa_attn_desc* d);

/* -------------------------------------------------------- measurement --
 * Read-only HBM stream: reads every byte of `buf` once (128-bit non-temporal
 * loads, the decode kernels' loads) and writes nothing but, in a practically
 * impossible case, one word to `sink`.  Its rate is the measured read
 * ceiling that decode's achieved bandwidth (KV bytes per step, the
 * "bandwidth argument" of "Multi-query attention") is compared with beside
 * the vendor peak.  bytes: a nonzero multiple of 16; buf 16-byte aligned;
 * sink: one caller-owned uint32 of device memory (contents unspecified
 * afterwards). */
gqa_status gqa_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------- errors --- */
/* Static, human-readable name of a status code. */
const char* gqa_status_string(gqa_status s);
/* Message of the last HIP error seen by this thread's calls ("" if none). */
const char* gqa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
