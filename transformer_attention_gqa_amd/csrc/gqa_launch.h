// Internal launch interface between the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Decode work schedule.  The keys of one (sequence b, kv-head g, head chunk hc)
// form a "slab" of ceil(L_b / tile) tiles; slabs are ordered (b, g, hc) and
// their tiles concatenated into one global tile range [0, T).  Workgroup w of
// the W launched takes the balanced range [w*T/W, (w+1)*T/W), which may cross
// slab boundaries; for each slab sigma it touches it leaves one partial
// (O, m, l) per head in slot (w + sigma).  Distinct (w, sigma) pairs of
// non-empty ranges never share a slot, so there are at most W + n_slabs slots
// and no atomics.  The combine for a slab recomputes which workgroups covered
// it: tile t belongs to workgroup ((t+1)*W - 1) / T; for T >= W every range
// is non-empty and the slab's partials come from all workgroups between the
// owners of its first and last tile; for T < W each range holds at most one
// tile and the owners are taken tile by tile.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* seq_lens;
  // paged cache (block_table != null): k/v (and the fp8 scales) are a pool of
  // pages [num_pages][n_kv][page_size][...], page_size = 1 << page_shift, and
  // token t of sequence b lives in page block_table[b * max_pages + t / page_size];
  // S_max is then max_pages * page_size
  const int32_t* block_table;
  int page_shift, max_pages, num_pages;
  float* part_o;   // [W + n_slabs][heads_per_chunk][D]
  float* part_ml;  // [W + n_slabs][heads_per_chunk][2]: running max (log2 domain), running sum
  float qk_scale_log2;
  int B, h_q, n_kv, S_max, n_hchunk, heads_per_chunk;
  int deterministic;  // nonzero: wave i takes tiles i, i + NW, ... of a segment (no tile claims)
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* seq_lens;
  void* out;
  int B, h_q, n_kv, S_max, n_hchunk, heads_per_chunk, tile, W;
};

// Absorbed latent-attention decode: one latent row c[b][t][0..D) per token
// serves as key and value of every query head.  Slabs are (sequence b, head
// chunk hc), n_hchunk per sequence, and use the decode schedule and partial
// layout above (n_kv = 1).
struct MlaArgs {
  const void* q;   // [B][h_q][D] bf16, absorbed queries
  const void* c;   // [B][S_max][D] bf16, latent cache
  const int32_t* seq_lens;
  float* part_o;   // [W + n_slabs][heads_per_chunk][D]
  float* part_ml;  // [W + n_slabs][heads_per_chunk][2]
  float qk_scale_log2;
  int B, h_q, S_max, n_hchunk, heads_per_chunk;
};

// kind: 0 = float32 Q/K/V, 1 = bf16 Q/K/V; bf16 Q with 2 = e4m3, 3 = int8 or
// 4 = packed int4 K/V (each with per-row scales).
// hb: 16-head blocks per workgroup on the matrix-core paths (1 or 2).
// W: number of workgroups (balanced key ranges).
hipError_t launch_decode_split(const DecodeArgs& a, int D, int hb, int kind, int W, hipStream_t stream);
// hb: 32-head blocks per workgroup (1 or 2); D = 256 or 512.
hipError_t launch_mla_decode_split(const MlaArgs& a, int D, int hb, int W, hipStream_t stream);
hipError_t launch_decode_combine(const CombineArgs& c, int D, bool out_bf16, hipStream_t stream);
hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S, int h_q, int n_kv, int D, int n_cu, hipStream_t stream);
// General masks: S_q query rows, S_k keys, optional end-aligned causal rule,
// key lengths [B] and dense mask [B][S_q][S_k] (nonzero = visible).  With a
// mask and mask_tiles (prefill_mask_tiles_bytes bytes), a pass over the mask
// forms every row block's key-tile bitmaps there first; mask_tiles null: each
// workgroup scans its own mask rows.
hipError_t launch_prefill_masked(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S_q, int S_k, int h_q, int n_kv, int D, int causal, const int32_t* kv_lens,
                                 const uint8_t* mask, uint32_t* mask_tiles, int n_cu, hipStream_t stream);
// fp8 (e4m3) q/k/v with per-(batch, head) descale factors, d = 64 or 128, general masks.
hipError_t launch_prefill_fp8(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                              int S_q, int S_k, int h_q, int n_kv, int D, int causal, const int32_t* kv_lens,
                              const uint8_t* mask, const float* q_descale, const float* k_descale,
                              const float* v_descale, uint32_t* mask_tiles, int n_cu, hipStream_t stream);
// Bytes of the key-tile bitmaps of all row blocks (see launch_prefill_masked).
size_t prefill_mask_tiles_bytes(int B, int S_q, int S_k, int h_q, int n_kv);

// Read-only stream over `bytes` (a multiple of 16) at `buf`: the measured HBM
// read ceiling.  One workgroup of 512 threads per compute unit.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t stream);

}  // namespace gqa
