// Internal launch interface between the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* seq_lens;
  float* part_o;   // [B][h_q][n_split][D]
  float* part_ml;  // [B][h_q][n_split][2]: running max (log2 domain), running sum
  float qk_scale_log2;
  int h_q, n_kv, S_max, chunk, n_split, n_hchunk, heads_per_chunk;
};

// kind: 0 = float32 Q/K/V, 1 = bf16 Q/K/V, 2 = bf16 Q with e4m3 K/V.
// hb: 16-head blocks per workgroup on the matrix-core paths (1 or 2).
hipError_t launch_decode_split(const DecodeArgs& a, int B, int D, int hb, int kind, hipStream_t stream);
hipError_t launch_decode_combine(const float* part_o, const float* part_ml, const int32_t* seq_lens, void* out,
                                 bool out_bf16, int B, int h_q, int S_max, int D, int chunk, int n_split,
                                 hipStream_t stream);
hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S, int h_q, int n_kv, int D, hipStream_t stream);

}  // namespace gqa
