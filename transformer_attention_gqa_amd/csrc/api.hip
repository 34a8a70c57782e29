// Host side of libgqa_attn.so: argument checks, the sequence-split plan, and
// kernel launches.  Every check happens before any HIP call; nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "gqa_attn.h"
#include "gqa_launch.h"

namespace gqa {

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr int kWaves = 4;
constexpr int kTileMfma = 32;
constexpr int kTileF32 = 64;
// Split heuristic: aim for this many workgroups over the whole call, but keep
// each chunk long enough that the per-chunk partial (heads x (d+2) floats,
// written once and read once) stays a small fraction of the chunk's K/V bytes.
constexpr long kTargetWorkgroups = 1024;
constexpr double kMaxPartialFraction = 1.0 / 32.0;

thread_local char g_last_hip_error[256] = "";

void record_hip_error(hipError_t e) {
  const char* msg = hipGetErrorString(e);
  std::strncpy(g_last_hip_error, msg ? msg : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct DecodePlan {
  int kind;             // 0 f32, 1 bf16 K/V, 2 fp8 K/V
  int tile;             // tokens per wave tile
  int hb;               // 16-head blocks per workgroup (matrix-core paths)
  int heads_per_chunk;  // query heads one workgroup serves
  int n_hchunk;         // workgroups along the head axis of one group
  int chunk;            // tokens per sequence chunk (multiple of tile)
  int n_split;          // chunks covering S_max
};

gqa_status validate_decode_desc(const gqa_decode_desc* d) {
  if (!d) return GQA_ERR_NULL;
  if (d->B <= 0 || d->h_q <= 0 || d->n_kv <= 0 || d->S_max <= 0 || d->d_h <= 0 || d->n_split < 0)
    return GQA_ERR_SHAPE;
  if (d->h_q % d->n_kv != 0) return GQA_ERR_SHAPE;
  if (d->d_h != 64 && d->d_h != 128) return GQA_ERR_SHAPE;
  const bool ok = (d->q_dtype == GQA_F32 && d->kv_dtype == GQA_F32) ||
                  (d->q_dtype == GQA_BF16 && d->kv_dtype == GQA_BF16) ||
                  (d->q_dtype == GQA_BF16 && d->kv_dtype == GQA_FP8_E4M3);
  if (!ok) return GQA_ERR_DTYPE;
  // index arithmetic inside the kernels: B*h_q rows, B*n_kv*S_max cache rows
  if ((int64_t)d->B * d->h_q > (int64_t)1 << 30) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->n_kv * d->S_max > (int64_t)1 << 40) return GQA_ERR_SHAPE;
  return GQA_OK;
}

DecodePlan plan_decode(const gqa_decode_desc* d) {
  DecodePlan p{};
  const int G = d->h_q / d->n_kv;
  p.kind = d->kv_dtype == GQA_F32 ? 0 : (d->kv_dtype == GQA_BF16 ? 1 : 2);
  if (p.kind == 0) {
    p.tile = kTileF32;
    p.hb = 1;
    p.heads_per_chunk = 16;
  } else {
    p.tile = kTileMfma;
    p.hb = G > 16 ? 2 : 1;
    p.heads_per_chunk = 16 * p.hb;
  }
  p.n_hchunk = (G + p.heads_per_chunk - 1) / p.heads_per_chunk;
  const int heads_eff = G < p.heads_per_chunk ? G : p.heads_per_chunk;
  const long max_tiles = (d->S_max + p.tile - 1) / p.tile;
  long n_split;
  if (d->n_split > 0) {
    n_split = d->n_split;
  } else {
    const long units = (long)d->B * d->n_kv * p.n_hchunk;
    n_split = (kTargetWorkgroups + units - 1) / units;
    // floor on the chunk length from the partial-traffic bound
    const int elem = p.kind == 0 ? 4 : (p.kind == 1 ? 2 : 1);
    const double partial_bytes = (double)heads_eff * (d->d_h + 2) * 4.0 * 2.0;  // written + read
    const double bytes_per_token = 2.0 * d->d_h * elem;
    long min_chunk = (long)(partial_bytes / (kMaxPartialFraction * bytes_per_token));
    const long wave_round = (long)kWaves * p.tile;
    min_chunk = (min_chunk + wave_round - 1) / wave_round * wave_round;
    const long max_split_by_len = (d->S_max + min_chunk - 1) / min_chunk;
    if (n_split > max_split_by_len) n_split = max_split_by_len;
  }
  if (n_split < 1) n_split = 1;
  if (n_split > max_tiles) n_split = max_tiles;
  long chunk_tiles = (max_tiles + n_split - 1) / n_split;
  p.chunk = (int)(chunk_tiles * p.tile);
  p.n_split = (int)((d->S_max + p.chunk - 1) / p.chunk);
  return p;
}

size_t workspace_layout(const gqa_decode_desc* d, const DecodePlan& p, size_t* ml_offset) {
  const size_t rows = (size_t)d->B * d->h_q * p.n_split;
  const size_t o_bytes = rows * d->d_h * sizeof(float);
  const size_t ml_off = (o_bytes + 255) & ~(size_t)255;
  if (ml_offset) *ml_offset = ml_off;
  return ml_off + rows * 2 * sizeof(float);
}

gqa_status check_decode_ptrs(const gqa_decode_desc* d, const void* q, const void* k, const void* v,
                             const float* ks, const float* vs, const int32_t* seq_lens) {
  if (!q || !k || !v || !seq_lens) return GQA_ERR_NULL;
  if (d->kv_dtype == GQA_FP8_E4M3 && (!ks || !vs)) return GQA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  if (d->kv_dtype == GQA_FP8_E4M3 && (misaligned(ks) || misaligned(vs))) return GQA_ERR_ALIGN;
  return GQA_OK;
}

gqa_status do_partials(const gqa_decode_desc* d, const DecodePlan& p, const void* q, const void* k, const void* v,
                       const float* ks, const float* vs, const int32_t* seq_lens, float scale, void* ws,
                       hipStream_t stream) {
  size_t ml_off = 0;
  workspace_layout(d, p, &ml_off);
  DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_scale = ks;
  a.v_scale = vs;
  a.seq_lens = seq_lens;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ml_off);
  a.qk_scale_log2 = (float)((double)scale * kLog2e);
  a.h_q = d->h_q;
  a.n_kv = d->n_kv;
  a.S_max = d->S_max;
  a.chunk = p.chunk;
  a.n_split = p.n_split;
  a.n_hchunk = p.n_hchunk;
  a.heads_per_chunk = p.heads_per_chunk;
  hipError_t e = launch_decode_split(a, d->B, d->d_h, p.hb, p.kind, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

gqa_status do_combine(const gqa_decode_desc* d, const DecodePlan& p, const int32_t* seq_lens, const void* ws,
                      void* out, hipStream_t stream) {
  size_t ml_off = 0;
  workspace_layout(d, p, &ml_off);
  const float* part_o = static_cast<const float*>(ws);
  const float* part_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + ml_off);
  hipError_t e = launch_decode_combine(part_o, part_ml, seq_lens, out, d->q_dtype == GQA_BF16, d->B, d->h_q,
                                       d->S_max, d->d_h, p.chunk, p.n_split, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

}  // namespace
}  // namespace gqa

using namespace gqa;

extern "C" {

int32_t attn_decode_num_splits(const gqa_decode_desc* d) {
  if (validate_decode_desc(d) != GQA_OK) return -1;
  return plan_decode(d).n_split;
}

size_t attn_decode_workspace_bytes(const gqa_decode_desc* d) {
  if (validate_decode_desc(d) != GQA_OK) return 0;
  return workspace_layout(d, plan_decode(d), nullptr);
}

gqa_status attn_decode_partials(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = validate_decode_desc(d);
  if (st != GQA_OK) return st;
  st = check_decode_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, seq_lens);
  if (st != GQA_OK) return st;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p, nullptr)) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  return do_partials(d, p, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, workspace, stream);
}

gqa_status attn_decode_combine(const gqa_decode_desc* d, const int32_t* seq_lens, const void* workspace,
                               size_t workspace_bytes, void* out, hipStream_t stream) {
  gqa_status st = validate_decode_desc(d);
  if (st != GQA_OK) return st;
  if (!seq_lens || !out) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p, nullptr)) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  return do_combine(d, p, seq_lens, workspace, out, stream);
}

gqa_status attn_decode(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = validate_decode_desc(d);
  if (st != GQA_OK) return st;
  st = check_decode_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, seq_lens);
  if (st != GQA_OK) return st;
  if (!out) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p, nullptr)) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  st = do_partials(d, p, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, workspace, stream);
  if (st != GQA_OK) return st;
  return do_combine(d, p, seq_lens, workspace, out, stream);
}

gqa_status attn_prefill_causal(const gqa_prefill_desc* d, const void* q, const void* k, const void* v, float scale,
                               void* out, hipStream_t stream) {
  if (!d) return GQA_ERR_NULL;
  if (d->B <= 0 || d->S <= 0 || d->h_q <= 0 || d->n_kv <= 0 || d->d_h <= 0) return GQA_ERR_SHAPE;
  if (d->h_q % d->n_kv != 0) return GQA_ERR_SHAPE;
  if (d->d_h != 64 && d->d_h != 128) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->S * d->h_q > (int64_t)1 << 31) return GQA_ERR_SHAPE;
  if (d->dtype != GQA_BF16) return GQA_ERR_DTYPE;
  if (!q || !k || !v || !out) return GQA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return GQA_ERR_ALIGN;
  hipError_t e = launch_prefill_causal(q, k, v, out, (float)((double)scale * kLog2e), d->B, d->S, d->h_q, d->n_kv,
                                       d->d_h, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL: return "GQA_ERR_NULL: a required pointer is NULL";
    case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE: invalid dimensions";
    case GQA_ERR_DTYPE: return "GQA_ERR_DTYPE: unsupported element types";
    case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN: pointer not 16-byte aligned";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: HIP launch failed";
  }
  return "unknown gqa_status";
}

const char* gqa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
