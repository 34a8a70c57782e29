// Host side of libgqa_attn.so: argument checks, the sequence-split plan, and
// kernel launches.  Every check happens before any HIP call; nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gqa_attn.h"
#include "gqa_launch.h"

namespace gqa {

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr int kTileMfma = 32;
constexpr int kTileF32 = 64;
// Default number of decode workgroups: one per compute unit of the current
// device (each runs 8 wavefronts and owns an equal share of all key tiles);
// 256, a whole MI355X, when no device can be queried.
constexpr int kFallbackComputeUnits = 256;
constexpr long kMaxWorkgroups = 65536;
constexpr int kMaxDevices = 64;

thread_local char g_last_hip_error[256] = "";

void record_hip_error(hipError_t e) {
  const char* msg = hipGetErrorString(e);
  std::strncpy(g_last_hip_error, msg ? msg : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Compute units of the current device, queried once per device and cached
// (a device partitioned into fewer CUs gets a persistent grid of its own
// size).  The query enqueues nothing; if it fails (no device), the count of a
// whole MI355X is used and the error is cleared so that it cannot be taken
// for a launch failure later.
int device_compute_units() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kFallbackComputeUnits;
  }
  if (dev < kMaxDevices) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return kFallbackComputeUnits;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// scale * log2(e) as the kernels take it.  A scale so small that the product
// is not a normal float is raised to the smallest normal: the scores are then
// effectively zero either way, and a zero factor would turn the -inf of a
// hidden key into NaN.
float qk_scale_log2(float scale) { return fmaxf((float)((double)scale * kLog2e), FLT_MIN); }

// K/V element types that come with per-row scales
bool is_quantized(int32_t t) { return t == GQA_FP8_E4M3 || t == GQA_INT8 || t == GQA_INT4; }

// The kernels take the running max on unscaled scores, which needs scale > 0.
// A scale must be finite and >= 0: the kernels take the maximum of the
// unscaled scores, which needs scale >= 0 to be the maximum of the scaled ones.
bool bad_scale(float s) { return !(s >= 0.0f) || !(s < __builtin_huge_valf()); }

struct DecodePlan {
  int kind;             // 0 f32, 1 bf16 K/V, 2 fp8, 3 int8, 4 int4 K/V
  int tile;             // tokens per wave tile
  int hb;               // 16-head blocks per workgroup (matrix-core paths)
  int heads_per_chunk;  // query heads one workgroup serves at a time
  int n_hchunk;         // head chunks per K/V group
  long n_slabs;         // B * n_kv * n_hchunk
  int W;                // workgroups launched (balanced key ranges)
  int deterministic;    // static tile order inside a workgroup
};

gqa_status validate_decode_desc(const gqa_decode_desc* d) {
  if (!d) return GQA_ERR_NULL;
  if (d->B <= 0 || d->h_q <= 0 || d->n_kv <= 0 || d->S_max <= 0 || d->d_h <= 0 || d->n_split < 0)
    return GQA_ERR_SHAPE;
  if ((d->flags & ~GQA_DECODE_DETERMINISTIC) != 0) return GQA_ERR_VALUE;
  if (d->h_q % d->n_kv != 0) return GQA_ERR_SHAPE;
  if (d->d_h != 64 && d->d_h != 128) return GQA_ERR_SHAPE;
  const bool ok = (d->q_dtype == GQA_F32 && d->kv_dtype == GQA_F32) ||
                  (d->q_dtype == GQA_BF16 && (d->kv_dtype == GQA_BF16 || is_quantized(d->kv_dtype)));
  if (!ok) return GQA_ERR_DTYPE;
  // index arithmetic inside the kernels: B*h_q rows, B*n_kv*S_max cache rows
  if ((int64_t)d->B * d->h_q > (int64_t)1 << 30) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->n_kv * d->S_max > (int64_t)1 << 40) return GQA_ERR_SHAPE;
  if (d->S_max > (1 << 30)) return GQA_ERR_SHAPE;
  return GQA_OK;
}

DecodePlan plan_decode(const gqa_decode_desc* d) {
  DecodePlan p{};
  const int G = d->h_q / d->n_kv;
  switch (d->kv_dtype) {
    case GQA_F32: p.kind = 0; break;
    case GQA_BF16: p.kind = 1; break;
    case GQA_FP8_E4M3: p.kind = 2; break;
    case GQA_INT8: p.kind = 3; break;
    default: p.kind = 4; break;  // GQA_INT4
  }
  if (p.kind == 0) {
    p.tile = kTileF32;
    p.hb = 1;
    p.heads_per_chunk = 16;
  } else {
    p.hb = G > 16 ? 2 : 1;
    // int4 with one block of 16 heads schedules 64-token tiles (two register
    // halves per wave in the split kernel); the combine must use the same
    p.tile = p.kind == 4 && p.hb == 1 ? 2 * kTileMfma : kTileMfma;
    p.heads_per_chunk = 16 * p.hb;
  }
  p.n_hchunk = (G + p.heads_per_chunk - 1) / p.heads_per_chunk;
  p.n_slabs = (long)d->B * d->n_kv * p.n_hchunk;
  const long max_tiles = p.n_slabs * ((d->S_max + p.tile - 1) / p.tile);
  long W = d->n_split > 0 ? (long)d->n_split : device_compute_units();
  if (W > max_tiles) W = max_tiles;
  if (W > kMaxWorkgroups) W = kMaxWorkgroups;
  if (W < 1) W = 1;
  p.W = (int)W;
  p.deterministic = (d->flags & GQA_DECODE_DETERMINISTIC) != 0;
  return p;
}

// Workspace: [partial O][partial (m, l)], the second part starting on a
// 256-byte boundary.
struct WorkspaceLayout {
  size_t o_off, ml_off, total;
};

WorkspaceLayout workspace_layout(const gqa_decode_desc* d, const DecodePlan& p) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)(p.W + p.n_slabs) * p.heads_per_chunk;
  WorkspaceLayout l;
  l.o_off = 0;
  l.ml_off = up(rows * d->d_h * sizeof(float));
  l.total = l.ml_off + rows * 2 * sizeof(float);
  return l;
}

gqa_status check_decode_ptrs(const gqa_decode_desc* d, const void* q, const void* k, const void* v,
                             const float* ks, const float* vs, const int32_t* seq_lens) {
  if (!q || !k || !v || !seq_lens) return GQA_ERR_NULL;
  if (is_quantized(d->kv_dtype) && (!ks || !vs)) return GQA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  if (is_quantized(d->kv_dtype) && (misaligned(ks) || misaligned(vs))) return GQA_ERR_ALIGN;
  return GQA_OK;
}

// Paging of the cache for do_partials (block_table null: contiguous cache).
struct Paging {
  const int32_t* block_table = nullptr;
  int page_shift = 0, max_pages = 0, num_pages = 0;
};

gqa_status do_partials(const gqa_decode_desc* d, const DecodePlan& p, const void* q, const void* k, const void* v,
                       const float* ks, const float* vs, const int32_t* seq_lens, float scale, void* ws,
                       hipStream_t stream, const Paging& pg = Paging()) {
  const WorkspaceLayout wl = workspace_layout(d, p);
  DecodeArgs a;
  a.block_table = pg.block_table;
  a.page_shift = pg.page_shift;
  a.max_pages = pg.max_pages;
  a.num_pages = pg.num_pages;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_scale = ks;
  a.v_scale = vs;
  a.seq_lens = seq_lens;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.o_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.ml_off);
  a.qk_scale_log2 = qk_scale_log2(scale);
  a.B = d->B;
  a.h_q = d->h_q;
  a.n_kv = d->n_kv;
  a.S_max = d->S_max;
  a.n_hchunk = p.n_hchunk;
  a.heads_per_chunk = p.heads_per_chunk;
  a.deterministic = p.deterministic;
  hipError_t e = launch_decode_split(a, d->d_h, p.hb, p.kind, p.W, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

gqa_status do_combine(const gqa_decode_desc* d, const DecodePlan& p, const int32_t* seq_lens, const void* ws,
                      void* out, hipStream_t stream) {
  const WorkspaceLayout wl = workspace_layout(d, p);
  CombineArgs c;
  c.part_o = reinterpret_cast<const float*>(static_cast<const char*>(ws) + wl.o_off);
  c.part_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + wl.ml_off);
  c.seq_lens = seq_lens;
  c.out = out;
  c.B = d->B;
  c.h_q = d->h_q;
  c.n_kv = d->n_kv;
  c.S_max = d->S_max;
  c.n_hchunk = p.n_hchunk;
  c.heads_per_chunk = p.heads_per_chunk;
  c.tile = p.tile;
  c.W = p.W;
  hipError_t e = launch_decode_combine(c, d->d_h, d->q_dtype == GQA_BF16, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

// Paged decode: checks the paged descriptor and maps it onto the contiguous
// one (S_max = max_pages * page_size), which fixes the plan and workspace.
gqa_status paged_to_decode_desc(const gqa_paged_desc* pd, gqa_decode_desc* d, int* page_shift) {
  if (!pd) return GQA_ERR_NULL;
  const int ps = pd->page_size;
  if (ps < 32 || ps > (1 << 20) || (ps & (ps - 1)) != 0) return GQA_ERR_SHAPE;
  if (pd->num_pages <= 0 || pd->max_pages_per_seq <= 0) return GQA_ERR_SHAPE;
  if ((int64_t)pd->max_pages_per_seq * ps > (int64_t)1 << 30) return GQA_ERR_SHAPE;
  if ((int64_t)pd->B * pd->max_pages_per_seq > (int64_t)1 << 31) return GQA_ERR_SHAPE;
  if ((int64_t)pd->num_pages * pd->n_kv * ps > (int64_t)1 << 40) return GQA_ERR_SHAPE;
  *d = gqa_decode_desc{pd->B, pd->h_q, pd->n_kv, pd->max_pages_per_seq * ps, pd->d_h, pd->q_dtype, pd->kv_dtype,
                       pd->n_split, pd->flags};
  int sh = 0;
  while ((1 << sh) < ps) ++sh;
  *page_shift = sh;
  return validate_decode_desc(d);
}

// ---- absorbed latent-attention decode
struct MlaPlan {
  int hb;               // 32-head blocks per workgroup
  int heads_per_chunk;  // 32 * hb
  int n_hchunk;         // head chunks per sequence
  long n_slabs;         // B * n_hchunk
  int W;
};

gqa_status validate_mla_desc(const gqa_mla_desc* d) {
  if (!d) return GQA_ERR_NULL;
  if (d->B <= 0 || d->h_q <= 0 || d->S_max <= 0 || d->d_c <= 0 || d->n_split < 0) return GQA_ERR_SHAPE;
  if (d->d_c != 256 && d->d_c != 512) return GQA_ERR_SHAPE;
  if (d->dtype != GQA_BF16) return GQA_ERR_DTYPE;
  if ((int64_t)d->B * d->h_q > (int64_t)1 << 30) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->S_max > (int64_t)1 << 40) return GQA_ERR_SHAPE;
  if (d->S_max > (1 << 30)) return GQA_ERR_SHAPE;
  return GQA_OK;
}

MlaPlan plan_mla(const gqa_mla_desc* d) {
  MlaPlan p{};
  p.hb = d->h_q > 32 ? 2 : 1;
  p.heads_per_chunk = 32 * p.hb;
  p.n_hchunk = (d->h_q + p.heads_per_chunk - 1) / p.heads_per_chunk;
  p.n_slabs = (long)d->B * p.n_hchunk;
  const long max_tiles = p.n_slabs * ((d->S_max + kTileMfma - 1) / kTileMfma);
  long W = d->n_split > 0 ? (long)d->n_split : device_compute_units();
  if (W > max_tiles) W = max_tiles;
  if (W > kMaxWorkgroups) W = kMaxWorkgroups;
  if (W < 1) W = 1;
  p.W = (int)W;
  return p;
}

WorkspaceLayout mla_workspace_layout(const gqa_mla_desc* d, const MlaPlan& p) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)(p.W + p.n_slabs) * p.heads_per_chunk;
  WorkspaceLayout l;
  l.o_off = 0;
  l.ml_off = up(rows * d->d_c * sizeof(float));
  l.total = l.ml_off + rows * 2 * sizeof(float);
  return l;
}

// ---- scratch of attn_decode_noalloc: the split kernel's partial rows live in
// one file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy for the life of the process.  In host
// code `scratch` names a host-side stand-in, not device memory: kernels and
// copies take the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (null + status on
// failure).
gqa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    const hipError_t e = hipGetLastError();
    record_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
    return GQA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      (void)hipGetLastError();
      return GQA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace
}  // namespace gqa

using namespace gqa;

extern "C" {

int32_t attn_decode_num_splits(const gqa_decode_desc* d) {
  if (validate_decode_desc(d) != GQA_OK) return -1;
  return plan_decode(d).W;
}

size_t attn_decode_workspace_bytes(const gqa_decode_desc* d) {
  if (validate_decode_desc(d) != GQA_OK) return 0;
  return workspace_layout(d, plan_decode(d)).total;
}

gqa_status attn_decode_partials(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = validate_decode_desc(d);
  if (st != GQA_OK) return st;
  st = check_decode_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, seq_lens);
  if (st != GQA_OK) return st;
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p).total) return GQA_ERR_WORKSPACE;
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
  if (!workspace || workspace_bytes < workspace_layout(d, p).total) return GQA_ERR_WORKSPACE;
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
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p).total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  st = do_partials(d, p, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, workspace, stream);
  if (st != GQA_OK) return st;
  return do_combine(d, p, seq_lens, workspace, out, stream);
}

size_t attn_decode_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

gqa_status attn_decode_noalloc(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                               void* out, hipStream_t stream) {
  gqa_status st = validate_decode_desc(d);
  if (st != GQA_OK) return st;
  st = check_decode_ptrs(d, q, k_cache, v_cache, k_scale, v_scale, seq_lens);
  if (st != GQA_OK) return st;
  if (!out) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const DecodePlan p = plan_decode(d);
  if (workspace_layout(d, p).total > kScratchBytes) return GQA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != GQA_OK) return st;
  // the split kernel writes every partial the combine kernel reads, so the
  // scratch needs no clearing between calls
  st = do_partials(d, p, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, ws, stream);
  if (st != GQA_OK) return st;
  return do_combine(d, p, seq_lens, ws, out, stream);
}

int32_t attn_decode_paged_num_splits(const gqa_paged_desc* pd) {
  gqa_decode_desc d;
  int sh;
  if (paged_to_decode_desc(pd, &d, &sh) != GQA_OK) return -1;
  return plan_decode(&d).W;
}

size_t attn_decode_paged_workspace_bytes(const gqa_paged_desc* pd) {
  gqa_decode_desc d;
  int sh;
  if (paged_to_decode_desc(pd, &d, &sh) != GQA_OK) return 0;
  return workspace_layout(&d, plan_decode(&d)).total;
}

gqa_status attn_decode_paged(const gqa_paged_desc* pd, const void* q, const void* k_pages, const void* v_pages,
                             const float* k_scale_pages, const float* v_scale_pages, const int32_t* block_table,
                             const int32_t* seq_lens, float scale, void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  gqa_decode_desc dd;
  Paging pg;
  gqa_status st = paged_to_decode_desc(pd, &dd, &pg.page_shift);
  if (st != GQA_OK) return st;
  const gqa_decode_desc* d = &dd;
  st = check_decode_ptrs(d, q, k_pages, v_pages, k_scale_pages, v_scale_pages, seq_lens);
  if (st != GQA_OK) return st;
  if (!out || !block_table) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0) return GQA_ERR_ALIGN;
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const DecodePlan p = plan_decode(d);
  if (!workspace || workspace_bytes < workspace_layout(d, p).total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  pg.block_table = block_table;
  pg.max_pages = pd->max_pages_per_seq;
  pg.num_pages = pd->num_pages;
  st = do_partials(d, p, q, k_pages, v_pages, k_scale_pages, v_scale_pages, seq_lens, scale, workspace, stream, pg);
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
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  hipError_t e = launch_prefill_causal(q, k, v, out, qk_scale_log2(scale), d->B, d->S, d->h_q, d->n_kv, d->d_h,
                                       device_compute_units(), stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

int32_t attn_decode_mla_num_splits(const gqa_mla_desc* d) {
  if (validate_mla_desc(d) != GQA_OK) return -1;
  return plan_mla(d).W;
}

size_t attn_decode_mla_workspace_bytes(const gqa_mla_desc* d) {
  if (validate_mla_desc(d) != GQA_OK) return 0;
  return mla_workspace_layout(d, plan_mla(d)).total;
}

gqa_status attn_decode_mla_partials(const gqa_mla_desc* d, const void* q_abs, const void* c_kv,
                                    const int32_t* seq_lens, float scale, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  gqa_status st = validate_mla_desc(d);
  if (st != GQA_OK) return st;
  if (!q_abs || !c_kv || !seq_lens) return GQA_ERR_NULL;
  if (misaligned(q_abs) || misaligned(c_kv)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const MlaPlan p = plan_mla(d);
  const WorkspaceLayout wl = mla_workspace_layout(d, p);
  if (!workspace || workspace_bytes < wl.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  MlaArgs a;
  a.q = q_abs;
  a.c = c_kv;
  a.seq_lens = seq_lens;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  a.qk_scale_log2 = qk_scale_log2(scale);
  a.B = d->B;
  a.h_q = d->h_q;
  a.S_max = d->S_max;
  a.n_hchunk = p.n_hchunk;
  a.heads_per_chunk = p.heads_per_chunk;
  const hipError_t e = launch_mla_decode_split(a, d->d_c, p.hb, p.W, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

gqa_status attn_decode_mla_combine(const gqa_mla_desc* d, const int32_t* seq_lens, const void* workspace,
                                   size_t workspace_bytes, void* out, hipStream_t stream) {
  gqa_status st = validate_mla_desc(d);
  if (st != GQA_OK) return st;
  if (!seq_lens || !out) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  const MlaPlan p = plan_mla(d);
  const WorkspaceLayout wl = mla_workspace_layout(d, p);
  if (!workspace || workspace_bytes < wl.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  // the GQA combine with one K/V head: slab (b, hc) merges into heads
  // hc * heads_per_chunk ... of sequence b
  CombineArgs c;
  c.part_o = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + wl.o_off);
  c.part_ml = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + wl.ml_off);
  c.seq_lens = seq_lens;
  c.out = out;
  c.B = d->B;
  c.h_q = d->h_q;
  c.n_kv = 1;
  c.S_max = d->S_max;
  c.n_hchunk = p.n_hchunk;
  c.heads_per_chunk = p.heads_per_chunk;
  c.tile = kTileMfma;
  c.W = p.W;
  const hipError_t e = launch_decode_combine(c, d->d_c, true, stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

gqa_status attn_decode_mla(const gqa_mla_desc* d, const void* q_abs, const void* c_kv, const int32_t* seq_lens,
                           float scale, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = validate_mla_desc(d);
  if (st != GQA_OK) return st;
  if (!out) return GQA_ERR_NULL;
  if (misaligned(out)) return GQA_ERR_ALIGN;
  st = attn_decode_mla_partials(d, q_abs, c_kv, seq_lens, scale, workspace, workspace_bytes, stream);
  if (st != GQA_OK) return st;
  return attn_decode_mla_combine(d, seq_lens, workspace, workspace_bytes, out, stream);
}

namespace {

// Shape checks of a general-mask prefill descriptor (host only).
gqa_status check_attn_desc(const gqa_attn_desc* d, bool has_mask) {
  if (!d) return GQA_ERR_NULL;
  if (d->B <= 0 || d->S_q <= 0 || d->S_k <= 0 || d->h_q <= 0 || d->n_kv <= 0 || d->d_h <= 0) return GQA_ERR_SHAPE;
  if (d->h_q % d->n_kv != 0) return GQA_ERR_SHAPE;
  if (d->d_h != 64 && d->d_h != 128) return GQA_ERR_SHAPE;
  if (d->causal != 0 && d->causal != 1) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->S_q * d->h_q > (int64_t)1 << 31) return GQA_ERR_SHAPE;
  if ((int64_t)d->B * d->S_k * d->n_kv > (int64_t)1 << 31) return GQA_ERR_SHAPE;
  // 4-key mask words; a workgroup's mask rows (up to 256) within a 31-bit buffer range
  if (has_mask && (d->S_k % 4 != 0 || d->S_k > (1 << 23))) return GQA_ERR_SHAPE;
  if (d->dtype != GQA_BF16 && d->dtype != GQA_FP8_E4M3) return GQA_ERR_DTYPE;
  return GQA_OK;
}

gqa_status prefill_general(const gqa_attn_desc* d, const void* q, const void* k, const void* v,
                           const float* q_descale, const float* k_descale, const float* v_descale,
                           const int32_t* kv_lens, const uint8_t* mask, float scale, void* out, void* workspace,
                           size_t workspace_bytes, bool with_workspace, hipStream_t stream) {
  gqa_status st = check_attn_desc(d, mask != nullptr);
  if (st != GQA_OK) return st;
  const bool fp8 = d->dtype == GQA_FP8_E4M3;
  if (!fp8 && (q_descale || k_descale || v_descale)) return GQA_ERR_DTYPE;
  if (!q || !k || !v || !out) return GQA_ERR_NULL;
  if (fp8 && (!q_descale || !k_descale || !v_descale)) return GQA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(mask)) return GQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0) return GQA_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(q_descale) | reinterpret_cast<uintptr_t>(k_descale) |
        reinterpret_cast<uintptr_t>(v_descale)) & 3u) != 0)
    return GQA_ERR_ALIGN;
  uint32_t* mask_tiles = nullptr;
  if (with_workspace && mask) {
    if (!workspace || workspace_bytes < prefill_mask_tiles_bytes(d->B, d->S_q, d->S_k, d->h_q, d->n_kv))
      return GQA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GQA_ERR_ALIGN;
    mask_tiles = static_cast<uint32_t*>(workspace);
  }
  if (bad_scale(scale)) return GQA_ERR_VALUE;
  const float sl2 = qk_scale_log2(scale);
  const hipError_t e =
      fp8 ? launch_prefill_fp8(q, k, v, out, sl2, d->B, d->S_q, d->S_k, d->h_q, d->n_kv, d->d_h, d->causal, kv_lens, mask,
                               q_descale, k_descale, v_descale, mask_tiles, device_compute_units(), stream)
          : launch_prefill_masked(q, k, v, out, sl2, d->B, d->S_q, d->S_k, d->h_q, d->n_kv, d->d_h, d->causal,
                                  kv_lens, mask, mask_tiles, device_compute_units(), stream);
  if (e != hipSuccess) {
    record_hip_error(e);
    return GQA_ERR_HIP;
  }
  return GQA_OK;
}

}  // namespace

gqa_status attn_prefill(const gqa_attn_desc* d, const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, const float* v_descale, const int32_t* kv_lens, const uint8_t* mask,
                        float scale, void* out, hipStream_t stream) {
  return prefill_general(d, q, k, v, q_descale, k_descale, v_descale, kv_lens, mask, scale, out, nullptr, 0, false,
                         stream);
}

gqa_status attn_prefill_ws(const gqa_attn_desc* d, const void* q, const void* k, const void* v,
                           const float* q_descale, const float* k_descale, const float* v_descale,
                           const int32_t* kv_lens, const uint8_t* mask, float scale, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return prefill_general(d, q, k, v, q_descale, k_descale, v_descale, kv_lens, mask, scale, out, workspace,
                         workspace_bytes, true, stream);
}

size_t attn_prefill_workspace_bytes(const gqa_attn_desc* d) {
  if (check_attn_desc(d, false) != GQA_OK) return 0;
  return prefill_mask_tiles_bytes(d->B, d->S_q, d->S_k, d->h_q, d->n_kv);
}

gqa_status gqa_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return GQA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return GQA_ERR_SHAPE;
  if (misaligned(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return GQA_ERR_ALIGN;
  const hipError_t e = launch_stream_read(buf, bytes, sink, device_compute_units(), stream);
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
    case GQA_ERR_VALUE: return "GQA_ERR_VALUE: scale not finite and >= 0, or unknown flag bits";
    case GQA_ERR_SCRATCH:
      return "GQA_ERR_SCRATCH: the call needs more partial rows than the library's static scratch holds";
  }
  return "unknown gqa_status";
}

const char* gqa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
