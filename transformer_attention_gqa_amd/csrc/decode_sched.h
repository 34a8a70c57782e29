// Balanced split-sequence schedule shared by the decode kernels.
//
// The tiles of every (sequence, kv-head, head chunk) slab are concatenated
// into one range [0, T); workgroup w of W takes [w*T/W, (w+1)*T/W), which may
// cross slab boundaries ("segments").  The helpers below find T and the slab
// of a tile with wave-level scans over seq_lens.
#pragma once

#include "gqa_device.h"

namespace gqa {

// ------------------------------------------------------------------------
// Balanced schedule helpers.  All are wave-uniform: every lane returns the
// same values, so every wave of a workgroup can evaluate them on its own.
// Sequences are visited 64 at a time, one per lane.
// ------------------------------------------------------------------------
__device__ __forceinline__ int clamp_len(int L, int S_max) { return min(max(L, 0), S_max); }

__device__ __forceinline__ int seq_tiles(const int32_t* seq_lens, int b, int S_max, int tile) {
  return (clamp_len(seq_lens[b], S_max) + tile - 1) / tile;
}

// Wave-uniform values produced by cross-lane operations live in VGPRs unless
// told otherwise; these move them to scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform(long long v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes in registers (every lane active):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then lane 15 of a row
// into the next row and lane 31 into the upper half.  Each step is one VALU
// operation, against one LDS round trip per step for a shuffle-based scan;
// the schedule's scans sit between the length load and the first cache load.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  const int rl = lane & 15;
  int t = __builtin_amdgcn_mov_dpp(x, 0x111, 0xf, 0xf, false);  // row_shr:1
  if (rl >= 1) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x112, 0xf, 0xf, false);  // row_shr:2
  if (rl >= 2) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x114, 0xf, 0xf, false);  // row_shr:4
  if (rl >= 4) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x118, 0xf, 0xf, false);  // row_shr:8
  if (rl >= 8) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x142, 0xf, 0xf, false);  // row_bcast:15
  if ((lane & 31) >= 16) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x143, 0xf, 0xf, false);  // row_bcast:31
  if (lane >= 32) x += t;
  return x;
}

// Value of x in lane `src` (wave-uniform), as a scalar.
__device__ __forceinline__ int lane_value(int x, int src) { return __builtin_amdgcn_readlane(x, src); }

// Tile counts up to B * spb * ceil(S_max / tile) fit 32-bit integers (every
// practical cache): the scans and divisions of the schedule then run on
// 32-bit values, half the cross-lane traffic of the 64-bit forms and no
// emulated 64-bit division, which matters at kernel start where the first
// cache loads wait for the schedule.
__device__ __forceinline__ bool small_range(int B, int S_max, int tile, int spb) {
  return (long long)B * spb * ((S_max + tile - 1) / tile) < (1LL << 31);
}

// The range [0, T) cut into W workgroup ranges: workgroup w takes
// [lo(w), lo(w + 1)) with lo(w) = floor(w T / W), and tile t belongs to
// owner(t) = floor(((t + 1) W - 1) / T), the last w with lo(w) <= t.  For
// T < 2^31, T = qW + r gives lo(w) = wq + floor(wr / W) in 32-bit integers,
// and owner starts from a float estimate (off by at most one) and steps to
// the exact workgroup.
struct TileRanges {
  long long T;
  int W, q, r;
  bool small;
  __device__ __forceinline__ TileRanges(long long T_, int W_) : T(T_), W(W_) {
    small = T_ < (1LL << 31) && W_ <= 32768;  // w q <= T and w r < W^2 stay below 2^31
    q = small ? (int)T_ / W_ : 0;
    r = small ? (int)T_ - q * W_ : 0;
  }
  __device__ __forceinline__ long long lo(int w) const {
    if (__builtin_expect(small, 1)) return (long long)(w * q + (w * r) / W);
    return (long long)w * T / W;
  }
  __device__ __forceinline__ long long owner(long long t) const {
    if (__builtin_expect(!small, 0)) return ((t + 1) * W - 1) / T;
    int w = (int)(((float)(t + 1) * (float)W - 1.0f) / (float)T);
    w = min(max(w, 0), W - 1);
    while (w + 1 < W && lo(w + 1) <= t) ++w;
    while (w > 0 && lo(w) > t) --w;
    return w;
  }
};

// Tiles of all slabs of sequences 0 .. n-1 (n = B gives the total T).
static __device__ long long tiles_before(const int32_t* seq_lens, int n, int S_max, int tile, int spb, int lane) {
  long long acc = 0;
  for (int base = 0; base < n; base += 64) {
    const int b = base + lane;
    acc += wave_sum_ll(b < n ? (long long)seq_tiles(seq_lens, b, S_max, tile) * spb : 0);
  }
  return acc;
}

// (local / nt, local % nt) for a tile offset inside one sequence's slabs;
// 32-bit division whenever the offset allows it.
__device__ __forceinline__ void split_local(long long local, int nt, int& slab, int& tile0) {
  if (__builtin_expect(local < (1LL << 31), 1)) {
    slab = (int)local / nt;
    tile0 = (int)local - slab * nt;
  } else {
    slab = (int)(local / nt);
    tile0 = (int)(local - (long long)slab * nt);
  }
}

// Lengths of sequences 0..63 held one per lane (B <= 64, the common case):
// the schedule then needs a single load of seq_lens per wave.
struct LaneLens {
  int len;    // clamped length of sequence `lane` (0 past B)
  bool fits;  // B <= 64
};

__device__ __forceinline__ LaneLens load_lane_lens(const int32_t* seq_lens, int B, int S_max, int lane) {
  LaneLens r;
  r.fits = B <= 64;
  r.len = (r.fits && lane < B) ? clamp_len(seq_lens[lane], S_max) : 0;
  return r;
}

__device__ __forceinline__ long long total_tiles_cached(const LaneLens& ll, const int32_t* seq_lens, int B, int S_max,
                                                        int tile, int spb, int lane) {
  if (__builtin_expect(!ll.fits, 0)) return tiles_before(seq_lens, B, S_max, tile, spb, lane);
  if (__builtin_expect(small_range(B, S_max, tile, spb), 1)) return lane_value(wave_incl_scan((ll.len + tile - 1) / tile * spb, lane), 63);
  return wave_sum_ll((long long)((ll.len + tile - 1) / tile) * spb);
}

// The sequence whose slabs contain global tile t (0 <= t < T): its index, the
// global index of its first tile, its tiles per slab and its clamped length.
static __device__ void locate_tile(const int32_t* seq_lens, int B, int S_max, int tile, int spb, long long t, int lane,
                            int& b_out, long long& base_out, int& nt_out, int& len_out) {
  long long acc = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int len = b < B ? clamp_len(seq_lens[b], S_max) : 0;
    const int nt = (len + tile - 1) / tile;
    long long incl = (long long)nt * spb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    const long long tot = __shfl(incl, 63, 64);
    if (t < acc + tot) {
      const unsigned long long mask = __ballot(acc + incl > t);
      const int first = __ffsll((long long)mask) - 1;
      b_out = base + first;
      nt_out = __shfl(nt, first, 64);
      len_out = __shfl(len, first, 64);
      base_out = acc + __shfl(incl, first, 64) - (long long)nt_out * spb;
      return;
    }
    acc += tot;
  }
  b_out = B;
  base_out = acc;
  nt_out = 0;
  len_out = 0;
}

static __device__ void locate_tile_cached(const LaneLens& ll, const int32_t* seq_lens, int B, int S_max, int tile, int spb,
                                   long long t, int lane, int& b_out, long long& base_out, int& nt_out, int& len_out) {
  if (__builtin_expect(!ll.fits, 0)) {
    locate_tile(seq_lens, B, S_max, tile, spb, t, lane, b_out, base_out, nt_out, len_out);
    return;
  }
  const int nt = (ll.len + tile - 1) / tile;
  if (__builtin_expect(small_range(B, S_max, tile, spb), 1)) {
    const int incl = wave_incl_scan(nt * spb, lane);
    // t < T: some lane's prefix exceeds t; the clamp keeps the index in range regardless
    const int first = min(max(__builtin_amdgcn_readfirstlane(__ffsll((long long)__ballot(incl > (int)t)) - 1), 0), B - 1);
    b_out = first;
    nt_out = lane_value(nt, first);
    len_out = lane_value(ll.len, first);
    base_out = lane_value(incl, first) - nt_out * spb;
    return;
  }
  long long incl = (long long)nt * spb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  const unsigned long long mask = __ballot(incl > t);
  const int first = __ffsll((long long)mask) - 1;
  b_out = first;
  nt_out = __shfl(nt, first, 64);
  len_out = __shfl(ll.len, first, 64);
  base_out = __shfl(incl, first, 64) - (long long)nt_out * spb;
}

// For sequence b: the tiles of all slabs of all sequences (T), those of the
// sequences before b, and b's tiles per slab -- one length load per lane when
// B <= 64.
static __device__ void slab_position(const LaneLens& ll, const int32_t* seq_lens, int B, int S_max, int tile,
                                     int spb, int b, int lane, long long& T, long long& before_b, int& nt_b) {
  if (__builtin_expect(!ll.fits, 0)) {
    T = tiles_before(seq_lens, B, S_max, tile, spb, lane);
    before_b = tiles_before(seq_lens, b, S_max, tile, spb, lane);
    nt_b = seq_tiles(seq_lens, b, S_max, tile);
    return;
  }
  const int nt = (ll.len + tile - 1) / tile;
  if (__builtin_expect(small_range(B, S_max, tile, spb), 1)) {
    const int incl = wave_incl_scan(nt * spb, lane);
    T = lane_value(incl, 63);
    before_b = b > 0 ? lane_value(incl, b - 1) : 0;
    nt_b = lane_value(nt, b);
    return;
  }
  nt_b = __shfl(nt, b, 64);
  const long long own = (long long)nt * spb;
  T = wave_sum_ll(own);
  before_b = wave_sum_ll(lane < b ? own : 0);
}

}  // namespace gqa
