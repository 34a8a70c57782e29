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

// Tiles of all slabs of sequences 0 .. n-1 (n = B gives the total T).
static __device__ long long tiles_before(const int32_t* seq_lens, int n, int S_max, int tile, int spb, int lane) {
  long long acc = 0;
  for (int base = 0; base < n; base += 64) {
    const int b = base + lane;
    acc += wave_sum_ll(b < n ? (long long)seq_tiles(seq_lens, b, S_max, tile) * spb : 0);
  }
  return acc;
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
  if (!ll.fits) return tiles_before(seq_lens, B, S_max, tile, spb, lane);
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
  if (!ll.fits) {
    locate_tile(seq_lens, B, S_max, tile, spb, t, lane, b_out, base_out, nt_out, len_out);
    return;
  }
  const int nt = (ll.len + tile - 1) / tile;
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
  if (!ll.fits) {
    T = tiles_before(seq_lens, B, S_max, tile, spb, lane);
    before_b = tiles_before(seq_lens, b, S_max, tile, spb, lane);
    nt_b = seq_tiles(seq_lens, b, S_max, tile);
    return;
  }
  const int nt = (ll.len + tile - 1) / tile;
  const long long own = (long long)nt * spb;
  T = wave_sum_ll(own);
  before_b = wave_sum_ll(lane < b ? own : 0);
  nt_b = __shfl(nt, b, 64);
}

}  // namespace gqa
