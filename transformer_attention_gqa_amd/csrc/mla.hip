// Absorbed multi-head latent attention decode (split kernel; the combine is
// the decode combine kernel).
//
// "Evolution of AI Attention Mechanisms", section "Generation 3: MLA": the
// cache holds one latent row c_kv (d_c values) per token, and with the
// absorption step every query head attends in the latent space,
//     o_c,h = softmax(scale * q_abs,h . c_kv^T) c_kv,
// so the latent rows are the keys and the values of one head shared by all
// h query heads.  A token costs d_c * 2 bytes, read once for both products.
//
// Work decomposition (MI355X): the same persistent balanced schedule as the
// GQA decode (slabs of one sequence and one chunk of up to 64 heads, all
// heads of a chunk in one workgroup).  The 8 wavefronts of a workgroup share
// each 32-token tile:
//  * wave w loads the latent slice [w * d_c / 8, (w + 1) * d_c / 8) of every
//    row of the tile (a 128-byte piece at d_c = 512) and writes it into the
//    workgroup's LDS copy of the tile (three tiles resident: the one in use
//    and the next two);
//  * the scores S^T[token][head] of the tile are cut into 16-token x 16-head
//    blocks on v_mfma_f32_16x16x32_bf16; with fewer blocks than waves (32
//    heads give 4) each block's latent width is split over 8 / blocks waves.
//    The (partial) blocks go to LDS and, after one barrier, every wave reads
//    the scores of all heads, summing the partials, and runs the same online
//    softmax;
//  * the weighted sum O^T[latent][head] += C^T P^T runs on the wave's own
//    latent slice (v_mfma_f32_32x32x16_bf16), so a wave's accumulator holds
//    d_c / 8 latent values of every head and the partials need no merge
//    across waves.
#include <type_traits>

#include "decode_sched.h"
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kMlaTile = 32;   // tokens per tile
constexpr int kMlaWaves = 8;   // wavefronts per workgroup
constexpr float kMlaSlack = 8.0f;  // log2 units the running max may lag the true max
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;

// The tiles of one (sequence, head chunk) slab that a workgroup's range covers.
struct MlaSegment {
  int b, hc;           // sequence, head chunk
  int ntile;           // tiles of the segment
  int t_begin, t_end;  // token range [t_begin, t_end)
  long long slot;      // partial slot (workgroup + slab)
};

__device__ __forceinline__ MlaSegment mla_segment(const MlaArgs& a, const LaneLens& ll, long long t, long long hi,
                                                  int w, int lane) {
  int b, nt, L;
  long long base;
  locate_tile_cached(ll, a.seq_lens, a.B, a.S_max, kMlaTile, a.n_hchunk, t, lane, b, base, nt, L);
  b = uniform(b);
  nt = uniform(nt);
  L = uniform(L);
  base = uniform(base);
  int hc, tile0;
  split_local(t - base, nt, hc, tile0);
  MlaSegment s;
  s.b = b;
  s.hc = hc;
  s.ntile = (int)min(hi - t, (long long)(nt - tile0));
  s.t_begin = tile0 * kMlaTile;
  s.t_end = min((tile0 + s.ntile) * kMlaTile, L);
  s.slot = w + (long long)b * a.n_hchunk + hc;
  return s;
}

template <int D, int HB>
__global__ __launch_bounds__(kMlaWaves * 64) void gqa_mla_decode_split(MlaArgs a) {
  constexpr int NW = kMlaWaves;
  constexpr int DS = D / NW;          // latent values per wave (weighted sum, loads)
  constexpr int ROWB = 2 * D;         // bytes of a token row
  constexpr int HPC = 32 * HB;        // query heads per chunk
  constexpr int NT = DS / 32;         // 32-wide latent tiles of the wave's weighted sum
  constexpr int NBLK = 2 * (HPC / 16);  // score blocks: 2 token halves x HPC/16 head groups
  constexpr int KSPLIT = NW / NBLK;   // waves per block, each over 1/KSPLIT of the latent width
  constexpr int KQ = D / 32 / KSPLIT; // k-steps of a wave's share of a 16 x 16 score block
  constexpr int SROW = kMlaTile + 4;  // floats per score row (padded: 16 rows -> 16 bank positions)
  constexpr int LPR = 2 * DS / 16;    // lanes per row of a slice load
  constexpr int RPL = 64 / LPR;       // rows per load instruction
  constexpr int NLD = kMlaTile / RPL;
  // register sets of tile loads in flight (64 heads at d_c = 512 leave room for one)
  constexpr int NSET = D == 512 ? (HB == 1 ? 2 : 1) : (HB == 1 ? 3 : 2);
  static_assert(NT >= 1 && NLD >= 1 && NLD * RPL == kMlaTile && NBLK * KSPLIT == NW, "latent tile shape");
  __shared__ __attribute__((aligned(16))) char tiles[3][kMlaTile * ROWB];
  __shared__ __attribute__((aligned(16))) float sc[2][KSPLIT][HPC * SROW];  // partial scores per latent share

  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int gi = lane >> 4, s16 = lane & 15;

  const LaneLens ll = load_lane_lens(a.seq_lens, a.B, a.S_max, lane);
  const long long T = uniform(total_tiles_cached(ll, a.seq_lens, a.B, a.S_max, kMlaTile, a.n_hchunk, lane));
  const TileRanges rg(T, W);
  const long long lo = rg.lo(w);
  const long long hi = rg.lo(w + 1);
  if (lo >= hi) return;  // uniform over the workgroup
  const int n_local = (int)(hi - lo);
  const int dsl = wave * DS;  // first latent index of this wave's slice

  // Row r, chunk c of a tile sits at chunk position c ^ swz(r) (swz permutes
  // the 16 positions of a 256-byte window): the score reads (16 rows, one
  // chunk) and the transposed reads of the weighted sum (4 rows x 4 chunks)
  // each hit 16 positions.
  auto tile_off = [](int r, int c) { return r * ROWB + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4); };
  auto tile_at = [&](const char* t, int r, int c) { return t + tile_off(r, c); };

  // ---- tile loads: this wave's slice, lane (row ld_row, chunk ld_chunk of the slice)
  const int ld_row = lane / LPR, ld_chunk = lane % LPR;
  const unsigned lane_off = ld_row * ROWB + 2 * dsl + 16 * ld_chunk;
  u32x4 cr0[NLD], cr1[NSET >= 2 ? NLD : 1], cr2[NSET == 3 ? NLD : 1];
  // a tile's first row is the base of a buffer resource that ends at the
  // segment's last valid row: rows past it read as zero without an access
  auto issue = [&](u32x4* creg, const MlaSegment& s, int tile) {
    const int tt0 = s.t_begin + tile * kMlaTile;
    const size_t row0 = (size_t)uniform((long long)((size_t)s.b * a.S_max + tt0));
    const int nvalid = uniform(min(kMlaTile, s.t_end - tt0));
    const auto rc = make_rsrc(static_cast<const char*>(a.c) + row0 * ROWB, nvalid * ROWB);
#pragma unroll
    for (int u = 0; u < NLD; ++u) creg[u] = buffer_load_x4_nt(rc, lane_off + u * RPL * ROWB);
  };
  // this wave's slice of a staged tile into the workgroup's copy; readers see
  // it after the next barrier
  auto stage = [&](const u32x4* creg, char* t) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int r = u * RPL + ld_row;
      lds_store(t + tile_off(r, dsl / 8 + ld_chunk), creg[u]);
    }
  };

  // ---- score share of this wave: tokens 16 tb .. +15 of the tile, heads
  // 16 hq .. +15 of the chunk, latent values [kq0, kq0 + D / KSPLIT); B
  // operand fragments Q[head][kq0 + 32 ks + 8 gi .. +7], zero past h_q
  const int blk = wave % NBLK, ksh = wave / NBLK;
  const int tb = blk & 1, hq = blk >> 1;
  const int kq0 = ksh * (D / KSPLIT);
  u32x4 qf[KQ];
  auto load_q = [&](const MlaSegment& s) {
    const int head = s.hc * HPC + 16 * hq + s16;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((size_t)s.b * a.h_q + head) * D + kq0 + 8 * gi;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
      qf[ks] = head < a.h_q ? *reinterpret_cast<const u32x4*>(qb + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  };

  f32x16 o[HB][NT];
  float m[HB], l[HB];
  auto reset = [&]() {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m[hb] = kNegInf;
      l[hb] = 0.f;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[hb][n][r] = 0.f;
    }
  };
  // partial O (this wave's slice of every head) and, from wave 0, (m, l)
  auto write_partials = [&](const MlaSegment& s) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float lt = wave_sum_xor(l[hb], 32);
      const size_t row = (size_t)s.slot * HPC + 32 * hb + l32;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(a.part_o + row * D + dsl + 32 * n + 8 * r4 + 4 * h2) =
              f32x4{o[hb][n][4 * r4], o[hb][n][4 * r4 + 1], o[hb][n][4 * r4 + 2], o[hb][n][4 * r4 + 3]};
      if (wave == 0 && h2 == 0) {
        a.part_ml[row * 2 + 0] = m[hb];
        a.part_ml[row * 2 + 1] = lt;
      }
    }
  };

  // ---- prologue: tile 0 in LDS, the next NSET in flight (tile t in register
  // set t % NSET); tile 1 is staged by step 0 once its scores are issued, so
  // the first products do not wait for the second tile to land
  MlaSegment cur = mla_segment(a, ll, lo, hi, w, lane);
  MlaSegment ld = cur;  // segment of the tile issued last
  int cur0 = 0, ld0 = 0;  // local index of each segment's first tile
  load_q(cur);
  // issue local tile k; past the range, loads against an empty buffer range
  // (zeros, no memory access), so that every step issues the same loads
  auto prefetch = [&](u32x4* creg, int k) {
    if (k >= n_local) {
      const auto none = make_rsrc(a.c, 0);
#pragma unroll
      for (int u = 0; u < NLD; ++u) creg[u] = buffer_load_x4_nt(none, lane_off + u * RPL * ROWB);
      return;
    }
    if (k - ld0 >= ld.ntile) {
      ld0 += ld.ntile;
      ld = mla_segment(a, ll, lo + ld0, hi, w, lane);
    }
    issue(creg, ld, k - ld0);
  };
  auto set_of = [&](int t) -> u32x4* {  // (t is a compile-time residue where it matters)
    if constexpr (NSET == 1) return cr0;
    else if constexpr (NSET == 2) return (t & 1) ? cr1 : cr0;
    else return t % 3 == 0 ? cr0 : (t % 3 == 1 ? cr1 : cr2);
  };
  issue(cr0, ld, 0);
  if constexpr (NSET >= 2) prefetch(cr1, 1);
  if constexpr (NSET == 3) prefetch(cr2, 2);
  stage(cr0, tiles[0]);
  prefetch(cr0, NSET);
  reset();
  __syncthreads();  // every wave's slice of tile 0 written before its scores are read

  // one tile: its scores (score waves), one barrier, softmax and weighted sum
  // (every wave), then stage tile k + 2 from `next` (which takes tile k + 2 +
  // NSET) and close the segment at its end
  auto step = [&](int k, u32x4* next, auto first) {
    const char* ts = tiles[k % 3];
    float (*sk)[HPC * SROW] = sc[k & 1];
    const int tl = k - cur0;
    const int tt0 = cur.t_begin + tl * kMlaTile;
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int row = 16 * tb + s16;
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks)
        acc = mfma16(lds_load<u32x4>(tile_at(ts, row, kq0 / 8 + 4 * ks + gi)), qf[ks], acc);
      // lane holds the share's S^T[token 16 tb + 4 gi + i][head 16 hq + s16]
      lds_store(sk[ksh] + (16 * hq + s16) * SROW + 16 * tb + 4 * gi, acc);
    }
    if constexpr (decltype(first)::value) {  // step 0: tile 1, read by step 1 after this barrier
      stage(set_of(1), tiles[1]);
      prefetch(set_of(1), 1 + NSET);
    }
    __syncthreads();
    // ---- online softmax (the same on every wave) and the weighted sum of
    // this wave's slice; O and l share a reference max that moves only when a
    // tile's max exceeds it by more than kMlaSlack.  Lane (l32, h2) takes
    // head 32 hb + l32, tokens 8 (r/4) + 4 h2 + r%4.
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x16 s;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v = lds_load<f32x4>(sk[0] + (32 * hb + l32) * SROW + 8 * r4 + 4 * h2);
#pragma unroll
        for (int q = 1; q < KSPLIT; ++q) v += lds_load<f32x4>(sk[q] + (32 * hb + l32) * SROW + 8 * r4 + 4 * h2);
        s[4 * r4] = v[0];
        s[4 * r4 + 1] = v[1];
        s[4 * r4 + 2] = v[2];
        s[4 * r4 + 3] = v[3];
      }
      if (tt0 + kMlaTile > cur.t_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = tt0 + 8 * (r >> 2) + 4 * h2 + (r & 3) < cur.t_end ? s[r] : kNegInf;
      }
      // lane-local test first; the exchange with lane ^ 32 only when one of
      // the lane's scores exceeds the reference by more than the slack (the
      // same head-wide test, so the result does not change)
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
      bool grow = false;
      float alpha = 1.0f;
      if (__builtin_amdgcn_ballot_w64(mt * a.qk_scale_log2 > m[hb] + kMlaSlack)) {
        mt = wave_max_xor(mt, 32) * a.qk_scale_log2;
        grow = mt > m[hb] + kMlaSlack;
        const float m_up = grow ? mt : m[hb];
        alpha = grow ? fast_exp2(m[hb] - m_up) : 1.0f;
        m[hb] = m_up;
      }
      const float m_new = m[hb];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(__builtin_fmaf(s[r], a.qk_scale_log2, -m_new));
        psum += s[r];
      }
      l[hb] = l[hb] * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) o[hb][n] *= alpha;
      }
      // O^T += C^T P^T, two k-steps of 16 tokens (token order as in S)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4 pf = {pack_bf16x2(s[8 * p + 0], s[8 * p + 1]), pack_bf16x2(s[8 * p + 2], s[8 * p + 3]),
                          pack_bf16x2(s[8 * p + 4], s[8 * p + 5]), pack_bf16x2(s[8 * p + 6], s[8 * p + 7])};
        const int ra = 16 * p + 4 * h2 + (s16 >> 2), rb = ra + 8;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int col = dsl + 32 * n + 16 * (gi & 1) + 4 * (s16 & 3);
          const int c = col >> 3, wsub = col & 7;
          const u32x2 va = lds_read_tr16(tile_at(ts, ra, c) + 2 * wsub);
          const u32x2 vb = lds_read_tr16(tile_at(ts, rb, c) + 2 * wsub);
          o[hb][n] = mfma32(u32x4{va[0], va[1], vb[0], vb[1]}, pf, o[hb][n]);
        }
      }
    }
    // ---- tile k + 2 into the buffer tile k - 1 used (every wave is past its
    // reads: they precede this step's barrier); readers see it after the next
    stage(next, tiles[(k + 2) % 3]);
    prefetch(next, k + 2 + NSET);
    // ---- segment end: one partial per head, then the next sequence
    if (tl + 1 == cur.ntile) {
      write_partials(cur);
      if (k + 1 < n_local) {
        cur0 = k + 1;
        cur = mla_segment(a, ll, lo + cur0, hi, w, lane);
        load_q(cur);
        // wait for the new query here, once per segment: left pending, it
        // would make every tile wait for all loads in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        reset();
      }
    }
  };
  // step k stages tile k + 2 from set (k + 2) % NSET: whole groups of NSET
  // steps in a loop without early exits (each set then has the same loads
  // issued after it on every path, so a stage waits only for its own set),
  // the remainder after it
  // (step 0 is peeled off: it alone stages tile 1)
  using first_step = std::integral_constant<bool, true>;
  using later_step = std::integral_constant<bool, false>;
  step(0, set_of(2), first_step{});
  int k = 1;
  if constexpr (NSET == 1) {
    for (; k < n_local; ++k) step(k, cr0, later_step{});
  } else if constexpr (NSET == 2) {
    for (; k + 2 <= n_local; k += 2) {
      step(k, cr1, later_step{});
      step(k + 1, cr0, later_step{});
    }
    if (k < n_local) step(k, cr1, later_step{});
  } else {
    for (; k + 3 <= n_local; k += 3) {
      step(k, cr0, later_step{});
      step(k + 1, cr1, later_step{});
      step(k + 2, cr2, later_step{});
    }
    if (k < n_local) step(k, cr0, later_step{});
    if (k + 1 < n_local) step(k + 1, cr1, later_step{});
  }
}

}  // namespace

hipError_t launch_mla_decode_split(const MlaArgs& a, int D, int hb, int W, hipStream_t stream) {
  const dim3 grid(W), block(kMlaWaves * 64);
  if (D == 512) {
    if (hb == 1) hipLaunchKernelGGL((gqa_mla_decode_split<512, 1>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_mla_decode_split<512, 2>), grid, block, 0, stream, a);
  } else {
    if (hb == 1) hipLaunchKernelGGL((gqa_mla_decode_split<256, 1>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_mla_decode_split<256, 2>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gqa
