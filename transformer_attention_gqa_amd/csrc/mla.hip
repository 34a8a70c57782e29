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
// GQA decode (one slab per sequence, all heads in one workgroup).  The 8
// wavefronts of a workgroup work on the same 32-token tile, wave w owning the
// latent slice [w * d_c / 8, (w + 1) * d_c / 8):
//  * each wave loads only its slice of the tile (a 128-byte piece of every
//    token row at d_c = 512) into a private LDS slab, which serves as its
//    share of K (scores) and of V (weighted sum);
//  * partial scores S^T[token][head] over the slice come from
//    v_mfma_f32_32x32x16_bf16; the 8 partials are summed through LDS (each
//    wave sums a quarter of the tile's rows, two barriers per tile) and every
//    wave runs the same online softmax on the full scores;
//  * the weighted sum O^T[latent][head] += C^T P^T runs on the wave's own
//    slice, so a wave's accumulator holds d_c / 8 latent values of every head
//    and the partial results need no merge across waves.
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
  const long long local = t - base;
  const int hc = (int)(local / nt);
  const int tile0 = (int)(local - (long long)hc * nt);
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
  constexpr int DS = D / NW;        // latent values per wave
  constexpr int RB = 2 * DS;        // bytes of one token's slice
  constexpr int CHS = RB / 16;      // 16-byte chunks per slice row
  constexpr int SWS = 256 / RB;     // slice rows per 256-byte bank window
  constexpr int KSW = DS / 16;      // k-steps of the partial score product
  constexpr int NT = DS / 32;       // 32-wide latent tiles of the weighted sum
  constexpr int HPC = 32 * HB;      // query heads per chunk
  constexpr int LPR = RB / 16;      // lanes per row of the tile load
  constexpr int RPL = 64 / LPR;     // rows per load instruction
  constexpr int NLD = kMlaTile / RPL;
  static_assert(NT >= 1 && NLD >= 1 && NLD * RPL == kMlaTile, "latent slice shape");
  __shared__ __attribute__((aligned(16))) char slab[NW][2][kMlaTile * RB];
  __shared__ __attribute__((aligned(16))) f32x4 part[NW][HB][4][64];  // partial scores, accumulator layout
  __shared__ __attribute__((aligned(16))) f32x4 fin[HB][4][64];       // summed scores

  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int gi = lane >> 4, s16 = lane & 15;

  const LaneLens ll = load_lane_lens(a.seq_lens, a.B, a.S_max, lane);
  const long long T = uniform(total_tiles_cached(ll, a.seq_lens, a.B, a.S_max, kMlaTile, a.n_hchunk, lane));
  const long long lo = (long long)w * T / W;
  const long long hi = (long long)(w + 1) * T / W;
  if (lo >= hi) return;  // uniform over the workgroup
  const int n_local = (int)(hi - lo);
  const int dsl = wave * DS;  // first latent index of this wave's slice

  // slice row r, chunk c sits at chunk position c ^ swz_row(r).  SWS rows
  // share a 256-byte window of 16 chunk positions; swz_row permutes the chunk
  // positions of the rows that share a window position, so the 16 lanes of a
  // score fragment read (16 consecutive rows, one chunk) hit 16 positions.
  // With 8 chunks per row it also sends rows r and r + 2 of a 4-row group to
  // different halves of the row, so the transposed reads of the weighted sum
  // (4 consecutive rows x 4 consecutive chunks) hit 16 positions as well.
  auto swz_row = [](int r) {
    const int j = (r / SWS) % CHS;
    if constexpr (CHS == 8) return ((j & 1) << 2) | (j >> 1);
    else return j;
  };

  // ---- tile loads: lane (row ld_row, chunk ld_chunk) of each instruction
  const int ld_row = lane / LPR, ld_chunk = lane % LPR;
  const unsigned lane_off = ld_row * (2 * D) + 2 * dsl + 16 * ld_chunk;
  // NSET register sets of NLD loads each: while a wave computes one tile
  // from LDS, the next NSET tiles are in flight (64 heads at d_c = 512 leave
  // registers for one set only)
  constexpr int NSET = HB == 1 ? 3 : (D == 512 ? 1 : 2);
  u32x4 cr0[NLD], cr1[NSET >= 2 ? NLD : 1], cr2[NSET == 3 ? NLD : 1];
  // a tile's first row is the base of a buffer resource that ends at the
  // segment's last valid row: rows past it read as zero without an access
  auto issue = [&](u32x4* creg, const MlaSegment& s, int tile) {
    const int tt0 = s.t_begin + tile * kMlaTile;
    const size_t row0 = (size_t)uniform((long long)((size_t)s.b * a.S_max + tt0));
    const int nvalid = uniform(min(kMlaTile, s.t_end - tt0));
    const auto rc = make_rsrc(static_cast<const char*>(a.c) + row0 * (2 * D), nvalid * (2 * D));
#pragma unroll
    for (int u = 0; u < NLD; ++u) creg[u] = buffer_load_x4_nt(rc, lane_off + u * RPL * (2 * D));
  };
  auto stage = [&](const u32x4* creg, int buf) {
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int r = u * RPL + ld_row;
      lds_store(slab[wave][buf] + r * RB + ((ld_chunk ^ swz_row(r)) << 4), creg[u]);
    }
    wave_lds_fence();
  };

  // ---- query fragments of the slice (B operand of S^T = C Q^T); heads past
  // h_q in the last chunk read as zero
  u32x4 qf[HB][KSW];
  auto load_q = [&](const MlaSegment& s) {
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (size_t)s.b * a.h_q * D + dsl + 8 * h2;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = s.hc * HPC + 32 * hb + l32;
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks)
        qf[hb][ks] = head < a.h_q ? *reinterpret_cast<const u32x4*>(qb + (size_t)head * D + 16 * ks)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
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

  // ---- prologue: the first tile in LDS, the next NSET in flight
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
      for (int u = 0; u < NLD; ++u) creg[u] = buffer_load_x4_nt(none, lane_off + u * RPL * (2 * D));
      return;
    }
    if (k - ld0 >= ld.ntile) {
      ld0 += ld.ntile;
      ld = mla_segment(a, ll, lo + ld0, hi, w, lane);
    }
    issue(creg, ld, k - ld0);
  };
  issue(cr0, ld, 0);
  if constexpr (NSET >= 2) prefetch(cr1, 1);
  if constexpr (NSET == 3) prefetch(cr2, 2);
  stage(cr0, 0);
  prefetch(cr0, NSET);
  reset();

  // one tile: compute it from LDS, stage the next one from `next` (which
  // then takes the tile NSET further on), close the segment at its end
  auto step = [&](int k, u32x4* next) {
    const int buf = k & 1;
    const int tl = k - cur0;
    const int tt0 = cur.t_begin + tl * kMlaTile;
    const char* cs = slab[wave][buf];
    // ---- partial scores over this wave's slice: lane holds tokens
    // 8(r/4) + 4h2 + r%4 of head 32hb + l32
    f32x16 s[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[hb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const u32x4 kf = lds_load<u32x4>(cs + l32 * RB + (((2 * ks + h2) ^ swz_row(l32)) << 4));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) s[hb] = mfma32(kf, qf[hb][ks], s[hb]);
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        part[wave][hb][r4][lane] = f32x4{s[hb][4 * r4], s[hb][4 * r4 + 1], s[hb][4 * r4 + 2], s[hb][4 * r4 + 3]};
    __syncthreads();
    // ---- sum the partials: thread e of the workgroup takes element e
    for (int e = threadIdx.x; e < HB * 4 * 64; e += NW * 64) {
      const int hb = e / 256, r4 = (e / 64) % 4, ln = e % 64;
      f32x4 acc = part[0][hb][r4][ln];
#pragma unroll
      for (int wv = 1; wv < NW; ++wv) acc += part[wv][hb][r4][ln];
      fin[hb][r4][ln] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v = fin[hb][r4][lane];
        s[hb][4 * r4] = v[0];
        s[hb][4 * r4 + 1] = v[1];
        s[hb][4 * r4 + 2] = v[2];
        s[hb][4 * r4 + 3] = v[3];
      }
    // ---- online softmax (the same on every wave) and the weighted sum of
    // this wave's slice; O and l share a reference max that moves only when a
    // tile's max exceeds it by more than kMlaSlack
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if (tt0 + kMlaTile > cur.t_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[hb][r] = tt0 + 8 * (r >> 2) + 4 * h2 + (r & 3) < cur.t_end ? s[hb][r] : kNegInf;
      }
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[hb][r]);
      mt = wave_max_xor(mt, 32) * a.qk_scale_log2;
      const bool grow = mt > m[hb] + kMlaSlack;
      const float m_new = grow ? mt : m[hb];
      const float alpha = grow ? fast_exp2(m[hb] - m_new) : 1.0f;
      m[hb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[hb][r] = fast_exp2(__builtin_fmaf(s[hb][r], a.qk_scale_log2, -m_new));
        psum += s[hb][r];
      }
      l[hb] = l[hb] * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) o[hb][n] *= alpha;
      }
      // O^T += C^T P^T, two k-steps of 16 tokens (token order as in S)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4 pf = {pack_bf16x2(s[hb][8 * p + 0], s[hb][8 * p + 1]), pack_bf16x2(s[hb][8 * p + 2], s[hb][8 * p + 3]),
                          pack_bf16x2(s[hb][8 * p + 4], s[hb][8 * p + 5]), pack_bf16x2(s[hb][8 * p + 6], s[hb][8 * p + 7])};
        const int ra = 16 * p + 4 * h2 + (s16 >> 2), rb = ra + 8;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int col = 32 * n + 16 * (gi & 1) + 4 * (s16 & 3);
          const int c = col >> 3, wsub = col & 7;
          const u32x2 va = lds_read_tr16(cs + ra * RB + ((c ^ swz_row(ra)) << 4) + 2 * wsub);
          const u32x2 vb = lds_read_tr16(cs + rb * RB + ((c ^ swz_row(rb)) << 4) + 2 * wsub);
          o[hb][n] = mfma32(u32x4{va[0], va[1], vb[0], vb[1]}, pf, o[hb][n]);
        }
      }
    }
    stage(next, buf ^ 1);
    prefetch(next, k + 1 + NSET);
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
  // the register sets rotate with period NSET: whole groups of NSET steps in
  // a loop without early exits (each set then has the same loads issued after
  // it on every path, so a stage waits only for its own set), the remainder
  // after it
  int k = 0;
  if constexpr (NSET == 1) {
    for (; k < n_local; ++k) step(k, cr0);
  } else if constexpr (NSET == 2) {
    for (; k + 2 <= n_local; k += 2) {
      step(k, cr1);
      step(k + 1, cr0);
    }
    if (k < n_local) step(k, cr1);
  } else {
    for (; k + 3 <= n_local; k += 3) {
      step(k, cr1);
      step(k + 1, cr2);
      step(k + 2, cr0);
    }
    if (k < n_local) step(k, cr1);
    if (k + 1 < n_local) step(k + 1, cr2);
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
