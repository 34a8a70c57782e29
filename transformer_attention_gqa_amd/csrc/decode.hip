// Split-sequence decode kernels and the combine kernel.
//
// One decode step: for every sequence b and query head j, softmax over the
// L_b visible cache positions of scale * q_j . k_t, weights applied to v_t,
// with query head j reading K/V head j / G ("GQA Implementation" and "MQA
// (Multi-Query Attention)" in "Evolution of AI Attention Mechanisms"; the
// decoding step softmax(Q_all K_shared^T) V_shared of the "Multi-Query
// Attention (MQA)" glossary).  Decode moves the whole cache through memory
// once per step and does Theta(h d_h S) flops ("Multi-query attention",
// "Why this is a bandwidth argument, not a FLOP argument"), so the kernels are
// built around reading every K/V byte exactly once, evenly over the chip:
//
//  * the launch is one wide workgroup per compute unit (persistent); the
//    32-token tiles (64 for int4 with one block of 16 heads, held as two
//    halves) of all (sequence, kv-head) slabs are concatenated and cut
//    into equal ranges, one per workgroup, so ragged sequence lengths cost no
//    load imbalance and no tail of lone workgroups (schedule: gqa_launch.h);
//  * a workgroup serves every query head of the slab's group (up to 32) from a
//    single read of each K/V tile;
//  * its wavefronts take tiles as they become free; each tile arrives through 128-bit
//    non-temporal loads (16 lanes cover one contiguous 256-byte cache row), is
//    written once to the wave's private LDS slab with an XOR chunk swizzle,
//    and is consumed from there by the matrix cores while the next tile is
//    already in flight in registers;
//  * scores S^T[token][head] = K Q^T and O^T[d][head] += V^T P^T run on
//    v_mfma_f32_16x16x32_bf16; the token order inside the PV product is
//    permuted so that the score layout produced by the first product is
//    directly the B operand of the second (no shuffles), and V is fetched
//    transposed with ds_read_b64_tr_b16;
//  * softmax is online: per head a running max m (log2 domain) and running
//    sum l; a tile rescales O and l by 2^(m_old - m_new) ("Flash Attention
//    Principle": running max and running sum, write only the final result);
//  * at the end of each slab segment the waves merge their (O, m, l) through
//    LDS and the workgroup writes one unnormalised partial per head; the
//    combine kernel merges the partials of a slab.
// The fp8 path reads e4m3 codes (half the bytes), converts them to bf16
// exactly in registers and folds the per-token scales into the score (K) and
// into the probability (V).  The fp32 path keeps float32 end to end on the
// vector ALUs.
#include "decode_sched.h"
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int kTile = 32;     // tokens per wave tile (matrix-core paths)
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag the true max
constexpr int kTileF32 = 64;  // tokens per wave tile (float32 path)
constexpr int kWavesF32 = 4;

// ------------------------------------------------------------------------
// Matrix-core decode: bf16 Q; bf16 or e4m3 K/V.  HB blocks of 16 heads,
// NW wavefronts per workgroup.
// ------------------------------------------------------------------------
// One contiguous piece of a workgroup's tile range that lies in a single slab.
struct Segment {
  int b, g, hc;        // sequence, kv-head, head chunk
  int ntile;           // tiles of the segment
  int t_begin, t_end;  // token range [t_begin, t_end) inside the sequence
  int nh, head0;       // heads served and the global index of the first
  size_t slab;         // contiguous cache: cache row of token 0 of (b, g)
  long long slot;      // partial slot
  int pwin;            // paged cache: first logical page of the block-table window ...
  int pg;              // ... whose entry pwin + lane this lane holds (a VGPR)
};

// Paged cache: lane i returns the physical page of logical page lp0 + i of
// sequence b (0 past the table's width), clamped into the pool so that a bad
// entry cannot address memory outside it.
__device__ __forceinline__ int load_page_window(const DecodeArgs& a, int b, int lp0, int lane) {
  const int lp = lp0 + lane;
  const int p = lp < a.max_pages ? a.block_table[(size_t)b * a.max_pages + lp] : 0;
  return min(max(p, 0), a.num_pages - 1);
}

// Cache row (in rows of d_h elements) of token t of segment s.  Paged: the
// page comes from the segment's block-table window, refilled (one load) when
// t lies past its 64 pages; rows never cross a page inside a 32-token tile.
template <bool PAGED>
__device__ __forceinline__ size_t cache_row(const DecodeArgs& a, Segment& s, int t, int lane) {
  if constexpr (PAGED) {
    const int lp = t >> a.page_shift;
    if (lp - s.pwin >= 64) {  // wave-uniform
      s.pwin = lp;
      s.pg = load_page_window(a, s.b, lp, lane);
    }
    const int page = __builtin_amdgcn_readlane(s.pg, lp - s.pwin);
    return ((((size_t)page * a.n_kv + s.g) << a.page_shift) | (size_t)(t & ((1 << a.page_shift) - 1)));
  } else {
    return s.slab + t;
  }
}

template <int TILE, bool PAGED>
__device__ __forceinline__ Segment make_segment(const DecodeArgs& a, const LaneLens& ll, long long t, long long hi,
                                                int w, int spb, int hpc, int lane) {
  int b, nt, L;
  long long base;
  locate_tile_cached(ll, a.seq_lens, a.B, a.S_max, TILE, spb, t, lane, b, base, nt, L);
  b = uniform(b);
  nt = uniform(nt);
  L = uniform(L);
  base = uniform(base);
  int slab_in_b, tile0;
  split_local(t - base, nt, slab_in_b, tile0);
  Segment s;
  s.b = b;
  s.g = slab_in_b / a.n_hchunk;
  s.hc = slab_in_b - s.g * a.n_hchunk;
  s.ntile = (int)min(hi - t, (long long)(nt - tile0));
  s.t_begin = tile0 * TILE;
  s.t_end = min((tile0 + s.ntile) * TILE, L);
  const int G = a.h_q / a.n_kv;
  s.nh = min(hpc, G - s.hc * hpc);
  s.head0 = s.g * G + s.hc * hpc;
  s.slab = ((size_t)b * a.n_kv + s.g) * (size_t)a.S_max;
  s.slot = w + (long long)b * spb + slab_in_b;
  s.pwin = 0;
  s.pg = 0;
  if constexpr (PAGED) {
    s.pwin = s.t_begin >> a.page_shift;
    s.pg = load_page_window(a, b, s.pwin, lane);
  }
  return s;
}

// Element format of a matrix-core decode's K/V cache.
enum KvFormat : int { kKvBf16 = 0, kKvFp8 = 1, kKvInt8 = 2, kKvInt4 = 3 };

template <int D, int HB, int KVF, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void gqa_decode_split_mfma(DecodeArgs a) {
  // quantized caches carry one float32 scale per (token, kv-head) row for K
  // and for V: the K scale multiplies the score, the V scale the probability
  constexpr bool QUANT = KVF != kKvBf16;
  constexpr int CH = D / 8;   // 16-byte bf16 chunks per row
  constexpr int KK = D / 32;  // k-steps of the score product
  constexpr int NT = D / 16;  // 16-wide d tiles of the PV product
  constexpr int TILE_BYTES = kTile * D * 2;
  constexpr int HPC = 16 * HB;
  // int4 with one block of 16 heads: 64-token tiles in two register halves (see below)
  constexpr bool SPLIT2 = KVF == kKvInt4 && HB == 1;
  constexpr int NH = SPLIT2 ? 2 : 1;  // register halves
  constexpr int TT = NH * kTile;      // tokens per scheduled tile
  // int4 caches with one 16-head block are converted to bf16 136 + code, the
  // offset removed in the products, with the codes of each 8-element chunk
  // in the order 0 2 4 6 1 3 5 7 (each bf16 pair then comes from one byte
  // permute, see i4x8_to_bf16x8_biased_eo).  Q is staged in the same order,
  // which leaves every score unchanged; with V staged the same way the rows
  // of O come out in that order and are put back at the segment end.  (With two head blocks the
  // extra registers spill, so that kernel converts through float.)
  constexpr bool BIAS4 = KVF == kKvInt4 && HB == 1;
  // With d = 128 such a kernel also skips the LDS for K: lane (q4, r16)
  // loads the 16 bytes (32 codes) q4 of token row r16 of each 16-token half,
  // exactly the codes of its score-product operand when k-slot (q4, j) of
  // k-step kk stands for d = 32 q4 + 8 kk + j (and Q is read to match), so
  // K goes from the load registers through the conversion into the product.
  // The fp8 and int8 kernels with one head block (d = 128) do the same with
  // their 128-byte rows: lane (q4, r16) loads bytes 32 q4 .. 32 q4 + 31 of
  // token row r16 of each 16-token half (two 16-byte loads) and converts them
  // exactly to the bf16 operands of its four k-steps.
  constexpr bool KDIR = (BIAS4 || ((KVF == kKvFp8 || KVF == kKvInt8) && HB == 1)) && D == 128;
  constexpr bool V4RAW = KDIR && KVF == kKvInt4;  // V as raw int4 codes (below)
  // Such a kernel keeps V as raw codes in LDS too (2 KiB per 32 tokens instead
  // of 8 KiB of bf16) and reads it with the 4-bit transposing LDS read: within
  // each 16-lane group, output lane i receives nibble i of the 8 bytes each of
  // the 16 lanes points at (nibble j from lane j).  Lane (q4, L) points at the
  // token of k-slot 8 q4 + (L % 8) and at the 8 bytes of d-tile 2p + L / 8,
  // so one read gives lane (q4, r16) the codes of d = 32p + r16 (first dword)
  // and 32p + 16 + r16 (second) over its 8 k-slots: the A operands of two
  // products, in natural d order.  8-byte chunk c of token row r sits at chunk
  // position c ^ vsw(r); vsw keeps both the 16-byte staging writes and the
  // transposed reads (8 rows x 2 chunks per 16 lanes) on distinct banks.
  auto vsw = [](int r) { return (((r >> 4) & 1) << 1) | (((r >> 2) & 1) << 2); };
  // V^T fragments of the weighted sum read ahead of the softmax (registers allowing)
  constexpr int NPRE = HB == 1 ? 4 : 0;
  // 32 heads of a bf16 cache: one 32x32 score tile per 32 tokens on
  // v_mfma_f32_32x32x16_bf16 (the same shape as the prefill kernel with heads
  // in place of query rows); otherwise HB blocks of 16 heads on 16x16x32.
  constexpr bool M32 = HB == 2 && KVF == kKvBf16;
  constexpr int KS = D / 16;  // k-steps of the 32x32 score product
  constexpr int NT32 = D / 32;
  static_assert(HPC * D * 4 <= 2 * TILE_BYTES, "partial O does not fit the wave slab");
  constexpr int QCH = (HPC * CH + NW * 64 - 1) / (NW * 64);  // 16-byte query chunks per thread
  __shared__ __attribute__((aligned(16))) char smem[NW][2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sq[HPC * D * 2];  // the segment's query rows, bf16, swizzled
  __shared__ float sm_ml[NW][HPC][2];
  __shared__ int s_next_tile;  // next unclaimed tile of the current segment
  // quantized caches: the staged tile's K scales (entries 0..31) and V scales
  // (32..63), one per row, in each wave's own slot
  __shared__ __attribute__((aligned(16))) float ssc[QUANT ? NW : 1][64];

  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4;
  const int r16 = lane & 15;
  const int spb = a.n_kv * a.n_hchunk;

  const LaneLens ll = load_lane_lens(a.seq_lens, a.B, a.S_max, lane);
  const long long T = uniform(total_tiles_cached(ll, a.seq_lens, a.B, a.S_max, TT, spb, lane));
  const TileRanges rg(T, W);
  long long lo = rg.lo(w);
  const long long hi = rg.lo(w + 1);
  if (lo >= hi) return;  // uniform over the workgroup

  char* kt = smem[wave][0];
  char* vt = smem[wave][1];
  float* ow = reinterpret_cast<float*>(smem[wave][0]);
  // O exchange layout in a wave slab: head h's D floats are one row, and its
  // 16-byte chunk q sits at q ^ (h % (D/4)).  A row is 512 bytes (d = 128),
  // so without the swizzle the heads of one store instruction would all hit
  // the same banks; with it both the fragment stores and the row reads of
  // the merge spread over all banks.
  auto ow_idx = [](int h, int d) { return h * D + ((((d >> 2) ^ (h % (D / 4))) << 2) | (d & 3)); };

  // per-lane load assignment: each lane loads 16 bytes of a cache row, a row
  // by ROWB/16 consecutive lanes (bf16: CH lanes of 8 elements; fp8 / int8:
  // D/16 lanes of 16 codes; int4: D/32 lanes of 32 codes).
  constexpr int ROWB = KVF == kKvBf16 ? 2 * D : (KVF == kKvInt4 ? D / 2 : D);  // bytes per cache row
  constexpr int NLD = (kTile * ROWB) / (64 * 16);  // load instructions per tensor and tile
  constexpr int LPR = ROWB / 16;                   // lanes per row
  constexpr int RPL = 64 / LPR;                    // rows per load instruction
  const int ld_row = lane / LPR;
  const int ld_chunk = lane % LPR;

  // An int4 tile (32 tokens) is only 2 KiB of K and 2 KiB of V, so with one
  // tile in flight per wave the loads cannot cover the memory latency.  With
  // one block of 16 heads the int4 path therefore schedules 64-token tiles
  // held as two 32-token halves in separate registers: while one half is
  // staged and computed, the next tile's same half is already loading, so
  // two halves are always in flight.  The LDS slab still holds 32 tokens.
  u32x4 kreg[NH][NLD], vreg[NH][NLD];
  float ksl[NH], vsl[NH];  // K and V scale of row lane % 32 of the tile in flight

  // loads of tile `tile` of segment s into kreg/vreg (and its K/V scales).
  // The tile's first row is wave-uniform: it becomes the base of a buffer
  // resource whose range ends at the segment's last valid row, so rows past
  // the end read as zero without a memory access (a cache tail may hold NaN)
  // and each load needs only a 32-bit lane offset.
  const unsigned lane_off = ld_row * ROWB + ld_chunk * 16;
  // byte offset of K load u from the tile's first row
  auto k_off = [&](int u) -> unsigned {
    if constexpr (!KDIR) return lane_off + u * RPL * ROWB;
    else if constexpr (KVF == kKvInt4) return (16 * u + r16) * ROWB + 16 * q4;  // half u
    else return (16 * (u >> 1) + r16) * ROWB + 32 * q4 + 16 * (u & 1);         // half u / 2, part u % 2
  };
  static_assert(!KDIR || (KVF == kKvInt4 ? NLD == 2 : NLD == 4), "direct K: two 16-token halves per tile");
  // (a half past the segment's end gets an empty range: its loads return
  // zeros without a memory access, so every path issues the same loads)
  auto issue_loads = [&](Segment& s, int tile, int half = 0) {
    const int tt0 = s.t_begin + tile * TT + half * kTile;
    const size_t row0 = (size_t)uniform((long long)cache_row<PAGED>(a, s, tt0, lane));
    const int nvalid = uniform(max(min(kTile, s.t_end - tt0), 0));
    const auto rk = make_rsrc(static_cast<const char*>(a.k) + row0 * ROWB, nvalid * ROWB);
    const auto rv = make_rsrc(static_cast<const char*>(a.v) + row0 * ROWB, nvalid * ROWB);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      kreg[half][u] = buffer_load_x4_nt(rk, k_off(u));
      vreg[half][u] = buffer_load_x4_nt(rv, lane_off + u * RPL * ROWB);
    }
    if constexpr (QUANT) {
      // one K and one V scale per lane (row lane % 32); rows past the end
      // read zero, and their scores are masked anyway
      const auto rks = make_rsrc(a.k_scale + row0, nvalid * 4);
      const auto rvs = make_rsrc(a.v_scale + row0, nvalid * 4);
      ksl[half] = buffer_load_f32(rks, 4 * (lane & 31));
      vsl[half] = buffer_load_f32(rvs, 4 * (lane & 31));
    }
  };
  struct QRows {
    u32x4 v[QCH];
  };
  auto load_q = [&](const Segment& s) {
    QRows r;
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int e = threadIdx.x + i * NW * 64;
      const int hl = e / CH, c = e % CH;
      r.v[i] = u32x4{0u, 0u, 0u, 0u};
      if (e < HPC * CH && hl < s.nh)
        r.v[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                 ((size_t)s.b * a.h_q + s.head0 + hl) * D + 8 * c);
    }
    return r;
  };
  auto store_q = [&](const QRows& r) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int e = threadIdx.x + i * NW * 64;
      const int hl = e / CH, c = e % CH;
      u32x4 x = r.v[i];
      if constexpr (BIAS4) x = bf16x8_even_odd(x);
      if (e < HPC * CH) lds_store(sq + hl * (2 * D) + ((c ^ swz<CH>(hl)) << 4), x);
    }
  };

  // Further tiles of a segment (after each wave's first two) are claimed
  // from an LDS counter, so waves whose loads are served faster take more
  // tiles and all reach the segment's merge at about the same time.  In the
  // deterministic mode wave i keeps the static order i, i + NW, i + 2 NW, ...,
  // which fixes every wave's summation order and rounding points.
  const bool det = a.deterministic != 0;
  auto claim_tile = [&](int cur_tile) {
    if (det) return cur_tile + NW;
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_next_tile, 1);
    return uniform(__shfl(v, 0, 64));
  };

  // Stage the tile whose loads were issued last into the wave's LDS slab as
  // bf16 (quantized codes are converted exactly) and its scales into the
  // wave's scale slot.
  u32x4 kcur[KDIR ? NLD : 1];  // direct K: the staged tile's codes, as loaded
  auto stage = [&](int half = 0) {
    wave_lds_fence();
    if constexpr (QUANT) ssc[wave][lane] = lane < 32 ? ksl[half] : vsl[half];
    if constexpr (KDIR) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) kcur[u] = kreg[half][u];
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int r = u * RPL + ld_row;
      if constexpr (KVF == kKvFp8) {
        // 16 codes -> 16 bf16 = logical bf16 chunks 2c, 2c+1 of row r
        const int c0 = 2 * ld_chunk;
        u32x2 t0, t1, t2, t3;
        const int sw = swz<CH>(r);
        if constexpr (!KDIR) {
          t0 = e4m3x4_to_bf16x4(kreg[half][u][0]);
          t1 = e4m3x4_to_bf16x4(kreg[half][u][1]);
          t2 = e4m3x4_to_bf16x4(kreg[half][u][2]);
          t3 = e4m3x4_to_bf16x4(kreg[half][u][3]);
          lds_store(kt + r * (2 * D) + ((c0 ^ sw) << 4), u32x4{t0[0], t0[1], t1[0], t1[1]});
          lds_store(kt + r * (2 * D) + (((c0 + 1) ^ sw) << 4), u32x4{t2[0], t2[1], t3[0], t3[1]});
        }
        t0 = e4m3x4_to_bf16x4(vreg[half][u][0]);
        t1 = e4m3x4_to_bf16x4(vreg[half][u][1]);
        t2 = e4m3x4_to_bf16x4(vreg[half][u][2]);
        t3 = e4m3x4_to_bf16x4(vreg[half][u][3]);
        const u32x4 vlo = u32x4{t0[0], t0[1], t1[0], t1[1]};
        const u32x4 vhi = u32x4{t2[0], t2[1], t3[0], t3[1]};
        lds_store(vt + r * (2 * D) + ((c0 ^ sw) << 4), vlo);
        lds_store(vt + r * (2 * D) + (((c0 + 1) ^ sw) << 4), vhi);
      } else if constexpr (KVF == kKvInt8) {
        // 16 codes -> logical bf16 chunks 2c, 2c+1 of row r
        const int c0 = 2 * ld_chunk;
        const int sw = swz<CH>(r);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (!KDIR) {
            const u32x2 k0 = i8x4_to_bf16x4(kreg[half][u][2 * h]), k1 = i8x4_to_bf16x4(kreg[half][u][2 * h + 1]);
            lds_store(kt + r * (2 * D) + (((c0 + h) ^ sw) << 4), u32x4{k0[0], k0[1], k1[0], k1[1]});
          }
          const u32x2 v0 = i8x4_to_bf16x4(vreg[half][u][2 * h]), v1 = i8x4_to_bf16x4(vreg[half][u][2 * h + 1]);
          lds_store(vt + r * (2 * D) + (((c0 + h) ^ sw) << 4), u32x4{v0[0], v0[1], v1[0], v1[1]});
        }
      } else if constexpr (V4RAW) {
        // V as raw codes: 8-byte chunks 2c and 2c+1 of row r, adjacent under
        // vsw (which leaves bit 0 of the chunk index alone)
        lds_store(vt + r * ROWB + 8 * ((2 * ld_chunk) ^ vsw(r)), vreg[half][u]);
      } else if constexpr (KVF == kKvInt4) {
        // 32 codes -> logical bf16 chunks 4c .. 4c+3 of row r (one per dword)
        const int c0 = 4 * ld_chunk;
        const int sw = swz<CH>(r);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if constexpr (BIAS4) {
            lds_store(kt + r * (2 * D) + (((c0 + h) ^ sw) << 4), i4x8_to_bf16x8_biased_eo(kreg[half][u][h]));
            lds_store(vt + r * (2 * D) + (((c0 + h) ^ sw) << 4), i4x8_to_bf16x8_biased_eo(vreg[half][u][h]));
          } else {
            lds_store(kt + r * (2 * D) + (((c0 + h) ^ sw) << 4), i4x8_to_bf16x8(kreg[half][u][h]));
            lds_store(vt + r * (2 * D) + (((c0 + h) ^ sw) << 4), i4x8_to_bf16x8(vreg[half][u][h]));
          }
        }
      } else {
        const int pc = ld_chunk ^ swz<CH>(r);
        lds_store(kt + r * (2 * D) + (pc << 4), kreg[half][u]);
        lds_store(vt + r * (2 * D) + (pc << 4), vreg[half][u]);
      }
    }
    wave_lds_fence();
  };

  Segment cur = make_segment<TT, PAGED>(a, ll, lo, hi, w, spb, HPC, lane);
  QRows qc = load_q(cur);
  wave_lds_fence();  // the first tile's loads go out after the query rows'
  if (wave < cur.ntile) {
#pragma unroll
    for (int h = 0; h < NH; ++h) issue_loads(cur, wave, h);
  }

  for (;;) {
    const bool has_next = lo + cur.ntile < hi;
    Segment nxt = cur;
    if (has_next) nxt = make_segment<TT, PAGED>(a, ll, lo + cur.ntile, hi, w, spb, HPC, lane);
    const int t_begin = cur.t_begin, t_end = cur.t_end;

    // ---- prologue: wave i takes tiles i and i + NW.  It stages the first and
    // puts the second (or its first tile of the next segment) in flight before
    // the workgroup waits for the segment's query rows, so that no wave's
    // second load waits for the slowest wave's first: at kernel start every
    // wave's first load is queued behind the whole chip's first burst.
    // half h of tile idx of this segment, or else of the wave's first tile of the next
    auto issue_next = [&](int idx, int h) {
      if (idx < cur.ntile) issue_loads(cur, idx, h);
      else if (has_next && wave < nxt.ntile) issue_loads(nxt, wave, h);
    };
    int tile = wave, next_tile = wave + NW;
    if (tile < cur.ntile) {
      stage(0);
      issue_next(next_tile, 0);
    } else if (has_next && wave < nxt.ntile) {
#pragma unroll
      for (int h = 0; h < NH; ++h) issue_loads(nxt, wave, h);
    }
    QRows q_next = {};
    if (has_next) q_next = load_q(nxt);  // used at the segment switch, long after it lands
    store_q(qc);
    if (threadIdx.x == 0) s_next_tile = 2 * NW;
    __syncthreads();  // sq and the tile counter ready

    // int4 caches are staged as 136 + code (see i4x8_to_bf16x8_biased).  For
    // the scores, q . (k + 136) - 136 sum(q) = q . k: every score
    // accumulator starts at -136 sum(q) of its head, formed by one product of
    // the head's query row with a row of ones (lane: head r16 of block hb).
    // For the weighted sum, sum_t p_t (v_t + 136) - 136 sum_t p_t = sum_t
    // p_t v_t: one extra product with a ones row carries sum_t p_t (the bf16
    // weights the products use) next to O, and the segment's end removes it.
    float kbias[BIAS4 ? HB : 1];
    f32x4 osum[BIAS4 ? HB : 1];  // row 0 (lane r16, register 0): sum of the weights of head r16
    u32x4 ones_row0 = {0u, 0u, 0u, 0u};
    if constexpr (BIAS4) {
      const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
      if (r16 == 0) ones_row0 = ones;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int qrow = 16 * hb + r16;
        f32x4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          qs = mfma16(ones, lds_load<u32x4>(sq + qrow * (2 * D) + (((4 * kk + q4) ^ swz<CH>(qrow)) << 4)), qs);
        kbias[hb] = -kInt4Bias * qs[0];
        osum[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // direct K: the B operands of the score product for k-step kk, Q[head
    // r16][32 q4 + 8 kk + pi(j)] = staged chunk 4 q4 + kk, held for the segment
    u32x4 qreg[KDIR ? KK : 1];
    if constexpr (KDIR) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qreg[kk] = lds_load<u32x4>(sq + r16 * (2 * D) + (((4 * q4 + kk) ^ swz<CH>(r16)) << 4));
    }

    // ---- running state (per lane: head r16 of every head block; head l32 in the 32x32 shape)
    f32x4 o[M32 ? 1 : HB][M32 ? 1 : NT];
    f32x16 o32[M32 ? NT32 : 1];
    float m[HB], l[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m[hb] = kNegInf;
      l[hb] = 0.f;
    }
    if constexpr (M32) {
#pragma unroll
      for (int n = 0; n < NT32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o32[n][r] = 0.f;
    } else {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int n = 0; n < NT; ++n) o[hb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- compute the staged tile, then stage the one in flight and put the
    // wave's next tile (of this segment, else its first of the next) in flight
    // Split int4 tiles: while half 0 of `tile` is computed, its half 1 and
    // half 0 of next_tile are in flight; half 1 is staged (and next_tile's
    // half 1 issued) before it is computed, in the next pass of the loop.
    int half = 0;  // the staged half of `tile`
    while (tile < cur.ntile) {
      const int tt0 = t_begin + tile * TT + (SPLIT2 ? half * kTile : 0);
      if constexpr (M32) {
        const int l32 = lane & 31, h2 = lane >> 5;
        // ---- S^T[32 tokens][32 heads] = K Q^T: lane holds tokens 8(r/4)+4h2+r%4 of head l32
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kf = lds_load<u32x4>(kt + l32 * (2 * D) + (((2 * ks + h2) ^ swz<CH>(l32)) << 4));
          const u32x4 qf = lds_load<u32x4>(sq + l32 * (2 * D) + (((2 * ks + h2) ^ swz<CH>(l32)) << 4));
          sacc = mfma32(kf, qf, sacc);
        }
        if (tt0 + kTile > t_end) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[r] = tt0 + 8 * (r >> 2) + 4 * h2 + (r & 3) < t_end ? sacc[r] : kNegInf;
        }
        // lane-local check first; the exchange only when a score exceeds the
        // reference by more than the slack (as in the 16 x 16 path below)
        float mt = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
        bool grow = false;
        float alpha = 1.0f;
        if (__builtin_amdgcn_ballot_w64(mt * a.qk_scale_log2 > m[0] + kRescaleSlack)) {
          mt = wave_max_xor(mt, 32) * a.qk_scale_log2;
          grow = mt > m[0] + kRescaleSlack;
          const float m_new = grow ? mt : m[0];
          alpha = grow ? fast_exp2(m[0] - m_new) : 1.0f;
          m[0] = m_new;
        }
        const float m_new = m[0];
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = fast_exp2(__builtin_fmaf(sacc[r], a.qk_scale_log2, -m_new));
          psum += sacc[r];
        }
        l[0] = l[0] * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
          for (int n = 0; n < NT32; ++n) o32[n] *= alpha;
        }
        // ---- O^T += V^T P^T, two k-steps of 16 tokens (token order permuted as in S)
        const int gi = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const u32x4 pf = {pack_bf16x2(sacc[8 * p + 0], sacc[8 * p + 1]), pack_bf16x2(sacc[8 * p + 2], sacc[8 * p + 3]),
                            pack_bf16x2(sacc[8 * p + 4], sacc[8 * p + 5]), pack_bf16x2(sacc[8 * p + 6], sacc[8 * p + 7])};
          const int ra = 16 * p + 4 * h2 + (s16 >> 2), rb = ra + 8;
#pragma unroll
          for (int n = 0; n < NT32; ++n) {
            const int col = 32 * n + 16 * (gi & 1) + 4 * (s16 & 3);
            const int c = col >> 3, wsub = col & 7;
            const u32x2 va = lds_read_tr16(vt + ra * (2 * D) + ((c ^ swz<CH>(ra)) << 4) + 2 * wsub);
            const u32x2 vb = lds_read_tr16(vt + rb * (2 * D) + ((c ^ swz<CH>(rb)) << 4) + 2 * wsub);
            o32[n] = mfma32(u32x4{va[0], va[1], vb[0], vb[1]}, pf, o32[n]);
          }
        }
      } else {
        // ---- scores S^T[token][head]: two 16-token halves
        f32x4 sc[2][HB];
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 16 * h + r16;
          u32x4 kf[KK];
          if constexpr (KDIR && KVF == kKvInt4) {
  #pragma unroll
            for (int kk = 0; kk < KK; ++kk) kf[kk] = i4x8_to_bf16x8_biased_eo(kcur[h][kk]);
          } else if constexpr (KDIR) {  // 8-bit codes d = 32 q4 + 8 kk .. +7: bytes 8 kk .. of the lane's 32
  #pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
              const u32x4& w = kcur[2 * h + (kk >> 1)];
              u32x2 lo4, hi4;
              if constexpr (KVF == kKvFp8) {
                lo4 = e4m3x4_to_bf16x4(w[2 * (kk & 1)]);
                hi4 = e4m3x4_to_bf16x4(w[2 * (kk & 1) + 1]);
              } else {
                lo4 = i8x4_to_bf16x4(w[2 * (kk & 1)]);
                hi4 = i8x4_to_bf16x4(w[2 * (kk & 1) + 1]);
              }
              kf[kk] = u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
            }
          } else {
  #pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              kf[kk] = lds_load<u32x4>(kt + row * (2 * D) + (((4 * kk + q4) ^ swz<CH>(row)) << 4));
          }
  #pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            // B operand of S^T = K Q^T: lane holds Q[head 16hb + r16][32kk + 8q4 .. +7]
            const int qrow = 16 * hb + r16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BIAS4) acc = f32x4{kbias[hb], kbias[hb], kbias[hb], kbias[hb]};
  #pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              acc = mfma16(kf[kk],
                           KDIR ? qreg[kk]
                                : lds_load<u32x4>(sq + qrow * (2 * D) + (((4 * kk + q4) ^ swz<CH>(qrow)) << 4)),
                           acc);
            sc[h][hb] = acc;
          }
        }
        // direct K (raw V): codes of d-tiles 2p and 2p + 1 over the lane's k-slots
        auto v_raw = [&](int pp) {
          const int L = r16 & 7;
          const int row = 16 * (L >> 2) + 4 * q4 + (L & 3);  // token of k-slot 8 q4 + L
          const int c = 2 * pp + (r16 >> 3);
          const auto v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(vt + row * ROWB + 8 * (c ^ vsw(row))));
          return __builtin_bit_cast(u32x2, v);
        };
        constexpr int NRAW = V4RAW ? NT / 2 : 1;
        u32x2 vraw[NRAW];
        if constexpr (V4RAW) {
  #pragma unroll
          for (int pp = 0; pp < NRAW; ++pp) vraw[pp] = v_raw(pp);  // latency hidden by the softmax
        }
        // V^T fragment n of the staged tile: lane holds V[token k-slot 8 q4 + j][d = 16 n + r16]
        auto v_frag = [&](int n) {
          const int col = 16 * n + 4 * (r16 & 3);  // bf16 column
          const int c = col >> 3, wsub = col & 7;
          const int row_lo = 4 * q4 + (r16 >> 2);
          const int row_hi = 16 + row_lo;
          const u32x2 lo2 = lds_read_tr16(vt + row_lo * (2 * D) + ((c ^ swz<CH>(row_lo)) << 4) + 2 * wsub);
          const u32x2 hi2 = lds_read_tr16(vt + row_hi * (2 * D) + ((c ^ swz<CH>(row_hi)) << 4) + 2 * wsub);
          return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        };
        // the first fragments are read now, so their latency hides under the softmax
        constexpr int NPRE_ = V4RAW ? 0 : NPRE;
        u32x4 vpre[NPRE_ > 0 ? NPRE_ : 1];
  #pragma unroll
        for (int n = 0; n < NPRE_; ++n) vpre[n] = v_frag(n);
        // ---- online softmax per head block -> bf16 probabilities (B operand of PV).
        // The reference max moves only when a tile's max exceeds it by more than
        // kRescaleSlack (log2 units): O and l always share the same reference, so
        // the result is unchanged, p stays <= 2^kRescaleSlack, and the rescale of
        // O is skipped on almost every tile.
        const bool tail = tt0 + kTile > t_end;
        u32x4 pf[HB];
        bool any_grow = false;
        float alpha[HB];
        f32x4 kscur[2], vscur[2];  // scales of rows 16h + 4q4 + i (unused for bf16)
        if constexpr (QUANT) {
  #pragma unroll
          for (int h = 0; h < 2; ++h) {
            kscur[h] = lds_load<f32x4>(&ssc[wave][16 * h + 4 * q4]);
            vscur[h] = lds_load<f32x4>(&ssc[wave][32 + 16 * h + 4 * q4]);
          }
        }
        // Each lane first checks its own scores against the reference: only
        // if one of them exceeds it by more than the slack (a head's first
        // tile of the segment, as a rule) does the wave form the per-head
        // tile maxima with the cross-lane exchanges and move the reference.
        // The head-wide test is the same one, so the result is unchanged.
        float sv[HB][2][4];
        float lmax[HB];
        bool need = false;
  #pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          lmax[hb] = kNegInf;
  #pragma unroll
          for (int h = 0; h < 2; ++h)
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sc[h][hb][i];
              if constexpr (QUANT) x *= kscur[h][i];  // the per-token K scale (> 0)
              sv[hb][h][i] = x;
            }
          if (tail) {
  #pragma unroll
            for (int h = 0; h < 2; ++h)
  #pragma unroll
              for (int i = 0; i < 4; ++i) sv[hb][h][i] = tt0 + 16 * h + 4 * q4 + i < t_end ? sv[hb][h][i] : kNegInf;
          }
  #pragma unroll
          for (int h = 0; h < 2; ++h)
  #pragma unroll
            for (int i = 0; i < 4; ++i) lmax[hb] = fmaxf(lmax[hb], sv[hb][h][i]);
          need = need || lmax[hb] * a.qk_scale_log2 > m[hb] + kRescaleSlack;  // scale > 0 keeps the order
          alpha[hb] = 1.0f;
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
  #pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            float mt = wave_max_xor(lmax[hb], 16);
            mt = wave_max_xor(mt, 32) * a.qk_scale_log2;
            const bool grow = mt > m[hb] + kRescaleSlack;
            const float m_new = grow ? mt : m[hb];
            alpha[hb] = grow ? fast_exp2(m[hb] - m_new) : 1.0f;
            any_grow = any_grow || grow;
            m[hb] = m_new;
          }
        }
  #pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          float psum = 0.f;
          float p[2][4];
  #pragma unroll
          for (int h = 0; h < 2; ++h)
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[h][i] = fast_exp2(__builtin_fmaf(sv[hb][h][i], a.qk_scale_log2, -m[hb]));
              psum += p[h][i];
            }
          l[hb] = l[hb] * alpha[hb] + psum;
          if constexpr (QUANT) {
  #pragma unroll
            for (int h = 0; h < 2; ++h)
  #pragma unroll
              for (int i = 0; i < 4; ++i) p[h][i] *= vscur[h][i];
          }
          if constexpr (V4RAW)  // k-slots in the order 0 2 4 6 1 3 5 7 of the converted V codes
            pf[hb] = u32x4{pack_bf16x2(p[0][0], p[0][2]), pack_bf16x2(p[1][0], p[1][2]), pack_bf16x2(p[0][1], p[0][3]),
                           pack_bf16x2(p[1][1], p[1][3])};
          else
            pf[hb] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]), pack_bf16x2(p[1][0], p[1][1]),
                           pack_bf16x2(p[1][2], p[1][3])};
        }
        if (__builtin_amdgcn_ballot_w64(any_grow)) {
  #pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
  #pragma unroll
            for (int n = 0; n < NT; ++n) o[hb][n] *= alpha[hb];
            if constexpr (BIAS4) osum[hb] *= alpha[hb];
          }
        }
        // ---- O^T += V^T P^T: one 16-wide d tile of V at a time, shared by all head blocks
        // (the first NPRE fragments were read before the softmax)
  #pragma unroll
        for (int n = 0; n < NT; ++n) {
          u32x4 vf;
          if constexpr (V4RAW) vf = i4x8_to_bf16x8_biased_eo(vraw[n >> 1][n & 1]);
          else vf = n < NPRE_ ? vpre[n < NPRE_ ? n : 0] : v_frag(n);
  #pragma unroll
          for (int hb = 0; hb < HB; ++hb) o[hb][n] = mfma16(vf, pf[hb], o[hb][n]);
        }
        if constexpr (BIAS4) {
  #pragma unroll
          for (int hb = 0; hb < HB; ++hb) osum[hb] = mfma16(ones_row0, pf[hb], osum[hb]);
        }
      }
      if constexpr (SPLIT2) {
        if (half == 0) {
          stage(1);
          issue_next(next_tile, 1);
          half = 1;
          if (tt0 + kTile < t_end) continue;  // half 1 holds tokens: compute it next
        }
        half = 0;
      }
      tile = next_tile;
      if (tile >= cur.ntile) break;
      stage(0);
      next_tile = claim_tile(tile);
      issue_next(next_tile, 0);
    }

    // ---- merge the waves of the workgroup, write one partial per head
    wave_lds_fence();
    if constexpr (M32) {
      // O^T[d = 32n + 8(r/4) + 4h2 + r%4][head l32] -> ow[head][d]
      const int l32 = lane & 31, h2 = lane >> 5;
      l[0] = wave_sum_xor(l[0], 32);
#pragma unroll
      for (int n = 0; n < NT32; ++n)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          lds_store(ow + ow_idx(l32, 32 * n + 8 * rq + 4 * h2),
                    f32x4{o32[n][4 * rq], o32[n][4 * rq + 1], o32[n][4 * rq + 2], o32[n][4 * rq + 3]});
      if (h2 == 0) {
        sm_ml[wave][l32][0] = m[0];
        sm_ml[wave][l32][1] = l[0];
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float lt = wave_sum_xor(l[hb], 16);
        lt = wave_sum_xor(lt, 32);
        l[hb] = lt;
      }
      if constexpr (BIAS4) {
        // remove 136 sum_t p_t (held by lane r16 of each head block)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const float c = kInt4Bias * __shfl(osum[hb][0], r16, 64);
#pragma unroll
          for (int n = 0; n < NT; ++n) o[hb][n] -= c;
        }
      }
      // O^T[d = 16n + 4q4 + i][head r16] -> ow[head][d] (float32), reusing the wave slab
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if constexpr (BIAS4 && !V4RAW) {
            // staged column 16n + 4q4 + i holds d = 16n + 8(q4/2) + 2i + q4%2
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ow[ow_idx(hb * 16 + r16, 16 * n + 8 * (q4 >> 1) + 2 * i + (q4 & 1))] = o[hb][n][i];
          } else {
            lds_store(ow + ow_idx(hb * 16 + r16, 16 * n + 4 * q4), o[hb][n]);
          }
        }
        if (q4 == 0) {
          sm_ml[wave][hb * 16 + r16][0] = m[hb];
          sm_ml[wave][hb * 16 + r16][1] = l[hb];
        }
      }
    }
    __syncthreads();
    // each thread merges whole 16-byte chunks (4 consecutive d of one head);
    // the trip count is a compile-time constant so the loads of all its
    // chunks are in flight together
    constexpr int D4 = D / 4;
#pragma unroll
    for (int i = 0; i < (HPC * D4 + NW * 64 - 1) / (NW * 64); ++i) {
      const int e4 = threadIdx.x + i * NW * 64;
      const int hl = e4 / D4, q = e4 - hl * D4;
      if (e4 < HPC * D4 && hl < cur.nh) {
        float M = kNegInf;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, sm_ml[wv][hl][0]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
          const float mw = sm_ml[wv][hl][0];
          const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
          acc += f * lds_load<f32x4>(reinterpret_cast<const float*>(smem[wv][0]) + ow_idx(hl, 4 * q));
          lsum += f * sm_ml[wv][hl][1];
        }
        const size_t row = (size_t)cur.slot * HPC + hl;
        *reinterpret_cast<f32x4*>(a.part_o + row * D + 4 * q) = acc;
        if (q == 0) {
          a.part_ml[row * 2 + 0] = M;
          a.part_ml[row * 2 + 1] = lsum;
        }
      }
    }
    if (!has_next) break;
    qc = q_next;
    __syncthreads();  // the merge's reads of the slabs are done before the next prologue stages into them
    lo += cur.ntile;
    cur = nxt;
  }
}

// ------------------------------------------------------------------------
// float32 decode on the vector ALUs (16 heads per workgroup, 4 waves,
// 64-token tiles: one token per lane for the scores, one d column per lane
// for the PV product).
// ------------------------------------------------------------------------
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void gqa_decode_split_f32(DecodeArgs a) {
  constexpr int HPC = 16;
  constexpr int NW = kWavesF32;
  constexpr int DL = D / 64;  // d columns per lane in the PV product
  __shared__ __attribute__((aligned(16))) float sq[HPC][D];
  __shared__ float sp[NW][kTileF32][HPC];
  __shared__ __attribute__((aligned(16))) float so[NW][HPC][D];
  __shared__ float sm_ml[NW][HPC][2];

  const int W = gridDim.x;
  const int w = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int spb = a.n_kv * a.n_hchunk;
  const int G = a.h_q / a.n_kv;
  const long long T = tiles_before(a.seq_lens, a.B, a.S_max, kTileF32, spb, lane);
  const TileRanges rg(T, W);
  const long long lo = rg.lo(w);
  const long long hi = rg.lo(w + 1);
  const float* qg = static_cast<const float*>(a.q);
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);

  for (long long t = lo; t < hi;) {
    int b, nt, L;
    long long base;
    locate_tile(a.seq_lens, a.B, a.S_max, kTileF32, spb, t, lane, b, base, nt, L);
    int slab_in_b, tile0;
    split_local(t - base, nt, slab_in_b, tile0);
    const int seg = (int)min(hi - t, (long long)(nt - tile0));
    const int g = slab_in_b / a.n_hchunk;
    const int hc = slab_in_b - g * a.n_hchunk;
    const long long slot = w + (long long)b * spb + slab_in_b;
    t += seg;

    const int t_begin = tile0 * kTileF32;
    const int t_end = min((tile0 + seg) * kTileF32, L);
    const int hloc0 = hc * HPC;
    const int nh = min(HPC, G - hloc0);
    const int head0 = g * G + hloc0;

    for (int e = threadIdx.x; e < HPC * D; e += NW * 64) {
      const int hl = e / D, d = e - hl * D;
      sq[hl][d] = hl < nh ? qg[((size_t)b * a.h_q + head0 + hl) * D + d] : 0.f;
    }
    __syncthreads();

    const size_t slab = ((size_t)b * a.n_kv + g) * (size_t)a.S_max;
    float m[HPC], l[HPC], o[HPC][DL];
#pragma unroll
    for (int h = 0; h < HPC; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) o[h][c] = 0.f;
    }

    for (int tile = wave; tile < seg; tile += NW) {
      const int tt0 = t_begin + tile * kTileF32;
      const int tok = tt0 + lane;
      const bool valid = tok < t_end;
      // cache row of this lane's token (the segment's last one past the end);
      // paged: one block-table lookup per lane
      size_t row = slab + min(tok, t_end - 1);
      if constexpr (PAGED) {
        const int tc = min(tok, t_end - 1);
        int page = a.block_table[(size_t)b * a.max_pages + (tc >> a.page_shift)];
        page = min(max(page, 0), a.num_pages - 1);
        row = (((size_t)page * a.n_kv + g) << a.page_shift) | (size_t)(tc & ((1 << a.page_shift) - 1));
      }
      float sc[HPC];
#pragma unroll
      for (int h = 0; h < HPC; ++h) sc[h] = 0.f;
      if (valid) {
        const float4* kr = reinterpret_cast<const float4*>(kg + row * D);
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kv = kr[d4];
#pragma unroll
          for (int h = 0; h < HPC; ++h) {
            const float4 qv = *reinterpret_cast<const float4*>(&sq[h][4 * d4]);
            sc[h] = fmaf(qv.x, kv.x, sc[h]);
            sc[h] = fmaf(qv.y, kv.y, sc[h]);
            sc[h] = fmaf(qv.z, kv.z, sc[h]);
            sc[h] = fmaf(qv.w, kv.w, sc[h]);
          }
        }
      }
      float alpha[HPC];
#pragma unroll
      for (int h = 0; h < HPC; ++h) {
        const float x = valid ? sc[h] * a.qk_scale_log2 : kNegInf;
        float mt = x;
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) mt = wave_max_xor(mt, msk);
        const float m_new = fmaxf(m[h], mt);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        alpha[h] = fast_exp2(m[h] - m_use);
        m[h] = m_new;
        const float p = fast_exp2(x - m_use);
        l[h] = l[h] * alpha[h] + p;
        sp[wave][lane][h] = p;
      }
      wave_lds_fence();
      const int nvalid = min(kTileF32, t_end - tt0);
#pragma unroll
      for (int h = 0; h < HPC; ++h)
#pragma unroll
        for (int c = 0; c < DL; ++c) o[h][c] *= alpha[h];
      // V rows U at a time: all U loads are issued before the first use;
      // rows past the last valid one are re-reads of it and are skipped
      constexpr int U = 64 / DL;
      for (int tt = 0; tt < nvalid; tt += U) {
        float vv[U][DL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int src = min(tt + u, nvalid - 1);  // a lane of this tile (uniform)
          const size_t vrow = ((size_t)(uint32_t)__builtin_amdgcn_readlane((int)(row >> 32), src) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)row, src);
          const float* vr = vg + vrow * D;
#pragma unroll
          for (int c = 0; c < DL; ++c) vv[u][c] = vr[lane + 64 * c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (tt + u >= nvalid) break;
#pragma unroll
          for (int h = 0; h < HPC; ++h) {
            const float p = sp[wave][tt + u][h];
#pragma unroll
            for (int c = 0; c < DL; ++c) o[h][c] = fmaf(p, vv[u][c], o[h][c]);
          }
        }
      }
      wave_lds_fence();
    }
#pragma unroll
    for (int h = 0; h < HPC; ++h) {
      float lt = l[h];
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) lt = wave_sum_xor(lt, msk);
#pragma unroll
      for (int c = 0; c < DL; ++c) so[wave][h][lane + 64 * c] = o[h][c];
      if (lane == 0) {
        sm_ml[wave][h][0] = m[h];
        sm_ml[wave][h][1] = lt;
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * D; e += NW * 64) {
      const int hl = e / D, d = e - hl * D;
      float M = kNegInf;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, sm_ml[wv][hl][0]);
      float acc = 0.f, lsum = 0.f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float mw = sm_ml[wv][hl][0];
        const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
        acc += f * so[wv][hl][d];
        lsum += f * sm_ml[wv][hl][1];
      }
      const size_t row = (size_t)slot * HPC + hl;
      a.part_o[row * D + d] = acc;
      if (d == 0) {
        a.part_ml[row * 2 + 0] = M;
        a.part_ml[row * 2 + 1] = lsum;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------
// Combine: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s, over the partials of one slab.
// ------------------------------------------------------------------------
// The partials of the slab whose tiles are [first, first + nt) of the global
// range [0, T) cut into W workgroup ranges: one per workgroup whose range
// touches the slab.  When T >= W every range is non-empty, so these are the
// workgroups from the owner of the slab's first tile to the owner of its last;
// when T < W a range holds at most one tile and the owners go tile by tile.
struct SlabPieces {
  TileRanges rg;
  long long first, wa, sigma;
  int nt, n;
  __device__ __forceinline__ SlabPieces(long long sigma_, long long first_, int nt_, long long T_, int W_)
      : rg(T_, W_), first(first_), wa(rg.owner(first_)), sigma(sigma_), nt(nt_) {
    n = nt == 0 ? 0 : T_ >= W_ ? (int)(rg.owner(first + nt - 1) - wa + 1) : nt;
  }
  __device__ __forceinline__ long long slot(int p) const {
    return (rg.T >= rg.W ? wa + p : rg.owner(first + p)) + sigma;
  }
};

// Merges the partials of one slab into its nh output rows (heads head0 ..
// head0 + nh - 1 of sequence b).  Thread tid of nthreads takes the elements
// tid, tid + nthreads, ... of the nh x D/4 grid of 4-column groups; each
// element folds the pieces with a running maximum, four at a time with all
// eight loads of a batch in flight together (indices past the last piece
// repeat it and are skipped).
template <int D, bool OUT_BF16>
__device__ __forceinline__ void merge_slab(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                           void* __restrict__ out, int hpc, int h_q, int b, int head0, int nh,
                                           const SlabPieces& sp, int tid, int nthreads) {
  constexpr int D4 = D / 4;
  constexpr int PB = 4;  // pieces per batch
  for (int e = tid; e < nh * D4; e += nthreads) {
    const int hl = e / D4, d4 = e - hl * D4;
    float M = kNegInf, denom = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < sp.n; p0 += PB) {
      f32x2 ml[PB];
      f32x4 os[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const size_t row = (size_t)sp.slot(min(p0 + u, sp.n - 1)) * hpc + hl;
        ml[u] = *reinterpret_cast<const f32x2*>(part_ml + row * 2);
        os[u] = *reinterpret_cast<const f32x4*>(part_o + row * D + 4 * d4);
      }
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const float ms = ml[u][0], ls = ml[u][1];
        if (p0 + u >= sp.n || ms == kNegInf) continue;  // past the last piece, or a piece with no visible key
        if (ms > M) {
          const float r = M == kNegInf ? 0.f : fast_exp2(M - ms);
          acc *= r;
          denom *= r;
          M = ms;
        }
        const float f = fast_exp2(ms - M);
        acc += f * os[u];
        denom += f * ls;
      }
    }
    acc *= denom > 0.f ? 1.0f / denom : 0.f;
    const size_t idx = ((size_t)b * h_q + head0 + hl) * D + 4 * d4;
    if constexpr (OUT_BF16) {
      u32x2 wv;
      wv[0] = pack_bf16x2(acc[0], acc[1]);
      wv[1] = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx) = wv;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = acc;
    }
  }
}

// One workgroup per (slab, chunk of 256 elements): each thread merges one
// 4-column group of one head, so every partial row is read by a single load.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void gqa_decode_combine(CombineArgs c) {
  const int sigma = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int spb = c.n_kv * c.n_hchunk;
  const int b = sigma / spb;
  const int slab_in_b = sigma - b * spb;
  const int g = slab_in_b / c.n_hchunk;
  const int hc = slab_in_b - g * c.n_hchunk;
  const int G = c.h_q / c.n_kv;
  const int hloc0 = hc * c.heads_per_chunk;
  const int nh = min(c.heads_per_chunk, G - hloc0);
  const LaneLens ll = load_lane_lens(c.seq_lens, c.B, c.S_max, lane);
  long long T, before_b;
  int nt;
  slab_position(ll, c.seq_lens, c.B, c.S_max, c.tile, spb, b, lane, T, before_b, nt);
  const int tid = blockIdx.y * 256 + threadIdx.x;
  if (nt == 0) {  // empty sequence: zero rows
    const SlabPieces none(sigma, 0, 0, 1, 1);
    merge_slab<D, OUT_BF16>(c.part_o, c.part_ml, c.out, c.heads_per_chunk, c.h_q, b, g * G + hloc0, nh,
                                   none, tid, gridDim.y * 256);
    return;
  }
  const long long first = before_b + (long long)slab_in_b * nt;
  const SlabPieces sp(sigma, first, nt, T, c.W);
  merge_slab<D, OUT_BF16>(c.part_o, c.part_ml, c.out, c.heads_per_chunk, c.h_q, b, g * G + hloc0, nh, sp,
                                 tid, gridDim.y * 256);
}

// ------------------------------------------------------------------------
// Host-side launchers (called from api.hip).
// ------------------------------------------------------------------------
constexpr int kWavesMfma = 8;

template <bool PAGED>
static void launch_split(const DecodeArgs& a, int D, int hb, int kind, int W, hipStream_t stream) {
  const dim3 grid(W);
  if (kind == 0) {
    const dim3 block(kWavesF32 * 64);
    if (D == 64) hipLaunchKernelGGL((gqa_decode_split_f32<64, PAGED>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_split_f32<128, PAGED>), grid, block, 0, stream, a);
    return;
  }
  const dim3 block(kWavesMfma * 64);
#define GQA_LAUNCH_DECODE(DD, HH, F) \
  hipLaunchKernelGGL((gqa_decode_split_mfma<DD, HH, F, kWavesMfma, PAGED>), grid, block, 0, stream, a)
#define GQA_LAUNCH_DECODE_KVF(DD, HH)                     \
  switch (kind) {                                         \
    case 2: GQA_LAUNCH_DECODE(DD, HH, kKvFp8); break;     \
    case 3: GQA_LAUNCH_DECODE(DD, HH, kKvInt8); break;    \
    case 4: GQA_LAUNCH_DECODE(DD, HH, kKvInt4); break;    \
    default: GQA_LAUNCH_DECODE(DD, HH, kKvBf16); break;   \
  }
  if (D == 64) {
    if (hb == 1) GQA_LAUNCH_DECODE_KVF(64, 1) else GQA_LAUNCH_DECODE_KVF(64, 2)
  } else {
    if (hb == 1) GQA_LAUNCH_DECODE_KVF(128, 1) else GQA_LAUNCH_DECODE_KVF(128, 2)
  }
#undef GQA_LAUNCH_DECODE_KVF
#undef GQA_LAUNCH_DECODE
}

hipError_t launch_decode_split(const DecodeArgs& a, int D, int hb, int kind, int W, hipStream_t stream) {
  if (a.block_table) launch_split<true>(a, D, hb, kind, W, stream);
  else launch_split<false>(a, D, hb, kind, W, stream);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const CombineArgs& c, int D, bool out_bf16, hipStream_t stream) {
  // a chunk holds at most G heads: no workgroups for the chunk's unused head rows
  const int heads = min(c.heads_per_chunk, c.h_q / c.n_kv);
  const dim3 grid(c.B * c.n_kv * c.n_hchunk, (heads * D / 4 + 255) / 256);
  const dim3 block(256);
  switch (D) {
    case 64:
      if (out_bf16) hipLaunchKernelGGL((gqa_decode_combine<64, true>), grid, block, 0, stream, c);
      else hipLaunchKernelGGL((gqa_decode_combine<64, false>), grid, block, 0, stream, c);
      break;
    case 128:
      if (out_bf16) hipLaunchKernelGGL((gqa_decode_combine<128, true>), grid, block, 0, stream, c);
      else hipLaunchKernelGGL((gqa_decode_combine<128, false>), grid, block, 0, stream, c);
      break;
    case 256:  // latent attention (bf16 output only)
      hipLaunchKernelGGL((gqa_decode_combine<256, true>), grid, block, 0, stream, c);
      break;
    default:  // 512, latent attention
      hipLaunchKernelGGL((gqa_decode_combine<512, true>), grid, block, 0, stream, c);
      break;
  }
  return hipGetLastError();
}

}  // namespace gqa
