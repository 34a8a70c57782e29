// Causal prefill kernel (bf16 in, float32 statistics, bf16 out).
//
// Computes, for every batch entry b, query head j (K/V head g = j / G) and
// query row r, softmax over keys 0..r of scale * q_r . k_c, applied to V --
// the causal mode of the flash_attn_func call in "Flash Attention Usage"
// ("Evolution of AI Attention Mechanisms"), token-major [B, S, H, d] layout.
// The score matrix is never written to memory: K and V move through LDS in
// 64-key tiles, the scores live in registers, and a running max / running sum
// per query row rescales the output accumulator ("Flash Attention Principle":
// tiled computation, softmax on chip, only the final O written back).
//
// Work decomposition (MI355X-specific, not the pages' GPU):
//  * a workgroup of 8 wavefronts (one workgroup per compute unit) serves HC
//    query heads of ONE K/V group over 32*(8/HC) query rows, so every K/V
//    tile it stages in LDS feeds 8 waves (GQA: the G heads of a group read the
//    same K/V), which halves the global->LDS traffic per flop against
//    4-wave workgroups at the same register occupancy;
//  * each wave owns 32 query rows of one head: S^T[key][query] = K Q^T and
//    O^T[d][query] += V^T P^T on v_mfma_f32_32x32x16_bf16.  The key order in
//    the PV product is permuted so the score accumulator registers are the B
//    operand as they stand, and V is read transposed with ds_read_b64_tr_b16;
//    every per-row statistic is then lane-local except one exchange with the
//    lane 32 apart;
//  * K/V tiles are double-buffered: the next tile's global loads are in flight
//    while the current one feeds the matrix cores;
//  * key tiles entirely above the diagonal are never visited (about half the
//    work of the dense product); only tiles crossing it apply the mask;
//  * workgroups are numbered so that each of the 8 XCDs (own L2 each) works
//    through a contiguous range of (batch, K/V head) groups -- their K/V then
//    stays in that XCD's L2 -- and within a group the longest (latest) query
//    blocks start first.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float qk_scale_log2;
  int B, S, h_q, n_kv;  // S = query rows (S_q)
  int n_qb, n_hc, n_wg, n_wg_pad;
  int grp_block;            // groups (batch, K/V head, head chunk) interleaved per row block (1: none)
  int batch_minor;          // groups numbered batch entry fastest (1) or K/V head chunk fastest (0)
  // general masks (the masked kernel only)
  int S_k;                  // keys per sequence
  int causal;               // query r sees keys c <= r + S_k - S_q
  const int32_t* kv_lens;   // [B] or null: keys c >= kv_lens[b] are invisible and never read
  const uint8_t* mask;      // [B][S][S_k] or null: key c invisible to row r where 0
  // with a mask: the row blocks' key-tile bitmaps, formed by a pass over the
  // mask before the kernel (null: each workgroup scans its mask rows);
  // [B][n_qb][2][mt_words] (visible, then fully visible)
  const uint32_t* mask_tiles;
  int mt_words;
  // fp8 kernel: q/k/v hold e4m3 codes; value = code * descale[b][head]
  const float* q_descale;   // [B][h_q]
  const float* k_descale;   // [B][n_kv]
  const float* v_descale;   // [B][n_kv]
};

constexpr int kBN = 64;  // keys per tile
// With a dense mask, groups interleaved per row block (workgroup order): the
// workgroups of 4 groups that read the same mask rows run side by side on one
// XCD.  Measured on the packed-document workload (4 x 4096, 8 K/V heads):
// 1 -> 372-378 us and 596 MB fetched, 4 -> 335-346 us and 362 MB, 8 -> 383 us
// and 429 MB (the K/V of 8 groups no longer fits one XCD's L2).
constexpr int kMaskGroupBlock = 4;
constexpr int kNumXcd = 8;
constexpr int kWaves = 8;  // wavefronts per workgroup

// Key-tile bitmaps of one row block (BM rows from the block's first) under a
// dense mask, into the workgroup's LDS words vis / full (kVisWords each): bit j
// of vis is set when some mask byte of the rows over the keys of tile j is
// nonzero, bit j of full when none of them is zero.  mrsrc covers the block's
// mask rows; rows past nrows do not count.  Tiles j_begin .. j_end - 1 are
// scanned (bits of other tiles stay clear).  The rows are read in order: a
// load instruction covers 1 KiB of one row (16 tiles, four lanes a tile), each
// wave takes BM / kWaves rows and issues the loads of two 16-tile segments of
// all its rows before it uses any (lanes of tiles past the range load
// nothing); the four lanes of a tile then combine by
// shuffles, and the waves by LDS atomics (OR into vis, and into full as
// "some byte is zero" bits, inverted at the end).  Called by all kWaves waves
// of the workgroup.
constexpr int kVisWords = 256;  // up to 8192 key tiles
template <int BM>
__device__ void scan_mask_tiles(__amdgpu_buffer_rsrc_t mrsrc, int j_begin, int j_end, int nrows, int SK,
                                uint32_t* vis, uint32_t* full, int wave, int lane, int tid) {
  for (int i = tid; i < kVisWords; i += kWaves * 64) {
    vis[i] = 0u;
    full[i] = 0u;
  }
  __syncthreads();
  static_assert(kBN == 64, "the scan assumes 64-key tiles");
  constexpr int RPW = BM / kWaves;  // rows per wave
  constexpr int RB = RPW < 8 ? RPW : 8;
  const int s_end = (j_end + 15) >> 4;  // 16-tile segments
  for (int s0 = j_begin >> 4; s0 < s_end; s0 += 2) {
    uint32_t any[2] = {0u, 0u}, zero[2] = {0u, 0u};
    // rows past nrows lie past the resource's range and read as zero: they
    // are loaded like the others and only kept out of the zero test
    for (int i0 = 0; i0 < RPW; i0 += RB) {  // RB rows' loads in flight at a time
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int r = wave * RPW + i0 + i;
        const uint32_t valid = r < nrows ? 0x80808080u : 0u;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const unsigned off = (unsigned)r * (unsigned)SK + (unsigned)((s0 + u) * 16 * kBN + 16 * lane);
          // lanes of tiles past the range load nothing
          u32x4 mv = {0u, 0u, 0u, 0u};
          if ((s0 + u) * 16 + (lane >> 2) < j_end) mv = buffer_load_x4(mrsrc, off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            any[u] |= mv[e];
            zero[u] |= (mv[e] - 0x01010101u) & ~mv[e] & valid;  // nonzero iff a byte is 0
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t av = any[u], zv = zero[u];
      av |= __shfl_xor(av, 1, 64);
      zv |= __shfl_xor(zv, 1, 64);
      av |= __shfl_xor(av, 2, 64);
      zv |= __shfl_xor(zv, 2, 64);
      const int j = (s0 + u) * 16 + (lane >> 2);
      if ((lane & 3) == 0 && j >= j_begin && j < j_end) {
        if (av) atomicOr(&vis[j >> 5], 1u << (j & 31));
        if (zv) atomicOr(&full[j >> 5], 1u << (j & 31));
      }
    }
  }
  __syncthreads();
  // full held "some byte is zero": invert it over the scanned tiles
  for (int i = tid; i < kVisWords; i += kWaves * 64) {
    const int lo = max(j_begin - 32 * i, 0), hi = min(j_end - 32 * i, 32);
    const uint32_t range = lo >= hi ? 0u : (hi == 32 ? ~0u : (1u << hi) - 1u) & ~((1u << lo) - 1u);
    full[i] = ~full[i] & range;
  }
  __syncthreads();
}

// Key tiles a row block [blk0, row_end) must consider: those holding keys
// below the last row's visible prefix (the causal rule, end-aligned, and the
// key length), before any dense mask.
__device__ __forceinline__ int block_key_tiles(int row_end, int S, int SK, int kv_n, int causal) {
  const int kend = causal ? max(min(kv_n, min(row_end - 1, S - 1) + 1 + SK - S), 0) : kv_n;
  return (kend + kBN - 1) / kBN;
}

// GEN = false: causal self-attention, S_q = S_k, every key of a row's causal
// range visible.  GEN = true: S_q and S_k independent, the causal rule
// optional and end-aligned, optional key lengths and dense mask; rows can
// then have no visible key at all (zero output).
// F8: q, k, v are OCP e4m3 codes with one descale factor per (batch, head)
// (the FP8 mode of FlashAttention-3, "Flash Attention 3 Features"); both
// products run on v_mfma_f32_32x32x64_f8f6f4, d = 64 or 128.  The softmax
// weights enter the second product as two e4m3 terms, p = hi + lo with hi =
// e4m3(p) and lo = e4m3(p - hi) (two products per d tile), so each weight
// carries a relative error of at most 2^-8 (2^-10 absolute for the smallest)
// instead of the 2^-4 of a single e4m3 value; the reference max keeps every
// p <= 256, below the format's 448.
// MASK (with GEN): a dense mask is given; without it the mask machinery
// (tile bitmaps, mask tiles, per-element masking) is compiled out.
template <int D, int HC, bool GEN, bool F8 = false, bool MASK = false>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a) {
  static_assert(!F8 || GEN, "the fp8 body serves general masks");
  constexpr int RB = kWaves / HC;  // 32-row blocks per head in one workgroup
  constexpr int BM = 32 * RB;    // query rows per workgroup
  constexpr int EB = F8 ? 1 : 2; // bytes per element
  constexpr int ROWB = D * EB;   // bytes per K/V row
  constexpr int CH = ROWB / 16;  // 16-byte chunks per K/V row
  constexpr int KS = D / 16;     // k-steps of the bf16 score product
  constexpr int KS8 = D / 64;    // k-steps of the fp8 score product
  constexpr int NT = D / 32;     // 32-wide d tiles of the PV product
  constexpr int TILE_BYTES = kBN * ROWB;
  // chunk swizzle of a tile row: bf16 rows use swz; fp8 rows are 128 bytes,
  // two per 256-byte bank window, and rows r, r + 2 of a 4-row group go to
  // different row halves, so the score reads (16 rows, one chunk) and the
  // transposed V reads (16 rows x 2 chunks) hit 16 chunk positions
  // (fp8 rows of 64 bytes, d = 64, four to a bank window: chunk position
  // c ^ ((r >> 2) & 3) keeps the 16 rows of a score read and the row pairs of
  // a transposed V read on distinct banks)
  auto sw = [](int r) {
    if constexpr (F8 && D == 64) {
      return (r >> 2) & 3;
    } else if constexpr (F8) {
      const int j = (r >> 1) & 7;
      return ((j & 1) << 2) | (j >> 1);
    } else {
      return swz<CH>(r);
    }
  };
  // two K/V buffers as four distinct LDS objects, selected at compile time,
  // so the compiler can tell the tile being read from the one being filled
  __shared__ __attribute__((aligned(16))) char sk0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sk1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv1[TILE_BYTES];
  // dense-mask tiles (GEN with a mask): BM rows x 64 key bytes, row words
  // permuted so a lane's 8 words (the keys of its score registers) are two
  // 16-byte reads: word w of a row sits at position (w & 1) * 8 + (w >> 1)
  constexpr int MASK_BYTES = GEN && MASK ? BM * kBN : 16;
  __shared__ __attribute__((aligned(16))) char sm0[MASK_BYTES];
  __shared__ __attribute__((aligned(16))) char sm1[MASK_BYTES];

  // Without a dense mask a workgroup loops over several row blocks (one per
  // compute unit is launched) and issues the next block's first K/V tile and
  // its Q rows during the current block's last step, so neither the launch of
  // a new workgroup nor those first loads sit between two blocks.
  constexpr bool PERSIST = !(GEN && MASK);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar addresses and M0
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;
  const int S = a.S;                     // query rows
  const int SK = GEN ? a.S_k : a.S;      // keys
  const size_t q_row_stride = (size_t)a.h_q * D;   // elements between consecutive tokens of q/out
  const size_t kv_row_bytes = (size_t)a.n_kv * ROWB;
  const int G = a.h_q / a.n_kv;

  // ---- XCD-aware, heavy-first work order.  Item wl (a row block of one
  // group) is numbered so that each XCD's share [x * per_xcd, (x+1) *
  // per_xcd) runs heaviest first.  Groups (batch, K/V head, head chunk) are
  // taken grp_block at a time; inside such a block the row blocks run
  // heaviest first with the block's groups interleaved, so workgroups that
  // read the same rows of a dense mask (every group of a batch entry does)
  // run side by side on one XCD and share them in its L2.  grp_block = 1
  // keeps each group's row blocks together, which keeps its K/V in L2.
  auto item_of = [&](int wl) {
    int grp, qb;
    if (a.grp_block <= 1) {
      grp = wl / a.n_qb;
      qb = a.n_qb - 1 - (wl - grp * a.n_qb);
    } else {
      const int span = a.grp_block * a.n_qb;
      const int blk = wl / span;
      const int r = wl - blk * span;
      const int ng = min(a.grp_block, a.n_wg / a.n_qb - blk * a.grp_block);  // groups in this block
      const int qr = r / ng;
      grp = blk * a.grp_block + (r - qr * ng);
      qb = a.n_qb - 1 - qr;
    }
    // batch entry fastest: the groups one XCD takes come from every batch
    // entry, so batch entries of unequal work (key lengths) spread over all
    // XCDs instead of loading the XCDs they land on
    const int b = a.batch_minor ? grp % a.B : grp / (a.n_hc * a.n_kv);
    const int hc = a.batch_minor ? (grp / a.B) % a.n_hc : grp % a.n_hc;
    const int g = a.batch_minor ? grp / (a.B * a.n_hc) : (grp / a.n_hc) % a.n_kv;
    return int4{b, g, hc, qb};
  };
  // Workgroup n runs on XCD n % 8 and is the c-th of the C there; it takes
  // the XCD's items c, 2C - 1 - c, 2C + c, ... (one per round, alternating
  // direction, so the heavy-first order spreads evenly).  With one
  // workgroup per item (C = per_xcd) that is item c alone.
  const int per_xcd = a.n_wg_pad / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd, cw = blockIdx.x / kNumXcd, C = gridDim.x / kNumXcd;
  int round = 0;
  auto next_wl = [&]() {  // the workgroup's next item, or -1
    for (;;) {
      const int idx = round * C + ((round & 1) ? C - 1 - cw : cw);
      ++round;
      if (idx >= per_xcd) return -1;
      const int wl = xcd * per_xcd + idx;
      if (wl < a.n_wg) return wl;
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T).  bf16: Q[qrow][16ks + 8h2 ..
  // +7]; fp8: Q[qrow][64ks + 32h2 .. +31] (the K fragments take the same k order)
  u32x4 qf[F8 ? 1 : KS];
  i32x8 qf8[F8 ? KS8 : 1];
  // rows past S load row S - 1 (every lane issues the same loads) and are
  // zeroed by zero_q_past_end once the loads have landed
  auto load_q = [&](int b, int qrow, int head) {
    const int qr = min(qrow, S - 1);
    if constexpr (!F8) {
      const uint16_t* qp = a.q + ((size_t)b * S + qr) * q_row_stride + (size_t)head * D + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
    } else {
      const char* qp = reinterpret_cast<const char*>(a.q) + ((size_t)b * S + qr) * q_row_stride +
                       (size_t)head * D + 32 * h2;
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
        qf8[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    }
  };
  auto zero_q_past_end = [&](int qrow) {
    if (qrow < S) return;
    if constexpr (!F8) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) qf8[ks] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  // The next item's Q rows (persistent kernels) go straight into LDS, 32
  // rows per wave, during the current item's last step: 16-byte chunk c of
  // row r at chunk position c ^ (r % QCH), so the fragment reads spread over
  // the banks.  Rows past S are past the copy's buffer range and read as 0.
  constexpr int QROWB = D * EB;    // bytes of one head's row of Q
  constexpr int QCH = QROWB / 16;  // 16-byte chunks per row
  constexpr int RPQ = 64 / QCH;    // rows per copy instruction
  __shared__ __attribute__((aligned(16))) char sq[PERSIST ? kWaves * 32 * QROWB : 16];
  char* const sq_w = sq + (PERSIST ? wave * 32 * QROWB : 0);
  auto dma_q = [&](int b_n, int row0_n, int head_n) {
    const int nvalid = min(32, S - row0_n);
    const unsigned q_row_bytes = (unsigned)(q_row_stride * EB);
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)b_n * S + row0_n) * q_row_bytes + (size_t)head_n * QROWB;
    const auto rs = make_rsrc(nvalid > 0 ? qb : reinterpret_cast<const char*>(a.q),
                              nvalid > 0 ? (int)((unsigned)(nvalid - 1) * q_row_bytes + QROWB) : 0);
    const int rl = lane / QCH, p = lane % QCH;
#pragma unroll
    for (int u = 0; u < 32 / RPQ; ++u) {
      const int r = RPQ * u + rl;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sq_w + RPQ * u * QROWB), 16,
                                               (unsigned)r * q_row_bytes + (unsigned)((p ^ (r % QCH)) << 4), 0, 0, 0);
    }
  };
  auto q_from_lds = [&]() {
    const char* qr = sq_w + l32 * QROWB;
    const int qs = l32 % QCH;
    if constexpr (!F8) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = lds_load<u32x4>(qr + (((2 * ks + h2) ^ qs) << 4));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const u32x4 lo = lds_load<u32x4>(qr + (((4 * ks + 2 * h2) ^ qs) << 4));
        const u32x4 hi = lds_load<u32x4>(qr + (((4 * ks + 2 * h2 + 1) ^ qs) << 4));
        qf8[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    }
  };

  // One row block (item wl).  pref: its Q and first K/V tile (in buffer pair
  // par) were issued by the previous item.  Returns the buffer pair of the
  // next item's first tile if this item issued it (with that item's Q), else
  // -1.
  auto run_item = [&](const int wl, const int wl_n, const bool pref, const int par) __attribute__((always_inline)) -> int {
  const int4 it = item_of(wl);
  const int b = it.x, g = it.y, hc = it.z, qb = it.w;
  const int head = g * G + hc * HC + wave / RB;
  const int row0 = qb * BM + (wave % RB) * 32;
  const int qrow = row0 + l32;  // this lane's query row
  float qk_log2 = a.qk_scale_log2, out_scale = 1.0f;
  if constexpr (F8) {
    // a zero descale (an all-zero head quantised by absmax) would make the
    // score factor 0 and turn the -inf of a hidden key into NaN; the smallest
    // normal float keeps hidden keys at -inf and every visible score at zero
    // to float precision, which is the exact result (equal weights)
    qk_log2 = fmaxf(qk_log2 * (a.q_descale[(size_t)b * a.h_q + head] * a.k_descale[(size_t)b * a.n_kv + g]),
                    __FLT_MIN__);
    out_scale = a.v_descale[(size_t)b * a.n_kv + g];
  }
  if (pref) {
    q_from_lds();
  } else {
    load_q(b, qrow, head);
    zero_q_past_end(qrow);
  }

  const int row_end = min(qb * BM + BM, S);        // exclusive, over the whole workgroup
  // keys visible to a row are a prefix [0, kend(row)) (before the dense
  // mask); rows past S act as the last row (their output is dropped)
  int kv_n = SK;
  if constexpr (GEN) {
    if (a.kv_lens) kv_n = min(max(a.kv_lens[b], 0), SK);
  }
  auto kend_of = [&](int row) {
    if constexpr (!GEN) {
      return min(row, S - 1) + 1;
    } else {
      return a.causal ? max(min(kv_n, min(row, S - 1) + 1 + SK - S), 0) : kv_n;
    }
  };
  // key tiles 0 .. n_tiles-1 (0: no visible key)
  const int n_tiles = GEN ? block_key_tiles(row_end, S, SK, kv_n, a.causal) : (kend_of(row_end - 1) + kBN - 1) / kBN;
  const int wave_kend = kend_of(row0 + 31);  // the wave's rows see keys below this
  const int wave_kmin = kend_of(row0);       // ... and all of them see keys below this
  const int lane_kend = kend_of(qrow);

  const char* kbase = reinterpret_cast<const char*>(a.k) + ((size_t)b * SK * a.n_kv + g) * ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((size_t)b * SK * a.n_kv + g) * ROWB;
  // ---- K/V tiles go straight from global memory into LDS (no VGPR staging).
  // One wave instruction fills 1 KiB of LDS at (wave-uniform base + lane*16),
  // i.e. 64/CH consecutive tile rows; each lane picks the global 16-byte chunk
  // that belongs at its LDS slot under the XOR chunk swizzle, so the 16 (or 8)
  // lanes of a row still read one contiguous cache row.  Rows at or past the
  // sequence end (or the key length) are never read (see dma_tile).
  constexpr int RPI = 64 / CH;                  // tile rows per wave instruction
  // A tile of fewer than kWaves instructions per tensor (fp8 at d = 64: four
  // of 16 rows) is loaded by half the waves for K and the other half for V.
  constexpr bool SPLIT_KV = kBN / RPI < kWaves;
  constexpr int NINS = SPLIT_KV ? 1 : kBN / (RPI * kWaves);  // instructions per wave per tensor
  static_assert(SPLIT_KV ? 2 * kBN == RPI * kWaves : NINS * RPI * kWaves == kBN,
                "tile rows must split evenly over the waves");
  const int dma_r = lane / CH;                  // row within an instruction's rows
  const int dma_c = (lane % CH);                // physical chunk of this lane's LDS slot
  // Per-lane element offsets inside a tile, computed once; a full tile then
  // costs one wave-uniform base and one instruction per 1 KiB.  Only a tile
  // that runs past the sequence end clamps its rows.
  // (a vector, not an array: a local array captured by the lambdas below
  // makes hipcc's host pass drop this kernel's launch stub)
  static_assert(NINS <= 4, "per-lane DMA offsets are kept in a u32x4");
  // first tile row of instruction u of this wave (split: the wave's row
  // block of its tensor)
  auto ins_row0 = [&](int u) { return SPLIT_KV ? (wave % (kWaves / 2)) * RPI : (u * kWaves + wave) * RPI; };
  u32x4 dma_off = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < NINS; ++u) {
    const int r = ins_row0(u) + dma_r;
    dma_off[u] = (uint32_t)(r * kv_row_bytes + (dma_c ^ sw(r)) * 16);
  }
  // The copies go through buffer resources whose base is the tile's first
  // row and whose range ends at the last valid row (the sequence end, or the
  // key length): rows past it read as zero without a memory access (their
  // keys are hidden for every valid query row, so they contribute nothing).
  // Raw buffer loads to LDS count only on the vector-memory counter, which
  // leaves the LDS counter to the LDS reads: the compiler can then wait for
  // the reads a product needs instead of all of them.
  auto tile_rsrc = [&](const char* base, int kvn, int key0) {
    const int nvalid = min(kBN, kvn - key0);  // >= 1 for a visited tile
    return make_rsrc(base + (size_t)key0 * kv_row_bytes,
                     (int)((unsigned)(nvalid - 1) * (unsigned)kv_row_bytes + ROWB));
  };
  // tile j of the K/V rows at (kb, vb), key length kvn
  auto dma_tile_of = [&](const char* kb, const char* vb, int kvn, int j, char* kdst, char* vdst) {
    const int key0 = j * kBN;
    if constexpr (SPLIT_KV) {
      // waves 0 .. kWaves/2 - 1 load K, the others V
      const bool is_k = wave < kWaves / 2;
      const auto rs = tile_rsrc(is_k ? kb : vb, kvn, key0);
      char* dst = is_k ? kdst : vdst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + ins_row0(0) * ROWB), 16, dma_off[0], 0, 0, 0);
      return;
    }
    const auto rk = tile_rsrc(kb, kvn, key0);
    const auto rv = tile_rsrc(vb, kvn, key0);
#pragma unroll
    for (int u = 0; u < NINS; ++u) {
      const int r0 = (u * kWaves + wave) * RPI;  // first tile row of this instruction
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + r0 * ROWB), 16, dma_off[u], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + r0 * ROWB), 16, dma_off[u], 0, 0, 0);
    }
  };
  auto dma_tile = [&](int j, char* kdst, char* vdst) { dma_tile_of(kbase, vbase, kv_n, j, kdst, vdst); };
  auto dma_wait = [&]() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nt][r] = 0.f;
  float m = kNegInf, l = 0.f;

  // ---- dense mask tile -> LDS, 4 rows (256 bytes) per wave instruction:
  // lane l fills position l % 16 of row l / 16 with the word that belongs
  // there.  The loads go through a buffer resource over the workgroup's mask
  // rows: one shared 32-bit lane offset, the row and key offsets in a scalar;
  // rows past S read as zero (their output is dropped) and keys past S_k
  // read whatever follows (they are invisible by the key prefix).
  constexpr bool has_mask = GEN && MASK;
  constexpr int MROWS_PER_WAVE = BM / kWaves;  // mask rows each wave loads per tile
  static_assert(!GEN || MROWS_PER_WAVE % 4 == 0, "mask rows split into 4-row instructions");
  const int mpos = lane & 15;
  const int mword = (mpos & 7) * 2 + (mpos >> 3);  // word held at this lane's position
  const uint32_t m_lane_off = (uint32_t)((lane >> 4) * SK + 4 * mword);
  const int blk0 = qb * BM;
  const __amdgpu_buffer_rsrc_t mrsrc =
      make_rsrc(has_mask ? a.mask + ((size_t)b * S + blk0) * SK : static_cast<const uint8_t*>(nullptr),
                // up to 256 rows x 2^23 keys = 2^31 bytes: formed unsigned
                has_mask ? (int)((unsigned)min(BM, S - blk0) * (unsigned)SK) : 0);
  auto dma_mask = [&](int j, char* mdst) {
    if constexpr (GEN) {
      const int key0 = j * kBN;
#pragma unroll
      for (int u = 0; u < MROWS_PER_WAVE / 4; ++u) {
        const int r0 = wave * MROWS_PER_WAVE + 4 * u;  // first of this instruction's 4 rows
        __builtin_amdgcn_raw_ptr_buffer_load_lds(mrsrc, (lds_void*)(mdst + r0 * kBN), 4, m_lane_off,
                                                 r0 * SK + key0, 0, 0);
      }
    }
  };
  // this lane's 8 mask words of the tile in `mt` (keys 8p + 4h2 + i in word p)
  const int mrow = (wave % RB) * 32 + l32;  // this lane's row within the workgroup's block
  auto mask_words = [&](const char* mt) {
    const u32x4 lo = lds_load<u32x4>(mt + mrow * kBN + 32 * h2);
    const u32x4 hi = lds_load<u32x4>(mt + mrow * kBN + 32 * h2 + 16);
    return u32x4x2{lo, hi};
  };

  // ---- with a dense mask: which key tiles any row of the workgroup can see.
  // Bit j of s_vis is set when some mask byte of rows [blk0, row_end) over
  // the keys of tile j is nonzero; the loop below visits only those tiles,
  // so a tile hidden from the whole block (most tiles of a batch of packed
  // documents) costs neither its K/V and mask loads nor a barrier.  Bit j of
  // s_full is set when none of those bytes is zero: such a tile (the inside
  // of a document) needs no mask tile and no per-element mask.  Bytes a row
  // cannot see by the causal rule or the key length still count (a tile
  // visited for nothing, or masked needlessly, gives the same result).
  // Blocks with more tiles than the bitmaps hold visit every tile, masked.
  constexpr int kVis = has_mask ? kVisWords : 1;
  __shared__ uint32_t s_vis[kVis];
  __shared__ uint32_t s_full[kVis];
  const bool skip_tiles = has_mask && n_tiles <= kVisWords * 32;
  int n_steps = n_tiles;  // key tiles the loop visits
  if (skip_tiles) {
    if constexpr (has_mask) {
      if (a.mask_tiles) {
        // formed by the pass over the mask before this kernel
        const uint32_t* src = a.mask_tiles + ((size_t)b * a.n_qb + qb) * 2 * a.mt_words;
        for (int i = tid; i < (n_tiles + 31) / 32; i += kWaves * 64) {
          s_vis[i] = src[i];
          s_full[i] = src[a.mt_words + i];
        }
        __syncthreads();
      } else {
        scan_mask_tiles<BM>(mrsrc, 0, n_tiles, min(BM, S - blk0), SK, s_vis, s_full, wave, lane, tid);
      }
    }
    int cnt = 0;
    for (int i = lane; i < (n_tiles + 31) / 32; i += 64) cnt += __popc(s_vis[i]);
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) cnt += __shfl_xor(cnt, msk, 64);
    n_steps = __builtin_amdgcn_readfirstlane(cnt);
  }
  // the key tile visited after tile j (n_tiles: none)
  // after the first visited tile a row can still lack a visible key only
  // under a dense mask, or with the causal rule and fewer keys than queries
  const bool may_unset = GEN && (has_mask || (a.causal && SK < S));
  // tile j needs the per-element mask
  auto masked_tile = [&](int j) { return has_mask && !(skip_tiles && ((s_full[j >> 5] >> (j & 31)) & 1u)); };
  auto next_tile_of = [&](int j) {
    if (!skip_tiles) return j + 1;
    int t = j + 1;
    while (t < n_tiles) {
      const uint32_t bits = s_vis[t >> 5] >> (t & 31);
      if (bits != 0u) return __builtin_amdgcn_readfirstlane(t + (int)__builtin_ctz(bits));
      t = (t | 31) + 1;
    }
    return n_tiles;
  };

  if (n_steps == 0) {  // no row of the workgroup sees a key: zero rows
    if (qrow < S) {
      uint16_t* op = a.out + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) *reinterpret_cast<u32x2*>(op + 32 * nt + 8 * rq + 4 * h2) = u32x2{0u, 0u};
    }
    return -1;
  }
  // the next item (persistent kernels): its first tile and Q are issued in
  // this item's last step when it has any key to visit (no dense mask here,
  // so it visits tiles 0 .. n_tiles - 1)
  bool pf = false;
  const char* kbase_n = nullptr;
  const char* vbase_n = nullptr;
  int kv_n_n = SK, b_n = 0, head_n = 0, row0_n = 0;
  if constexpr (PERSIST) {
    if (wl_n >= 0) {
      const int4 it_n = item_of(wl_n);
      b_n = it_n.x;
      const int g_n = it_n.y, hc_n = it_n.z, qb_n = it_n.w;
      if constexpr (GEN) {
        if (a.kv_lens) kv_n_n = min(max(a.kv_lens[b_n], 0), SK);
      }
      const int row_end_n = min(qb_n * BM + BM, S);
      const int n_tiles_n = GEN ? block_key_tiles(row_end_n, S, SK, kv_n_n, a.causal) : (row_end_n + kBN - 1) / kBN;
      pf = n_tiles_n > 0;
      head_n = g_n * G + hc_n * HC + wave / RB;
      row0_n = qb_n * BM + (wave % RB) * 32;
      kbase_n = reinterpret_cast<const char*>(a.k) + ((size_t)b_n * SK * a.n_kv + g_n) * ROWB;
      vbase_n = reinterpret_cast<const char*>(a.v) + ((size_t)b_n * SK * a.n_kv + g_n) * ROWB;
    }
  }
  const int j_first = next_tile_of(-1);
  const int p0 = pref ? par : 0;  // buffer pair of the first tile
  if (!pref) {
    dma_tile(j_first, sk0, sv0);
    if (masked_tile(j_first)) dma_mask(j_first, sm0);
    dma_wait();
    __syncthreads();
  }

  // step k visits key tile j: compute from (kt, vt) while the next visited
  // tile fills (kn, vn); returns that next tile
  auto tile_step = [&](int k, int j, const char* kt, const char* vt, const char* mt, char* kn, char* vn, char* mn) {
    // the other buffer was last read in step k-1, before its closing barrier
    const int jn = next_tile_of(j);
    const bool last = k + 1 == n_steps;
    if (!last) {
      dma_tile(jn, kn, vn);
      if (masked_tile(jn)) dma_mask(jn, mn);
    } else if (PERSIST && pf) {
      // the next item's first tile and Q (this wave's Q reads of sq_w have
      // returned: its registers fed this item's first products)
      dma_tile_of(kbase_n, vbase_n, kv_n_n, 0, kn, vn);
      __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_q(b_n, row0_n, head_n);
    }
    const bool tmask = masked_tile(j);  // the mask tile of j is in mt
    const int key0 = j * kBN;
    // no row of this wave sees a key of the tile (by the key prefix, or by a
    // mask that hides the whole tile from all its rows): nothing to do but
    // keep in step
    bool work = key0 < wave_kend;
    if (GEN && work && tmask) {
      const u32x4x2 mw = mask_words(mt);
      const uint32_t any = mw.lo[0] | mw.lo[1] | mw.lo[2] | mw.lo[3] | mw.hi[0] | mw.hi[1] | mw.hi[2] | mw.hi[3];
      work = __builtin_amdgcn_ballot_w64(any != 0u && qrow < S) != 0;
    }
    if (work) {
      // ---- S^T for the two 32-key halves, k-steps interleaved: the K
      // fragments of step ks+2 are read while the two products of step ks run.
      // Keys above the diagonal (past the row's visible prefix) get -inf.
      const bool diag = key0 + kBN > wave_kmin;
      auto scores = [&](f32x16(&sacc)[2]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[0][r] = 0.f;
          sacc[1][r] = 0.f;
        }
        if constexpr (F8) {
          // K[key][64ks + 32h2 .. +31]: two 16-byte reads; the swizzle of a
          // row is the same for both halves (32 rows apart)
          const char* kp0 = kt + l32 * ROWB;
          const int swk = sw(l32);
#pragma unroll
          for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const char* kp = kp0 + kh * 32 * ROWB;
              const u32x4 lo = lds_load<u32x4>(kp + (((4 * ks + 2 * h2) ^ swk) << 4));
              const u32x4 hi = lds_load<u32x4>(kp + (((4 * ks + 2 * h2 + 1) ^ swk) << 4));
              const i32x8 kf8 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
              sacc[kh] = mfma32_fp8(kf8, qf8[ks], sacc[kh]);
            }
        } else {
        // swz(krow) is the same for both halves (32 is a multiple of 16)
        const char* kp0 = kt + l32 * ROWB;
        auto kfrag = [&](int kh, int ks) {
          return lds_load<u32x4>(kp0 + kh * 32 * ROWB + (((2 * ks + h2) ^ sw(l32)) << 4));
        };
        u32x4 kf[KS][2];
        kf[0][0] = kfrag(0, 0);
        kf[0][1] = kfrag(1, 0);
        kf[1][0] = kfrag(0, 1);
        kf[1][1] = kfrag(1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 2 < KS) {
            kf[ks + 2][0] = kfrag(0, ks + 2);
            kf[ks + 2][1] = kfrag(1, ks + 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the reads for step ks+2,
          }
          sacc[0] = mfma32(kf[ks][0], qf[ks], sacc[0]);
          sacc[1] = mfma32(kf[ks][1], qf[ks], sacc[1]);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // then the products of step ks
        }
        }
        if (diag) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kh + 8 * (r >> 2) + 4 * h2 + (r & 3);
              sacc[kh][r] = key >= lane_kend ? kNegInf : sacc[kh][r];
            }
        }
        if (GEN && tmask) {
          const u32x4x2 mw = mask_words(mt);
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int p = 4 * kh + (r >> 2);
              const uint32_t word = p < 4 ? mw.lo[p] : mw.hi[p - 4];
              // rows past S (output dropped) ignore the mask, so their
              // lanes do not force the wave off the fast softmax path
              const uint32_t byte = (word >> (8 * (r & 3))) & 0xFFu;
              sacc[kh][r] = byte == 0u && qrow < S ? kNegInf : sacc[kh][r];
            }
        }
      };
      // p = 2^(scale*log2(e)*s - m) in place, returning this lane's sum
      auto probs = [&](f32x16(&sacc)[2], float mref) {
        float psum = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(__builtin_fmaf(sacc[kh][r], qk_log2, -mref));
            sacc[kh][r] = p;
            psum += p;
          }
        return psum;
      };
      f32x16 sacc[2];
      scores(sacc);
      // ---- online softmax (row = this lane's query; its keys are split with
      // lane ^ 32).  The reference max m (log2 units) is shared by O and l,
      // so any reference gives the same result as long as nothing overflows.
      // Fast path, every tile after the first: keep m and check that the
      // tile's p stay bounded (psum <= 2^30 in every lane).  Otherwise (the
      // first tile, or scores that rose far above m) the wave recomputes the
      // scores, moves m to the running max (one exchange with lane ^ 32),
      // rescales O and l, and takes p again.
      float psum = 0.f;
      bool slow = k == 0;
      if (!slow) {
        // with general masks a row may have seen no visible key yet (m =
        // -inf): it stays on the fast path (p = 0) while its scores in this
        // tile are all hidden, and takes the slow path at its first visible one
        bool unset = false;
        if constexpr (GEN) {
          if (may_unset && __builtin_amdgcn_ballot_w64(m == kNegInf) != 0) {
            float mx = kNegInf;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
              for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kh][r]);
            unset = m == kNegInf && mx != kNegInf;
          }
        }
        psum = probs(sacc, GEN && m == kNegInf ? 0.f : m);
        // bound: bf16 P has range to spare; e4m3 P must stay below its 448
        // maximum, which psum <= 256 guarantees for every p of the tile
        slow = __builtin_amdgcn_ballot_w64(unset || !(psum <= (F8 ? 256.0f : 0x1p30f))) != 0;  // also catches inf / NaN
        if (slow) scores(sacc);
      }
      if (slow) {
        float mt = kNegInf;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kh][r]);
        mt = wave_max_xor(mt, 32) * qk_log2;  // scale > 0 keeps the order
        const float m_new = fmaxf(m, mt);
        if constexpr (!GEN) {
          // finite: key 0 is visible to every row
          const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
          m = m_new;
          l *= alpha;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
          psum = probs(sacc, m);
        } else {
          // a row may have seen no visible key yet (m = -inf, O = l = 0), or
          // see none in this tile either (m_new = -inf: all its p are 0)
          const float alpha = m == kNegInf ? 0.f : fast_exp2(m - m_new);
          m = m_new;
          l *= alpha;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
          psum = probs(sacc, m == kNegInf ? 0.f : m);
        }
      }
      l += psum;
      if constexpr (F8) {
        // ---- O^T += V^T P^T on two 64-key products (hi and lo weights) per
        // 32-wide d tile.  P byte b = 16kh + r of a lane is the score register sacc[kh][r], key
        // 32kh + 8(r/4) + 4h2 + r%4.  ds_read_b64_tr_b8 hands output lane
        // 16gg + 8u + c byte j of source lane 16gg + 2j + u (byte c of its 8):
        // source lane (gg, j, u) therefore reads, for read t (bytes 8t..8t+7),
        // key 32(t/2) + 16(t%2) + 8(j/4) + 4(gg/2) + j%4 at d columns
        // 32dt + 16(gg%2) + 8u .. +7, so that output lane l holds d = 32dt +
        // l%32 for exactly the keys of its P bytes.
        i32x8 pf8, pl8;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const f32x16& sp = sacc[w >> 2];
          const int r0 = 4 * (w & 3);
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0], sp[r0 + 1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0 + 2], sp[r0 + 3], x, true);
          pf8[w] = x;
          // the rounding remainders, exact in float32, rounded to e4m3 again
          const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
          const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
          int y = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0] - h01[0], sp[r0 + 1] - h01[1], 0, false);
          y = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0 + 2] - h23[0], sp[r0 + 3] - h23[1], y, true);
          pl8[w] = y;
        }
        const int gg = lane >> 4, jj = (lane & 15) >> 1, uu = lane & 1;
        const int vkey = 8 * (jj >> 2) + 4 * (gg >> 1) + (jj & 3);  // plus 16t: same swizzle for every t
        const int swv = sw(vkey);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int chunk = (2 * nt + (gg & 1)) ^ swv;
          i32x8 vf8;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(vt + (16 * t + vkey) * ROWB + (chunk << 4) + 8 * uu));
            vf8[2 * t] = r[0];
            vf8[2 * t + 1] = r[1];
          }
          o[nt] = mfma32_fp8(vf8, pf8, o[nt]);
          o[nt] = mfma32_fp8(vf8, pl8, o[nt]);
        }
      } else {
      // ---- O^T += V^T P^T, 4 k-steps of 16 keys, products in (k-step, d tile)
      // order; the V^T fragment of product i + 2 is read while product i runs
      // (three fragments in flight), so no product waits for the latency of
      // its own LDS reads
      u32x4 pw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f32x16& sp = sacc[p >> 1];
        const int rb = 8 * (p & 1);
        pw[p] = u32x4{pack_bf16x2(sp[rb + 0], sp[rb + 1]), pack_bf16x2(sp[rb + 2], sp[rb + 3]),
                      pack_bf16x2(sp[rb + 4], sp[rb + 5]), pack_bf16x2(sp[rb + 6], sp[rb + 7])};
      }
      const int gi = lane >> 4, s16 = lane & 15;
      auto vfrag = [&](int i) {
        const int p = i / NT, nt = i % NT;
        const int col = 32 * nt + 16 * (gi & 1) + 4 * (s16 & 3);
        const int c = col >> 3, w = col & 7;
        const int ra = 16 * p + 4 * h2 + (s16 >> 2);
        const int rbw = ra + 8;
        const u32x2 va = lds_read_tr16(vt + ra * ROWB + ((c ^ sw(ra)) << 4) + 2 * w);
        const u32x2 vb = lds_read_tr16(vt + rbw * ROWB + ((c ^ sw(rbw)) << 4) + 2 * w);
        return u32x4{va[0], va[1], vb[0], vb[1]};
      };
      constexpr int NPV = 4 * NT;
      u32x4 vq[3];
      vq[0] = vfrag(0);
      vq[1] = vfrag(1);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + 2 < NPV) {
          vq[(i + 2) % 3] = vfrag(i + 2);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the reads for product i + 2,
        }
        o[i % NT] = mfma32(vq[i % 3], pw[i / NT], o[i % NT]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // then product i
      }
      }
    }
    dma_wait();
    __syncthreads();
    return jn;
  };
  // step k reads pair (k + p0) & 1: v = k + p0 counts pairs of steps, the
  // first of which is skipped when the first tile is in pair 1
  int j = j_first;
  for (int v = 0; v < n_steps + p0; v += 2) {
    if (v >= p0) j = tile_step(v - p0, j, sk0, sv0, sm0, sk1, sv1, sm1);
    if (v + 1 < n_steps + p0) j = tile_step(v + 1 - p0, j, sk1, sv1, sm1, sk0, sv0, sm0);
  }

  // ---- epilogue: O / l -> bf16, rows < S only
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = lt > 0.f ? out_scale / lt : 0.f;  // fp8: the V descale folds in here
  // Through LDS: a lane holds 8 bytes of each of 16 chunks of its row, so
  // direct stores would touch 32 rows per instruction.  The wave writes its
  // 32-row tile into its own LDS region and stores whole row slices back, CO
  // lanes per row, 16 bytes each (16-byte chunk c of row r at chunk position
  // c ^ (r % CO)), in NPASS column slices when the region is smaller than
  // the tile.  The regions are free after the last step's barrier: with a
  // next item the output goes through the buffer pair the last step read (the
  // other holds the next item's first tile), four waves to a buffer;
  // otherwise through both pairs, two waves to a buffer.
  constexpr int OUT_BYTES = 32 * D * 2;  // the wave's bf16 output tile
  constexpr int WPB = PERSIST ? 4 : 2;   // waves per buffer
  constexpr int REGION = OUT_BYTES < TILE_BYTES / WPB ? OUT_BYTES : TILE_BYTES / WPB;
  constexpr int NPASS = OUT_BYTES / REGION;
  if constexpr (NPASS <= NT) {
    constexpr int DP = D / NPASS;  // columns per pass
    constexpr int CO = DP / 8;     // 16-byte chunks per row slice
    constexpr int RPS = 64 / CO;   // rows per store instruction
    static_assert(NPASS * REGION == OUT_BYTES && (NT / NPASS) * NPASS == NT, "output passes split the d tiles");
    char* ep;
    if constexpr (PERSIST) {
      const int y = (n_steps - 1 + p0) & 1;  // the pair the last step read
      ep = (wave < 4 ? (y ? sk1 : sk0) : (y ? sv1 : sv0)) + (wave & 3) * REGION;
    } else {
      ep = (wave < 2 ? sk0 : wave < 4 ? sk1 : wave < 6 ? sv0 : sv1) + (wave & 1) * REGION;
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
      for (int ntp = 0; ntp < NT / NPASS; ++ntp)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int nt = ps * (NT / NPASS) + ntp;
          const int c = 4 * ntp + rq;  // chunk of d 32nt + 8rq .. +7 in this slice
          u32x2 w;
          w[0] = pack_bf16x2(o[nt][4 * rq + 0] * inv, o[nt][4 * rq + 1] * inv);
          w[1] = pack_bf16x2(o[nt][4 * rq + 2] * inv, o[nt][4 * rq + 3] * inv);
          *reinterpret_cast<u32x2*>(ep + l32 * (DP * 2) + ((c ^ (l32 % CO)) << 4) + 8 * h2) = w;
        }
      const int c = lane % CO;
#pragma unroll
      for (int t = 0; t < 32 / RPS; ++t) {
        const int r = RPS * t + lane / CO;
        const u32x4 v = lds_load<u32x4>(ep + r * (DP * 2) + ((c ^ (r % CO)) << 4));
        if (row0 + r < S)
          *reinterpret_cast<u32x4*>(a.out + ((size_t)b * S + row0 + r) * q_row_stride + (size_t)head * D + ps * DP +
                                    8 * c) = v;
      }
    }
  } else if (qrow < S) {  // fp8 at d = 64 with a next item: regions too small, direct stores
    uint16_t* op = a.out + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 w;
        w[0] = pack_bf16x2(o[nt][4 * rq + 0] * inv, o[nt][4 * rq + 1] * inv);
        w[1] = pack_bf16x2(o[nt][4 * rq + 2] * inv, o[nt][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * nt + 8 * rq + 4 * h2) = w;
      }
  }
  if constexpr (PERSIST) {
    if (wl_n >= 0) {
      // the next item's first step refills the pair read here
      __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
    }
  }
  return pf ? ((n_steps + p0) & 1) : -1;
  };  // run_item

  bool pref = false;
  int par = 0;
  for (int wl = next_wl(); wl >= 0;) {
    const int wl_n = PERSIST ? next_wl() : -1;
    const int np = run_item(wl, wl_n, pref, par);
    pref = np >= 0;
    par = pref ? np : 0;
    wl = wl_n;
  }
}

template <int D, int HC>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_causal_kernel(PrefillArgs a) {
  prefill_body<D, HC, false>(a);
}

template <int D, int HC, bool MASK>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_masked_kernel(PrefillArgs a) {
  prefill_body<D, HC, true, false, MASK>(a);
}

template <int D, int HC, bool MASK>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_fp8_kernel(PrefillArgs a) {
  prefill_body<D, HC, true, true, MASK>(a);
}

// The key-tile bitmaps of every (batch entry, row block) under a dense mask,
// formed once for all the K/V-head workgroups that share the block's mask
// rows: one workgroup per row block and 32-tile word of its bitmaps (grid
// n_qb x B x words), the same scan as a masked workgroup's own over that
// word's tiles.  Blocks with more key tiles than the bitmaps hold are
// skipped (their workgroups visit every tile).
template <int BM>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_mask_tiles_kernel(PrefillArgs a) {
  __shared__ uint32_t vis[kVisWords];
  __shared__ uint32_t full[kVisWords];
  const int qb = blockIdx.x, b = blockIdx.y, word = blockIdx.z;
  const int S = a.S, SK = a.S_k;
  const int blk0 = qb * BM;
  const int row_end = min(blk0 + BM, S);
  const int kv_n = a.kv_lens ? min(max(a.kv_lens[b], 0), SK) : SK;
  const int n_tiles = block_key_tiles(row_end, S, SK, kv_n, a.causal);
  // uniform over the workgroup
  if (n_tiles == 0 || n_tiles > kVisWords * 32 || 32 * word >= n_tiles) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const __amdgpu_buffer_rsrc_t mrsrc =
      make_rsrc(a.mask + ((size_t)b * S + blk0) * SK, (int)((unsigned)(row_end - blk0) * (unsigned)SK));
  scan_mask_tiles<BM>(mrsrc, 32 * word, min(n_tiles, 32 * word + 32), row_end - blk0, SK, vis, full, wave, lane,
                      tid);
  if (tid == 0) {
    uint32_t* dst = const_cast<uint32_t*>(a.mask_tiles) + ((size_t)b * a.n_qb + qb) * 2 * a.mt_words;
    dst[word] = vis[word];
    dst[a.mt_words + word] = full[word];
  }
}

static int gcd_int(int x, int y) {
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

// Workgroups of a kernel without a dense mask: one per compute unit (a
// multiple of the 8 XCDs), each looping over its share of the row blocks,
// or one per row block when there are fewer.
static int persistent_grid(const PrefillArgs& a, int n_cu) {
  const int per_cu = max(n_cu / kNumXcd, 1) * kNumXcd;
  return min(a.n_wg_pad, per_cu);
}

static PrefillArgs prefill_args(const void* q, const void* k, const void* v, void* out, float qk_scale_log2,
                                int B, int S, int h_q, int n_kv, int HC) {
  const int G = h_q / n_kv;
  const int BM = 32 * (kWaves / HC);
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.qk_scale_log2 = qk_scale_log2;
  a.B = B;
  a.S = S;
  a.h_q = h_q;
  a.n_kv = n_kv;
  a.n_qb = (S + BM - 1) / BM;
  a.n_hc = G / HC;
  a.n_wg = B * n_kv * a.n_hc * a.n_qb;
  a.n_wg_pad = (a.n_wg + kNumXcd - 1) / kNumXcd * kNumXcd;
  a.grp_block = 1;
  a.batch_minor = 0;
  a.S_k = S;
  a.causal = 1;
  a.kv_lens = nullptr;
  a.mask = nullptr;
  a.mask_tiles = nullptr;
  a.mt_words = 0;
  a.q_descale = nullptr;
  a.k_descale = nullptr;
  a.v_descale = nullptr;
  return a;
}

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S, int h_q, int n_kv, int D, int n_cu, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  const PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S, h_q, n_kv, HC);
  const dim3 grid(persistent_grid(a, n_cu)), block(kWaves * 64);
#define GQA_LAUNCH_PREFILL(DD, HH) hipLaunchKernelGGL((gqa_prefill_causal_kernel<DD, HH>), grid, block, 0, stream, a)
  if (D == 128) {
    if (HC == 8) GQA_LAUNCH_PREFILL(128, 8);
    else if (HC == 4) GQA_LAUNCH_PREFILL(128, 4);
    else if (HC == 2) GQA_LAUNCH_PREFILL(128, 2);
    else GQA_LAUNCH_PREFILL(128, 1);
  } else {
    if (HC == 8) GQA_LAUNCH_PREFILL(64, 8);
    else if (HC == 4) GQA_LAUNCH_PREFILL(64, 4);
    else if (HC == 2) GQA_LAUNCH_PREFILL(64, 2);
    else GQA_LAUNCH_PREFILL(64, 1);
  }
#undef GQA_LAUNCH_PREFILL
  return hipGetLastError();
}

// Words per bitmap of one row block's key tiles (S_k keys, at most kVisWords).
static int mask_tile_words(int S_k) { return min((S_k + kBN * 32 - 1) / (kBN * 32), kVisWords); }

size_t prefill_mask_tiles_bytes(int B, int S_q, int S_k, int h_q, int n_kv) {
  const int BM = 32 * (kWaves / gcd_int(h_q / n_kv, kWaves));
  return (size_t)B * ((S_q + BM - 1) / BM) * 2 * mask_tile_words(S_k) * sizeof(uint32_t);
}

// With a mask and a bitmap buffer: the pass that forms every row block's
// bitmaps, launched before the attention kernel on the same stream.
static hipError_t launch_mask_tiles(PrefillArgs& a, uint32_t* mask_tiles, int HC, hipStream_t stream) {
  if (!a.mask || !mask_tiles) return hipSuccess;
  a.mask_tiles = mask_tiles;
  a.mt_words = mask_tile_words(a.S_k);
  const dim3 grid(a.n_qb, a.B, a.mt_words), block(kWaves * 64);
  switch (kWaves / HC) {
    case 1: hipLaunchKernelGGL((gqa_mask_tiles_kernel<32>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gqa_mask_tiles_kernel<64>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gqa_mask_tiles_kernel<128>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((gqa_mask_tiles_kernel<256>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// Work order of the general kernels.  Without a dense mask, groups go batch
// entry fastest, which spreads batch entries of unequal key lengths over the
// XCDs: padded workload (4 x 4096, key lengths 2597..3954, 32/8 heads) 913 ->
// 811 us.  With a mask, a batch entry's groups run interleaved per row block
// on one XCD, sharing its mask rows in L2; measured on the packed-document
// workload, batch entry fastest lost there (with the bitmaps formed
// beforehand: 276 -> 282 us, and 320 us with the interleave kept).
static void set_work_order(PrefillArgs& a) {
  a.grp_block = a.mask ? kMaskGroupBlock : 1;
  a.batch_minor = a.mask ? 0 : 1;
}

hipError_t launch_prefill_masked(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S_q, int S_k, int h_q, int n_kv, int D, int causal, const int32_t* kv_lens,
                                 const uint8_t* mask, uint32_t* mask_tiles, int n_cu, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S_q, h_q, n_kv, HC);
  a.S_k = S_k;
  a.causal = causal;
  a.kv_lens = kv_lens;
  a.mask = mask;
  if (const hipError_t e = launch_mask_tiles(a, mask_tiles, HC, stream); e != hipSuccess) return e;
  set_work_order(a);
  const dim3 grid(mask ? a.n_wg_pad : persistent_grid(a, n_cu)), block(kWaves * 64);
#define GQA_LAUNCH_PREFILL(DD, HH)                                                                       \
  do {                                                                                                   \
    if (mask) hipLaunchKernelGGL((gqa_prefill_masked_kernel<DD, HH, true>), grid, block, 0, stream, a);  \
    else hipLaunchKernelGGL((gqa_prefill_masked_kernel<DD, HH, false>), grid, block, 0, stream, a);      \
  } while (0)
  if (D == 128) {
    if (HC == 8) GQA_LAUNCH_PREFILL(128, 8);
    else if (HC == 4) GQA_LAUNCH_PREFILL(128, 4);
    else if (HC == 2) GQA_LAUNCH_PREFILL(128, 2);
    else GQA_LAUNCH_PREFILL(128, 1);
  } else {
    if (HC == 8) GQA_LAUNCH_PREFILL(64, 8);
    else if (HC == 4) GQA_LAUNCH_PREFILL(64, 4);
    else if (HC == 2) GQA_LAUNCH_PREFILL(64, 2);
    else GQA_LAUNCH_PREFILL(64, 1);
  }
#undef GQA_LAUNCH_PREFILL
  return hipGetLastError();
}

hipError_t launch_prefill_fp8(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                              int S_q, int S_k, int h_q, int n_kv, int D, int causal, const int32_t* kv_lens,
                              const uint8_t* mask, const float* q_descale, const float* k_descale,
                              const float* v_descale, uint32_t* mask_tiles, int n_cu, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S_q, h_q, n_kv, HC);
  a.S_k = S_k;
  a.causal = causal;
  a.kv_lens = kv_lens;
  a.mask = mask;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  if (const hipError_t e = launch_mask_tiles(a, mask_tiles, HC, stream); e != hipSuccess) return e;
  set_work_order(a);
  const dim3 grid(mask ? a.n_wg_pad : persistent_grid(a, n_cu)), block(kWaves * 64);
#define GQA_LAUNCH_FP8(DD, HH)                                                                          \
  do {                                                                                                  \
    if (mask) hipLaunchKernelGGL((gqa_prefill_fp8_kernel<DD, HH, true>), grid, block, 0, stream, a);    \
    else hipLaunchKernelGGL((gqa_prefill_fp8_kernel<DD, HH, false>), grid, block, 0, stream, a);        \
  } while (0)
  if (D == 128) {
    if (HC == 8) GQA_LAUNCH_FP8(128, 8);
    else if (HC == 4) GQA_LAUNCH_FP8(128, 4);
    else if (HC == 2) GQA_LAUNCH_FP8(128, 2);
    else GQA_LAUNCH_FP8(128, 1);
  } else {
    if (HC == 8) GQA_LAUNCH_FP8(64, 8);
    else if (HC == 4) GQA_LAUNCH_FP8(64, 4);
    else if (HC == 2) GQA_LAUNCH_FP8(64, 2);
    else GQA_LAUNCH_FP8(64, 1);
  }
#undef GQA_LAUNCH_FP8
  return hipGetLastError();
}

}  // namespace gqa
