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
  // general masks (the masked kernel only)
  int S_k;                  // keys per sequence
  int causal;               // query r sees keys c <= r + S_k - S_q
  const int32_t* kv_lens;   // [B] or null: keys c >= kv_lens[b] are invisible and never read
  const uint8_t* mask;      // [B][S][S_k] or null: key c invisible to row r where 0
};

constexpr int kBN = 64;  // keys per tile
constexpr int kNumXcd = 8;
constexpr int kWaves = 8;  // wavefronts per workgroup

// GEN = false: causal self-attention, S_q = S_k, every key of a row's causal
// range visible.  GEN = true: S_q and S_k independent, the causal rule
// optional and end-aligned, optional key lengths and dense mask; rows can
// then have no visible key at all (zero output).
template <int D, int HC, bool GEN>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a) {
  constexpr int RB = kWaves / HC;  // 32-row blocks per head in one workgroup
  constexpr int BM = 32 * RB;    // query rows per workgroup
  constexpr int CH = D / 8;      // 16-byte chunks per K/V row
  constexpr int KS = D / 16;     // k-steps of the score product
  constexpr int NT = D / 32;     // 32-wide d tiles of the PV product
  constexpr int TILE_BYTES = kBN * D * 2;
  // two K/V buffers as four distinct LDS objects, selected at compile time,
  // so the compiler can tell the tile being read from the one being filled
  __shared__ __attribute__((aligned(16))) char sk0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sk1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv1[TILE_BYTES];
  // dense-mask tiles (GEN with a mask): BM rows x 64 key bytes, row words
  // permuted so a lane's 8 words (the keys of its score registers) are two
  // 16-byte reads: word w of a row sits at position (w & 1) * 8 + (w >> 1)
  constexpr int MASK_BYTES = GEN ? BM * kBN : 16;
  __shared__ __attribute__((aligned(16))) char sm0[MASK_BYTES];
  __shared__ __attribute__((aligned(16))) char sm1[MASK_BYTES];

  // ---- XCD-aware, heavy-first workgroup -> work mapping
  const int n = blockIdx.x;
  const int per_xcd = a.n_wg_pad / kNumXcd;
  const int wl = (n % kNumXcd) * per_xcd + n / kNumXcd;
  if (wl >= a.n_wg) return;
  const int grp = wl / a.n_qb;
  const int qb = a.n_qb - 1 - (wl - grp * a.n_qb);
  const int hc = grp % a.n_hc;
  const int g = (grp / a.n_hc) % a.n_kv;
  const int b = grp / (a.n_hc * a.n_kv);
  const int G = a.h_q / a.n_kv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar addresses and M0
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;
  const int head = g * G + hc * HC + wave / RB;
  const int row0 = qb * BM + (wave % RB) * 32;
  const int qrow = row0 + l32;  // this lane's query row
  const int S = a.S;                     // query rows
  const int SK = GEN ? a.S_k : a.S;      // keys
  const size_t q_row_stride = (size_t)a.h_q * D;   // elements between consecutive tokens of q/out
  const size_t kv_row_stride = (size_t)a.n_kv * D;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[qrow][16ks + 8h2 .. +7]
  u32x4 qf[KS];
  {
    const uint16_t* qp = a.q + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < S) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qf[ks] = v;
    }
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
  const int n_tiles = (kend_of(row_end - 1) + kBN - 1) / kBN;  // key tiles 0 .. n_tiles-1 (0: no visible key)
  const int wave_kend = kend_of(row0 + 31);  // the wave's rows see keys below this
  const int wave_kmin = kend_of(row0);       // ... and all of them see keys below this
  const int lane_kend = kend_of(qrow);

  const uint16_t* kbase = a.k + (size_t)b * SK * kv_row_stride + (size_t)g * D;
  const uint16_t* vbase = a.v + (size_t)b * SK * kv_row_stride + (size_t)g * D;
  // ---- K/V tiles go straight from global memory into LDS (no VGPR staging).
  // One wave instruction fills 1 KiB of LDS at (wave-uniform base + lane*16),
  // i.e. 64/CH consecutive tile rows; each lane picks the global 16-byte chunk
  // that belongs at its LDS slot under the XOR chunk swizzle, so the 16 (or 8)
  // lanes of a row still read one contiguous cache row.  Rows past the
  // sequence end re-read its last row (in bounds); their keys are always
  // masked for valid query rows, so they contribute nothing.  With key
  // lengths the same holds at the length: rows at or past it are never read.
  constexpr int RPI = 64 / CH;                  // tile rows per wave instruction
  constexpr int NINS = kBN / (RPI * kWaves);    // instructions per wave per tensor
  static_assert(NINS * RPI * kWaves == kBN, "tile rows must split evenly over the waves");
  const int dma_r = lane / CH;                  // row within an instruction's rows
  const int dma_c = (lane % CH);                // physical chunk of this lane's LDS slot
  // Per-lane element offsets inside a tile, computed once; a full tile then
  // costs one wave-uniform base and one instruction per 1 KiB.  Only a tile
  // that runs past the sequence end clamps its rows.
  // (a vector, not an array: a local array captured by the lambdas below
  // makes hipcc's host pass drop this kernel's launch stub)
  static_assert(NINS <= 4, "per-lane DMA offsets are kept in a u32x4");
  u32x4 dma_off = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < NINS; ++u) {
    const int r = (u * kWaves + wave) * RPI + dma_r;
    dma_off[u] = (uint32_t)(r * kv_row_stride + (dma_c ^ swz<CH>(r)) * 8);
  }
  auto dma_tile = [&](int j, char* kdst, char* vdst) {
    const int key0 = j * kBN;
    if (key0 + kBN <= kv_n) {
      const uint16_t* kt = kbase + (size_t)key0 * kv_row_stride;
      const uint16_t* vt = vbase + (size_t)key0 * kv_row_stride;
#pragma unroll
      for (int u = 0; u < NINS; ++u) {
        const int r0 = (u * kWaves + wave) * RPI;  // first tile row of this instruction
        __builtin_amdgcn_global_load_lds(kt + dma_off[u], (lds_void*)(kdst + r0 * (2 * D)), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + dma_off[u], (lds_void*)(vdst + r0 * (2 * D)), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NINS; ++u) {
        const int r0 = (u * kWaves + wave) * RPI;
        const int r = r0 + dma_r;
        const int key = min(key0 + r, kv_n - 1);
        const int c = dma_c ^ swz<CH>(r);         // logical chunk stored at this slot
        const size_t off = (size_t)key * kv_row_stride + c * 8;
        __builtin_amdgcn_global_load_lds(kbase + off, (lds_void*)(kdst + r0 * (2 * D)), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + off, (lds_void*)(vdst + r0 * (2 * D)), 16, 0, 0);
      }
    }
  };
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
  const bool has_mask = GEN && a.mask != nullptr;
  constexpr int MROWS_PER_WAVE = BM / kWaves;  // mask rows each wave loads per tile
  static_assert(!GEN || MROWS_PER_WAVE % 4 == 0, "mask rows split into 4-row instructions");
  const int mpos = lane & 15;
  const int mword = (mpos & 7) * 2 + (mpos >> 3);  // word held at this lane's position
  const uint32_t m_lane_off = (uint32_t)((lane >> 4) * SK + 4 * mword);
  const int blk0 = qb * BM;
  const __amdgpu_buffer_rsrc_t mrsrc =
      make_rsrc(has_mask ? a.mask + ((size_t)b * S + blk0) * SK : static_cast<const uint8_t*>(nullptr),
                has_mask ? min(BM, S - blk0) * SK : 0);
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

  if (n_tiles == 0) {  // no row of the workgroup sees a key: zero rows
    if (qrow < S) {
      uint16_t* op = a.out + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) *reinterpret_cast<u32x2*>(op + 32 * nt + 8 * rq + 4 * h2) = u32x2{0u, 0u};
    }
    return;
  }
  dma_tile(0, sk0, sv0);
  if (has_mask) dma_mask(0, sm0);
  dma_wait();
  __syncthreads();

  // one key tile: compute from (kt, vt) while the next tile fills (kn, vn)
  auto tile_step = [&](int j, const char* kt, const char* vt, const char* mt, char* kn, char* vn, char* mn) {
    // the other buffer was last read in iteration j-1, before its closing barrier
    if (j + 1 < n_tiles) {
      dma_tile(j + 1, kn, vn);
      if (has_mask) dma_mask(j + 1, mn);
    }
    const int key0 = j * kBN;
    // no row of this wave sees a key of the tile (by the key prefix, or by a
    // mask that hides the whole tile from all its rows): nothing to do but
    // keep in step
    bool work = key0 < wave_kend;
    if (GEN && work && has_mask) {
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
        // swz(krow) is the same for both halves (32 is a multiple of 16)
        const char* kp0 = kt + l32 * (2 * D);
        auto kfrag = [&](int kh, int ks) {
          return lds_load<u32x4>(kp0 + kh * 32 * (2 * D) + (((2 * ks + h2) ^ swz<CH>(l32)) << 4));
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
        if (diag) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kh + 8 * (r >> 2) + 4 * h2 + (r & 3);
              sacc[kh][r] = key >= lane_kend ? kNegInf : sacc[kh][r];
            }
        }
        if (GEN && has_mask) {
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
            const float p = fast_exp2(__builtin_fmaf(sacc[kh][r], a.qk_scale_log2, -mref));
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
      bool slow = j == 0;
      if (!slow) {
        psum = probs(sacc, m);
        slow = __builtin_amdgcn_ballot_w64(!(psum <= 0x1p30f)) != 0;  // also catches inf / NaN
        if (slow) scores(sacc);
      }
      if (slow) {
        float mt = kNegInf;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kh][r]);
        mt = wave_max_xor(mt, 32) * a.qk_scale_log2;  // scale > 0 keeps the order
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
      // ---- O^T += V^T P^T, 4 k-steps of 16 keys
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f32x16& sp = sacc[p >> 1];
        const int rb = 8 * (p & 1);
        const u32x4 pf = {pack_bf16x2(sp[rb + 0], sp[rb + 1]), pack_bf16x2(sp[rb + 2], sp[rb + 3]),
                          pack_bf16x2(sp[rb + 4], sp[rb + 5]), pack_bf16x2(sp[rb + 6], sp[rb + 7])};
        const int gi = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = 32 * nt + 16 * (gi & 1) + 4 * (s16 & 3);
          const int c = col >> 3, w = col & 7;
          const int ra = 16 * p + 4 * h2 + (s16 >> 2);
          const int rbw = ra + 8;
          const u32x2 va = lds_read_tr16(vt + ra * (2 * D) + ((c ^ swz<CH>(ra)) << 4) + 2 * w);
          const u32x2 vb = lds_read_tr16(vt + rbw * (2 * D) + ((c ^ swz<CH>(rbw)) << 4) + 2 * w);
          const u32x4 vf = {va[0], va[1], vb[0], vb[1]};
          o[nt] = mfma32(vf, pf, o[nt]);
        }
      }
    }
    dma_wait();
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    tile_step(j, sk0, sv0, sm0, sk1, sv1, sm1);
    if (j + 1 < n_tiles) tile_step(j + 1, sk1, sv1, sm1, sk0, sv0, sm0);
  }

  // ---- epilogue: O / l -> bf16, rows < S only
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qrow < S) {
    uint16_t* op = a.out + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * nt + 8 * rq + 4 * h2;
        u32x2 w;
        w[0] = pack_bf16x2(o[nt][4 * rq + 0] * inv, o[nt][4 * rq + 1] * inv);
        w[1] = pack_bf16x2(o[nt][4 * rq + 2] * inv, o[nt][4 * rq + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
  }
}

template <int D, int HC>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_causal_kernel(PrefillArgs a) {
  prefill_body<D, HC, false>(a);
}

template <int D, int HC>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_masked_kernel(PrefillArgs a) {
  prefill_body<D, HC, true>(a);
}

static int gcd_int(int x, int y) {
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
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
  a.S_k = S;
  a.causal = 1;
  a.kv_lens = nullptr;
  a.mask = nullptr;
  return a;
}

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S, int h_q, int n_kv, int D, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  const PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S, h_q, n_kv, HC);
  const dim3 grid(a.n_wg_pad), block(kWaves * 64);
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

hipError_t launch_prefill_masked(const void* q, const void* k, const void* v, void* out, float qk_scale_log2, int B,
                                 int S_q, int S_k, int h_q, int n_kv, int D, int causal, const int32_t* kv_lens,
                                 const uint8_t* mask, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S_q, h_q, n_kv, HC);
  a.S_k = S_k;
  a.causal = causal;
  a.kv_lens = kv_lens;
  a.mask = mask;
  const dim3 grid(a.n_wg_pad), block(kWaves * 64);
#define GQA_LAUNCH_PREFILL(DD, HH) hipLaunchKernelGGL((gqa_prefill_masked_kernel<DD, HH>), grid, block, 0, stream, a)
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

}  // namespace gqa
