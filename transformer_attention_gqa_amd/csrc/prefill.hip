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
  // fp8 kernel: q/k/v hold e4m3 codes; value = code * descale[b][head]
  const float* q_descale;   // [B][h_q]
  const float* k_descale;   // [B][n_kv]
  const float* v_descale;   // [B][n_kv]
};

constexpr int kBN = 64;  // keys per tile
constexpr int kNumXcd = 8;
constexpr int kWaves = 8;  // wavefronts per workgroup

// GEN = false: causal self-attention, S_q = S_k, every key of a row's causal
// range visible.  GEN = true: S_q and S_k independent, the causal rule
// optional and end-aligned, optional key lengths and dense mask; rows can
// then have no visible key at all (zero output).
// F8: q, k, v are OCP e4m3 codes with one descale factor per (batch, head)
// (the FP8 mode of FlashAttention-3, "Flash Attention 3 Features"); both
// products run on v_mfma_f32_32x32x64_f8f6f4, P rounded to e4m3 (kept <= 256
// by the reference max, below the format's 448), d = 128 only.
// MASK (with GEN): a dense mask is given; without it the mask machinery
// (tile bitmaps, mask tiles, per-element masking) is compiled out.
template <int D, int HC, bool GEN, bool F8 = false, bool MASK = false>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a) {
  static_assert(!F8 || (D == 128 && GEN), "the fp8 body serves d = 128 with general masks");
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
  auto sw = [](int r) {
    if constexpr (F8) {
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
  const size_t kv_row_bytes = (size_t)a.n_kv * ROWB;

  // ---- Q fragments (B operand of S^T = K Q^T).  bf16: Q[qrow][16ks + 8h2 ..
  // +7]; fp8: Q[qrow][64ks + 32h2 .. +31] (the K fragments take the same k order)
  u32x4 qf[F8 ? 1 : KS];
  i32x8 qf8[F8 ? KS8 : 1];
  float qk_log2 = a.qk_scale_log2, out_scale = 1.0f;
  if constexpr (!F8) {
    const uint16_t* qp = a.q + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < S) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qf[ks] = v;
    }
  } else {
    const char* qp = reinterpret_cast<const char*>(a.q) + ((size_t)b * S + qrow) * q_row_stride + (size_t)head * D +
                     32 * h2;
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (qrow < S) {
        lo = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
        hi = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
      }
      qf8[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    qk_log2 *= a.q_descale[(size_t)b * a.h_q + head] * a.k_descale[(size_t)b * a.n_kv + g];
    out_scale = a.v_descale[(size_t)b * a.n_kv + g];
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

  const char* kbase = reinterpret_cast<const char*>(a.k) + ((size_t)b * SK * a.n_kv + g) * ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((size_t)b * SK * a.n_kv + g) * ROWB;
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
    dma_off[u] = (uint32_t)(r * kv_row_bytes + (dma_c ^ sw(r)) * 16);
  }
  auto dma_tile = [&](int j, char* kdst, char* vdst) {
    const int key0 = j * kBN;
    if (key0 + kBN <= kv_n) {
      const char* kt = kbase + (size_t)key0 * kv_row_bytes;
      const char* vt = vbase + (size_t)key0 * kv_row_bytes;
#pragma unroll
      for (int u = 0; u < NINS; ++u) {
        const int r0 = (u * kWaves + wave) * RPI;  // first tile row of this instruction
        __builtin_amdgcn_global_load_lds(kt + dma_off[u], (lds_void*)(kdst + r0 * ROWB), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + dma_off[u], (lds_void*)(vdst + r0 * ROWB), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NINS; ++u) {
        const int r0 = (u * kWaves + wave) * RPI;
        const int r = r0 + dma_r;
        const int key = min(key0 + r, kv_n - 1);
        const int c = dma_c ^ sw(r);              // logical chunk stored at this slot
        const size_t off = (size_t)key * kv_row_bytes + c * 16;
        __builtin_amdgcn_global_load_lds(kbase + off, (lds_void*)(kdst + r0 * ROWB), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + off, (lds_void*)(vdst + r0 * ROWB), 16, 0, 0);
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
  constexpr int kVisWords = has_mask ? 256 : 1;  // up to 8192 key tiles
  __shared__ uint32_t s_vis[kVisWords];
  __shared__ uint32_t s_full[kVisWords];
  const bool skip_tiles = has_mask && n_tiles <= kVisWords * 32;
  int n_steps = n_tiles;  // key tiles the loop visits
  if (skip_tiles) {
    for (int i = tid; i < kVisWords; i += kWaves * 64) {
      s_vis[i] = 0u;
      s_full[i] = 0u;
    }
    __syncthreads();
    const int nrows = min(BM, S - blk0);
    constexpr int TPI = 4;  // tiles per wave and pass: their loads are in flight together
    for (int j0 = wave; j0 < n_tiles; j0 += TPI * kWaves) {
      uint32_t any[TPI], zero[TPI];
#pragma unroll
      for (int u = 0; u < TPI; ++u) {
        any[u] = 0u;
        zero[u] = 0u;
      }
      for (int r = lane; r < nrows; r += 64) {
#pragma unroll
        for (int u = 0; u < TPI; ++u) {
          const unsigned off = (unsigned)r * (unsigned)SK + (unsigned)((j0 + u * kWaves) * kBN);
#pragma unroll
          for (int i = 0; i < kBN / 16; ++i) {
            const u32x4 mv = buffer_load_x4(mrsrc, off + 16 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              any[u] |= mv[e];
              zero[u] |= (mv[e] - 0x01010101u) & ~mv[e] & 0x80808080u;  // nonzero iff a byte is 0
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < TPI; ++u) {
        const int j = j0 + u * kWaves;
        const bool vis = __builtin_amdgcn_ballot_w64(any[u] != 0u) != 0;
        const bool full = __builtin_amdgcn_ballot_w64(zero[u] != 0u) == 0;
        if (j < n_tiles && lane == 0) {
          if (vis) atomicOr(&s_vis[j >> 5], 1u << (j & 31));
          if (full) atomicOr(&s_full[j >> 5], 1u << (j & 31));
        }
      }
    }
    __syncthreads();
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
    return;
  }
  const int j_first = next_tile_of(-1);
  dma_tile(j_first, sk0, sv0);
  if (masked_tile(j_first)) dma_mask(j_first, sm0);
  dma_wait();
  __syncthreads();

  // step k visits key tile j: compute from (kt, vt) while the next visited
  // tile fills (kn, vn); returns that next tile
  auto tile_step = [&](int k, int j, const char* kt, const char* vt, const char* mt, char* kn, char* vn, char* mn) {
    // the other buffer was last read in step k-1, before its closing barrier
    const int jn = next_tile_of(j);
    if (k + 1 < n_steps) {
      dma_tile(jn, kn, vn);
      if (masked_tile(jn)) dma_mask(jn, mn);
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
        // ---- O^T += V^T P^T on one 64-key product per 32-wide d tile.  P
        // byte b = 16kh + r of a lane is the score register sacc[kh][r], key
        // 32kh + 8(r/4) + 4h2 + r%4.  ds_read_b64_tr_b8 hands output lane
        // 16gg + 8u + c byte j of source lane 16gg + 2j + u (byte c of its 8):
        // source lane (gg, j, u) therefore reads, for read t (bytes 8t..8t+7),
        // key 32(t/2) + 16(t%2) + 8(j/4) + 4(gg/2) + j%4 at d columns
        // 32dt + 16(gg%2) + 8u .. +7, so that output lane l holds d = 32dt +
        // l%32 for exactly the keys of its P bytes.
        i32x8 pf8;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const f32x16& sp = sacc[w >> 2];
          const int r0 = 4 * (w & 3);
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0], sp[r0 + 1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(sp[r0 + 2], sp[r0 + 3], x, true);
          pf8[w] = x;
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
        }
      } else {
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
          const u32x2 va = lds_read_tr16(vt + ra * ROWB + ((c ^ sw(ra)) << 4) + 2 * w);
          const u32x2 vb = lds_read_tr16(vt + rbw * ROWB + ((c ^ sw(rbw)) << 4) + 2 * w);
          const u32x4 vf = {va[0], va[1], vb[0], vb[1]};
          o[nt] = mfma32(vf, pf, o[nt]);
        }
      }
      }
    }
    dma_wait();
    __syncthreads();
    return jn;
  };
  int j = j_first;
  for (int k = 0; k < n_steps; k += 2) {
    j = tile_step(k, j, sk0, sv0, sm0, sk1, sv1, sm1);
    if (k + 1 < n_steps) j = tile_step(k + 1, j, sk1, sv1, sm1, sk0, sv0, sm0);
  }

  // ---- epilogue: O / l -> bf16, rows < S only
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = lt > 0.f ? out_scale / lt : 0.f;  // fp8: the V descale folds in here
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

template <int D, int HC, bool MASK>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_masked_kernel(PrefillArgs a) {
  prefill_body<D, HC, true, false, MASK>(a);
}

template <int HC, bool MASK>
__global__ __launch_bounds__(kWaves * 64, 1) void gqa_prefill_fp8_kernel(PrefillArgs a) {
  prefill_body<128, HC, true, true, MASK>(a);
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
  a.q_descale = nullptr;
  a.k_descale = nullptr;
  a.v_descale = nullptr;
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
                              int S_q, int S_k, int h_q, int n_kv, int causal, const int32_t* kv_lens,
                              const uint8_t* mask, const float* q_descale, const float* k_descale,
                              const float* v_descale, hipStream_t stream) {
  const int HC = gcd_int(h_q / n_kv, kWaves);
  PrefillArgs a = prefill_args(q, k, v, out, qk_scale_log2, B, S_q, h_q, n_kv, HC);
  a.S_k = S_k;
  a.causal = causal;
  a.kv_lens = kv_lens;
  a.mask = mask;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  const dim3 grid(a.n_wg_pad), block(kWaves * 64);
#define GQA_LAUNCH_FP8(HH)                                                                              \
  do {                                                                                                  \
    if (mask) hipLaunchKernelGGL((gqa_prefill_fp8_kernel<HH, true>), grid, block, 0, stream, a);        \
    else hipLaunchKernelGGL((gqa_prefill_fp8_kernel<HH, false>), grid, block, 0, stream, a);            \
  } while (0)
  if (HC == 8) GQA_LAUNCH_FP8(8);
  else if (HC == 4) GQA_LAUNCH_FP8(4);
  else if (HC == 2) GQA_LAUNCH_FP8(2);
  else GQA_LAUNCH_FP8(1);
#undef GQA_LAUNCH_FP8
  return hipGetLastError();
}

}  // namespace gqa
