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
// built around reading every K/V byte exactly once:
//
//  * one workgroup owns a chunk of keys of one (sequence, kv-head) pair and
//    serves every query head of the group (up to 32) from that single read;
//  * 4 wavefronts per workgroup take interleaved 32-token tiles; each tile
//    arrives through 128-bit non-temporal loads (a quarter-wave covers one
//    contiguous 256-byte cache row), is written once to the wave's private
//    LDS slab with an XOR chunk swizzle, and is consumed from there by the
//    matrix cores, while the next tile is already in flight in registers;
//  * scores S^T[token][head] = K Q^T and O^T[d][head] += V^T P^T run on
//    v_mfma_f32_16x16x32_bf16; the token order inside the PV product is
//    permuted so that the score layout produced by the first product is
//    directly the B operand of the second (no shuffles), and V is fetched
//    transposed with ds_read_b64_tr_b16;
//  * softmax is online: per head a running max m (log2 domain) and running
//    sum l; a tile rescales O and l by 2^(m_old - m_new) ("Flash Attention
//    Principle": running max and running sum, write only the final result);
//  * each workgroup leaves an unnormalised partial (O, m, l) per head; the
//    combine kernel merges the partials of all chunks.
// The fp8 path reads e4m3 codes (half the bytes), converts them to bf16
// exactly in registers and folds the per-token scales into the score (K) and
// into the probability (V).  The fp32 path keeps float32 end to end on the
// vector ALUs.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int kDecodeWaves = 4;
constexpr int kTile = 32;      // tokens per wave tile (matrix-core paths)
constexpr int kTileF32 = 64;   // tokens per wave tile (float32 path)

// ------------------------------------------------------------------------
// Matrix-core decode: bf16 Q; bf16 or e4m3 K/V.  HB blocks of 16 heads.
// ------------------------------------------------------------------------
template <int D, int HB, bool FP8>
__global__ __launch_bounds__(256, 2) void gqa_decode_split_mfma(DecodeArgs a) {
  constexpr int CH = D / 8;             // 16-byte bf16 chunks per row
  constexpr int KK = D / 32;            // k-steps of the score product
  constexpr int NT = D / 16;            // 16-wide d tiles of the PV product
  constexpr int TILE_BYTES = kTile * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[kDecodeWaves][2][TILE_BYTES];
  __shared__ float sm_ml[kDecodeWaves][HB * 16][2];

  const int s = blockIdx.x;
  const int g = blockIdx.y / a.n_hchunk;
  const int hc = blockIdx.y - g * a.n_hchunk;
  const int b = blockIdx.z;
  const int L = min(max(a.seq_lens[b], 0), a.S_max);
  const int t_begin = s * a.chunk;
  if (t_begin >= L) return;  // uniform over the workgroup
  const int t_end = min(t_begin + a.chunk, L);
  const int G = a.h_q / a.n_kv;
  const int hloc0 = hc * a.heads_per_chunk;
  const int nh = min(a.heads_per_chunk, G - hloc0);
  const int head0 = g * G + hloc0;  // global index of local head 0

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4;
  const int r16 = lane & 15;

  char* kt = smem[wave][0];
  char* vt = smem[wave][1];

  // ---- Q fragments: B operand of S^T = K Q^T: lane holds Q[head r16][32kk + 8q4 .. +7]
  u32x4 qf[HB][KK];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hl = hb * 16 + r16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hl < nh) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.h_q + head0 + hl) * D + 32 * kk + 8 * q4;
        v = *reinterpret_cast<const u32x4*>(qp);
      }
      qf[hb][kk] = v;
    }
  }

  const size_t slab = ((size_t)b * a.n_kv + g) * (size_t)a.S_max;  // row index of token 0
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;

  // ---- per-lane load assignment.  bf16: a load instruction covers 64/CH rows,
  // each row by CH consecutive lanes.  fp8: rows of D bytes, D/16 lanes per row.
  constexpr int NLD = FP8 ? (kTile * D) / (64 * 16) : (kTile * D * 2) / (64 * 16);
  constexpr int LPR = FP8 ? D / 16 : CH;  // lanes per row
  constexpr int RPL = 64 / LPR;            // rows per load instruction
  const int ld_row = lane / LPR;
  const int ld_chunk = lane % LPR;

  u32x4 kreg[NLD], vreg[NLD];
  float ksc[2][4], vsc[2][4];  // fp8: scales of the lane's 8 score tokens (next tile)

  auto issue_loads = [&](int tile) {
    const int t0 = t_begin + tile * kTile;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int t = t0 + u * RPL + ld_row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (t < t_end) {
        const size_t off = (slab + t) * (size_t)(FP8 ? D : 2 * D) + ld_chunk * 16;
        kv = load_nt(static_cast<const char*>(a.k) + off);
        vv = load_nt(static_cast<const char*>(a.v) + off);
      }
      kreg[u] = kv;
      vreg[u] = vv;
    }
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * h + 4 * q4 + i;
          ksc[h][i] = t < t_end ? a.k_scale[slab + t] : 0.f;
          vsc[h][i] = t < t_end ? a.v_scale[slab + t] : 0.f;
        }
    }
  };

  auto stage_to_lds = [&]() {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int r = u * RPL + ld_row;
      if constexpr (FP8) {
        // 16 codes -> 16 bf16 = logical bf16 chunks 2c, 2c+1 of row r
        const int c0 = 2 * ld_chunk;
        u32x4 klo, khi, vlo, vhi;
        u32x2 t0 = e4m3x4_to_bf16x4(kreg[u][0]), t1 = e4m3x4_to_bf16x4(kreg[u][1]);
        u32x2 t2 = e4m3x4_to_bf16x4(kreg[u][2]), t3 = e4m3x4_to_bf16x4(kreg[u][3]);
        klo = u32x4{t0[0], t0[1], t1[0], t1[1]};
        khi = u32x4{t2[0], t2[1], t3[0], t3[1]};
        t0 = e4m3x4_to_bf16x4(vreg[u][0]); t1 = e4m3x4_to_bf16x4(vreg[u][1]);
        t2 = e4m3x4_to_bf16x4(vreg[u][2]); t3 = e4m3x4_to_bf16x4(vreg[u][3]);
        vlo = u32x4{t0[0], t0[1], t1[0], t1[1]};
        vhi = u32x4{t2[0], t2[1], t3[0], t3[1]};
        const int sw = r % CH;
        lds_store(kt + r * (2 * D) + ((c0 ^ sw) << 4), klo);
        lds_store(kt + r * (2 * D) + (((c0 + 1) ^ sw) << 4), khi);
        lds_store(vt + r * (2 * D) + ((c0 ^ sw) << 4), vlo);
        lds_store(vt + r * (2 * D) + (((c0 + 1) ^ sw) << 4), vhi);
      } else {
        const int pc = ld_chunk ^ (r % CH);
        lds_store(kt + r * (2 * D) + (pc << 4), kreg[u]);
        lds_store(vt + r * (2 * D) + (pc << 4), vreg[u]);
      }
    }
  };

  // ---- running state (per lane: head r16 of every head block)
  f32x4 o[HB][NT];
  float m[HB], l[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m[hb] = kNegInf;
    l[hb] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[hb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int tile = wave;
  if (tile < n_tiles) issue_loads(tile);
  for (; tile < n_tiles; tile += kDecodeWaves) {
    float kscur[2][4], vscur[2][4];
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) { kscur[h][i] = ksc[h][i]; vscur[h][i] = vsc[h][i]; }
    }
    wave_lds_fence();
    stage_to_lds();
    wave_lds_fence();
    if (tile + kDecodeWaves < n_tiles) issue_loads(tile + kDecodeWaves);

    const int t0 = t_begin + tile * kTile;
    // ---- scores S^T[token][head]: two 16-token halves
    f32x4 sc[2][HB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + r16;
      u32x4 kf[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kf[kk] = lds_load<u32x4>(kt + row * (2 * D) + (((4 * kk + q4) ^ (row % CH)) << 4));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) acc = mfma16(kf[kk], qf[hb][kk], acc);
        sc[h][hb] = acc;
      }
    }
    // ---- V fragments (A operand of O^T = V^T P^T), shared by all head blocks
    u32x4 vf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      u32x2 lo, hi;
      {
        const int row = 4 * q4 + (r16 >> 2);
        const int col = 16 * nt + 4 * (r16 & 3);  // bf16 column
        const int c = col >> 3, w = col & 7;
        lo = lds_read_tr16(vt + row * (2 * D) + ((c ^ (row % CH)) << 4) + 2 * w);
      }
      {
        const int row = 16 + 4 * q4 + (r16 >> 2);
        const int col = 16 * nt + 4 * (r16 & 3);
        const int c = col >> 3, w = col & 7;
        hi = lds_read_tr16(vt + row * (2 * D) + ((c ^ (row % CH)) << 4) + 2 * w);
      }
      vf[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    wave_lds_fence();

    // ---- online softmax per head block and PV
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float sv[2][4];
      float mt = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * h + 4 * q4 + i;
          float x = sc[h][hb][i] * a.qk_scale_log2;
          if constexpr (FP8) x *= kscur[h][i];
          x = t < t_end ? x : kNegInf;
          sv[h][i] = x;
          mt = fmaxf(mt, x);
        }
      mt = wave_max_xor(mt, 16);
      mt = wave_max_xor(mt, 32);
      const float m_new = fmaxf(m[hb], mt);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m[hb] - m_use);
      m[hb] = m_new;
      float psum = 0.f;
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[h][i] = fast_exp2(sv[h][i] - m_use);
          psum += p[h][i];
        }
      l[hb] = l[hb] * alpha + psum;
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[h][i] *= vscur[h][i];
      }
      const u32x4 pf = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]), pack_bf16x2(p[1][0], p[1][1]),
                        pack_bf16x2(p[1][2], p[1][3])};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        o[hb][nt] *= alpha;
        o[hb][nt] = mfma16(vf[nt], pf, o[hb][nt]);
      }
    }
  }

  // ---- merge the 4 waves of the workgroup, write one partial per head
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float lt = wave_sum_xor(l[hb], 16);
    lt = wave_sum_xor(lt, 32);
    l[hb] = lt;
  }
  wave_lds_fence();
  // O^T[d = 16nt + 4q4 + i][head r16] -> ow[head][d] (float32), reusing the tile slab
  float* ow = reinterpret_cast<float*>(smem[wave][0]);
  static_assert(HB * 16 * D * 4 <= 2 * TILE_BYTES, "partial O does not fit the wave slab");
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lds_store(ow + (hb * 16 + r16) * D + 16 * nt + 4 * q4, o[hb][nt]);
    if (q4 == 0) {
      sm_ml[wave][hb * 16 + r16][0] = m[hb];
      sm_ml[wave][hb * 16 + r16][1] = l[hb];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nh * D; e += 256) {
    const int hl = e / D, d = e - hl * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_ml[w][hl][0]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = sm_ml[w][hl][0];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      acc += f * reinterpret_cast<const float*>(smem[w][0])[hl * D + d];
      lsum += f * sm_ml[w][hl][1];
    }
    const size_t row = ((size_t)b * a.h_q + head0 + hl) * a.n_split + s;
    a.part_o[row * D + d] = acc;
    if (d == 0) {
      a.part_ml[row * 2 + 0] = M;
      a.part_ml[row * 2 + 1] = lsum;
    }
  }
}

// ------------------------------------------------------------------------
// float32 decode on the vector ALUs (16 heads per workgroup).
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void gqa_decode_split_f32(DecodeArgs a) {
  constexpr int HPC = 16;
  constexpr int DL = D / 64;  // d columns per lane in the PV product
  __shared__ __attribute__((aligned(16))) float sq[HPC][D];
  __shared__ float sp[kDecodeWaves][kTileF32][HPC];
  __shared__ __attribute__((aligned(16))) float so[kDecodeWaves][HPC][D];
  __shared__ float sm_ml[kDecodeWaves][HPC][2];

  const int s = blockIdx.x;
  const int g = blockIdx.y / a.n_hchunk;
  const int hc = blockIdx.y - g * a.n_hchunk;
  const int b = blockIdx.z;
  const int L = min(max(a.seq_lens[b], 0), a.S_max);
  const int t_begin = s * a.chunk;
  if (t_begin >= L) return;
  const int t_end = min(t_begin + a.chunk, L);
  const int G = a.h_q / a.n_kv;
  const int hloc0 = hc * HPC;
  const int nh = min(HPC, G - hloc0);
  const int head0 = g * G + hloc0;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  const float* qg = static_cast<const float*>(a.q);
  for (int e = threadIdx.x; e < HPC * D; e += 256) {
    const int hl = e / D, d = e - hl * D;
    sq[hl][d] = hl < nh ? qg[((size_t)b * a.h_q + head0 + hl) * D + d] : 0.f;
  }
  __syncthreads();

  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);
  const size_t slab = ((size_t)b * a.n_kv + g) * (size_t)a.S_max;
  const int n_tiles = (t_end - t_begin + kTileF32 - 1) / kTileF32;

  float m[HPC], l[HPC], o[HPC][DL];
#pragma unroll
  for (int h = 0; h < HPC; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < DL; ++c) o[h][c] = 0.f;
  }

  for (int tile = wave; tile < n_tiles; tile += kDecodeWaves) {
    const int t0 = t_begin + tile * kTileF32;
    const int t = t0 + lane;
    const bool valid = t < t_end;
    float sc[HPC];
#pragma unroll
    for (int h = 0; h < HPC; ++h) sc[h] = 0.f;
    if (valid) {
      const float4* kr = reinterpret_cast<const float4*>(kg + (slab + t) * D);
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
    const int nvalid = min(kTileF32, t_end - t0);
#pragma unroll
    for (int h = 0; h < HPC; ++h)
#pragma unroll
      for (int c = 0; c < DL; ++c) o[h][c] *= alpha[h];
    for (int tt = 0; tt < nvalid; ++tt) {
      const float* vr = vg + (slab + t0 + tt) * D;
      float vv[DL];
#pragma unroll
      for (int c = 0; c < DL; ++c) vv[c] = vr[lane + 64 * c];
#pragma unroll
      for (int h = 0; h < HPC; ++h) {
        const float p = sp[wave][tt][h];
#pragma unroll
        for (int c = 0; c < DL; ++c) o[h][c] = fmaf(p, vv[c], o[h][c]);
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
  for (int e = threadIdx.x; e < nh * D; e += 256) {
    const int hl = e / D, d = e - hl * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_ml[w][hl][0]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = sm_ml[w][hl][0];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      acc += f * so[w][hl][d];
      lsum += f * sm_ml[w][hl][1];
    }
    const size_t row = ((size_t)b * a.h_q + head0 + hl) * a.n_split + s;
    a.part_o[row * D + d] = acc;
    if (d == 0) {
      a.part_ml[row * 2 + 0] = M;
      a.part_ml[row * 2 + 1] = lsum;
    }
  }
}

// ------------------------------------------------------------------------
// Combine: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  One wave per
// (sequence, query head); chunks past the sequence end were never written
// and are not read.
// ------------------------------------------------------------------------
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void gqa_decode_combine(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ seq_lens, void* out, int B,
                                                          int h_q, int S_max, int chunk, int n_split) {
  constexpr int DL = D / 64;
  const int row_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row_id >= B * h_q) return;
  const int b = row_id / h_q;
  const int L = min(max(seq_lens[b], 0), S_max);
  const int ns = (L + chunk - 1) / chunk;
  const size_t base = (size_t)row_id * n_split;
  float acc[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) acc[c] = 0.f;
  float denom = 0.f;
  if (ns > 0) {
    float M = kNegInf;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, part_ml[(base + s) * 2]);
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) M = wave_max_xor(M, msk);
    for (int s = 0; s < ns; ++s) {
      const float ms = part_ml[(base + s) * 2];
      const float ls = part_ml[(base + s) * 2 + 1];
      const float w = ms == kNegInf ? 0.f : fast_exp2(ms - M);
      denom += w * ls;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc[c] += w * part_o[(base + s) * D + lane + 64 * c];
    }
  }
  const float inv = denom > 0.f ? 1.0f / denom : 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    const float v = acc[c] * inv;
    const size_t idx = (size_t)row_id * D + lane + 64 * c;
    if constexpr (OUT_BF16) {
      static_cast<__bf16*>(out)[idx] = (__bf16)v;
    } else {
      static_cast<float*>(out)[idx] = v;
    }
  }
}

// ------------------------------------------------------------------------
// Host-side launchers (called from api.cpp).
// ------------------------------------------------------------------------
hipError_t launch_decode_split(const DecodeArgs& a, int B, int D, int hb, int kind, hipStream_t stream) {
  const dim3 grid(a.n_split, a.n_kv * a.n_hchunk, B);
  const dim3 block(256);
  // kind: 0 = f32, 1 = bf16 K/V, 2 = fp8 K/V
  if (kind == 0) {
    if (D == 64) hipLaunchKernelGGL(gqa_decode_split_f32<64>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(gqa_decode_split_f32<128>, grid, block, 0, stream, a);
  } else if (kind == 1) {
    if (D == 64 && hb == 1) hipLaunchKernelGGL((gqa_decode_split_mfma<64, 1, false>), grid, block, 0, stream, a);
    else if (D == 64) hipLaunchKernelGGL((gqa_decode_split_mfma<64, 2, false>), grid, block, 0, stream, a);
    else if (hb == 1) hipLaunchKernelGGL((gqa_decode_split_mfma<128, 1, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_split_mfma<128, 2, false>), grid, block, 0, stream, a);
  } else {
    if (D == 64 && hb == 1) hipLaunchKernelGGL((gqa_decode_split_mfma<64, 1, true>), grid, block, 0, stream, a);
    else if (D == 64) hipLaunchKernelGGL((gqa_decode_split_mfma<64, 2, true>), grid, block, 0, stream, a);
    else if (hb == 1) hipLaunchKernelGGL((gqa_decode_split_mfma<128, 1, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gqa_decode_split_mfma<128, 2, true>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const float* part_o, const float* part_ml, const int32_t* seq_lens, void* out,
                                 bool out_bf16, int B, int h_q, int S_max, int D, int chunk, int n_split,
                                 hipStream_t stream) {
  const dim3 grid((B * h_q + 3) / 4);
  const dim3 block(256);
  if (D == 64) {
    if (out_bf16) hipLaunchKernelGGL((gqa_decode_combine<64, true>), grid, block, 0, stream, part_o, part_ml, seq_lens, out, B, h_q, S_max, chunk, n_split);
    else hipLaunchKernelGGL((gqa_decode_combine<64, false>), grid, block, 0, stream, part_o, part_ml, seq_lens, out, B, h_q, S_max, chunk, n_split);
  } else {
    if (out_bf16) hipLaunchKernelGGL((gqa_decode_combine<128, true>), grid, block, 0, stream, part_o, part_ml, seq_lens, out, B, h_q, S_max, chunk, n_split);
    else hipLaunchKernelGGL((gqa_decode_combine<128, false>), grid, block, 0, stream, part_o, part_ml, seq_lens, out, B, h_q, S_max, chunk, n_split);
  }
  return hipGetLastError();
}

}  // namespace gqa
