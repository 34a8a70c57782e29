// Device-side helpers shared by the gfx950 attention kernels.
//
// Register layouts of the bf16 matrix-core instructions used here (verified on
// gfx950 hardware, lane l of a 64-wide wavefront):
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l % 16][8*(l/16) .. 8*(l/16)+7]
//     B: lane l holds B[8*(l/16) .. +7][l % 16]
//     D: lane l holds D[4*(l/16) + i][l % 16], i = 0..3
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8*(l/32) .. +7]
//     B: lane l holds B[8*(l/32) .. +7][l % 32]
//     D: lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15
// ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes,
//   if lane i reads the 8 bytes E[i][0..3] at its address, lane i receives
//   element j = E[4*j + i/4][i % 4].  So when lane s of the group points at
//   row (r0 + s/4), columns c0 + 4*(s%4) .. +3 of a row-major bf16 tile, lane i
//   receives column c0 + i of rows r0 .. r0+3: a 4x16 block read transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
struct u32x4x2 {
  u32x4 lo, hi;
};
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// D(32x32) += A(32x64) B(64x32) on OCP e4m3 operands (32 bytes per lane each;
// A and B place a given k at the same (lane half, byte) position, so any
// k order that both operands share gives the same product).
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS chunk swizzle of a K/V (or Q) tile: 16-byte chunk c of tile row r is stored at
// chunk position c ^ swz(r).  A row is 256 bytes (d = 128), exactly one pass
// over the 64 four-byte banks, so rows only spread over banks through the
// swizzle.  swz maps r % 16 one-to-one onto 0..15 (the 16 rows of a K
// fragment read hit 16 different chunk positions) and puts r's low two bits
// on the chunk's high two bits: the transposed V reads (4 consecutive rows x
// 4 consecutive chunks for the 32x32 products, 16 rows x 2 chunks for the
// 16x16 ones) then spread evenly over all 16 positions, so every fragment
// read takes the minimum number of bank passes.  With d = 64 (8 chunks, two
// rows per bank pass) the plain r % 8 is used.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return r % CH;
}

// Two float32 -> packed bf16x2 (round to nearest even; lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Four OCP e4m3 codes (one dword) -> four bf16 values (exact: every e4m3 value
// is a bf16 value).  Returns two dwords of packed bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Four signed int8 codes (one dword, code i in byte i) -> four bf16 values;
// exact (|code| <= 128 needs 8 significant bits).
__device__ __forceinline__ u32x2 i8x4_to_bf16x4(uint32_t w) {
  const float f0 = (float)((int)(w << 24) >> 24), f1 = (float)((int)(w << 16) >> 24);
  const float f2 = (float)((int)(w << 8) >> 24), f3 = (float)((int)w >> 24);
  u32x2 r;
  r[0] = pack_bf16x2(f0, f1);
  r[1] = pack_bf16x2(f2, f3);
  return r;
}

// Eight signed int4 codes (one dword, code i in bits 4i .. 4i+3, two's
// complement) -> eight bf16 values, exact.
__device__ __forceinline__ u32x4 i4x8_to_bf16x8(uint32_t w) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)((int)(w << (28 - 4 * i)) >> 28);
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// Eight signed int4 codes (one dword, code i in bits 4i .. 4i+3, two's
// complement) -> eight bf16 values 136 + code, exact, formed from the bit
// patterns alone: code ^ 8 is the offset-binary nibble u = code + 8 in
// 0..15, and a bf16 whose exponent field is that of 128 with u in its low
// mantissa bits is 128 + u (the mantissa step at 128 is 1).  Codes 2k and
// 2k+1 are byte k; or-ing the byte with a copy shifted up by 12 puts code
// 2k+1 in bits 16..19, the low mantissa bits of the upper bf16, so each pair
// costs a bit-field extract, a shift-or and an and-or.  The caller removes
// the 136.
constexpr float kInt4Bias = 136.0f;
__device__ __forceinline__ u32x4 i4x8_to_bf16x8_biased(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = (u >> (8 * k)) & 0xFFu;
    r[k] = ((x | (x << 12)) & 0x000F000Fu) | 0x43004300u;
  }
  return r;
}

// The same values in the order 0 2 4 6 1 3 5 7 (bf16 position j holds code
// pi(j)): with the even codes' nibbles in the bytes of one word and the odd
// ones' in another, each output dword is a byte permute of one of them with
// the bytes 0x43, so eight codes cost a shift, two masks and four permutes.  v_perm_b32 picks result byte k by selector byte k from the
// eight bytes of {first operand : second operand}, 0..3 being the second.
__device__ __forceinline__ u32x4 i4x8_to_bf16x8_biased_eo(uint32_t w) {
  // offset nibbles (code ^ 8) of codes 0 2 4 6 and of codes 1 3 5 7, one per byte
  // (written mask-then-flip so each is one three-input bit operation)
  const uint32_t ev = (w & 0x0F0F0F0Fu) ^ 0x08080808u;
  const uint32_t od = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
  constexpr uint32_t k43 = 0x43434343u;
  return u32x4{__builtin_amdgcn_perm(k43, ev, 0x04010400u), __builtin_amdgcn_perm(k43, ev, 0x04030402u),
               __builtin_amdgcn_perm(k43, od, 0x04010400u), __builtin_amdgcn_perm(k43, od, 0x04030402u)};
}

// Eight bf16 values (one 16-byte chunk, element j in the low half of dword
// j/2 when j is even, the high half when odd) put in the order 0 2 4 6 1 3 5
// 7 used by i4x8_to_bf16x8_biased_eo.
__device__ __forceinline__ u32x4 bf16x8_even_odd(const u32x4& x) {
  return u32x4{__builtin_amdgcn_perm(x[1], x[0], 0x05040100u), __builtin_amdgcn_perm(x[3], x[2], 0x05040100u),
               __builtin_amdgcn_perm(x[1], x[0], 0x07060302u), __builtin_amdgcn_perm(x[3], x[2], 0x07060302u)};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
__device__ __forceinline__ float wave_sum_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

// LDS pointer helpers.
template <typename T>
__device__ __forceinline__ T lds_load(const void* p) {
  return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_store(void* p, const T& v) {
  *reinterpret_cast<T*>(p) = v;
}

// 4 bf16 of a column block, read transposed (see the layout note above).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Compiler-only barrier for LDS traffic private to one wavefront: a wave's LDS
// instructions execute in issue order, so keeping the compiler from moving
// them across this point is all that is needed.
__device__ __forceinline__ void wave_lds_fence() { __asm__ __volatile__("" ::: "memory"); }

__device__ __forceinline__ u32x4 load_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer access (gfx9 buffer resource: base address, byte range, and the
// third-dword format word for 32-bit untyped data).  The base is wave-uniform
// and lives in scalar registers, so each load needs only a 32-bit lane offset;
// a load whose offset (lane offset + immediate) is at or past `bytes` returns
// zero without touching memory.
constexpr int kBufferFormatWord = 0x00020000;
constexpr int kCacheNonTemporal = 2;  // cache-policy operand: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFormatWord);
}

__device__ __forceinline__ u32x4 buffer_load_x4_nt(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNonTemporal));
}

__device__ __forceinline__ u32x4 buffer_load_x4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

}  // namespace gqa
