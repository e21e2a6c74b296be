// Device-side building blocks of the MXFP8 kernels (gfx950 / CDNA4).
//
// Format facts used here (Mojo DistributedAllGatherRMSNormQuantMXFP8 page,
// "Parameters": float8_e4m3fn elements, float8_e8m0fnu scales; Megatron-Core
// quantized_dbuffer page, "Data": blocks of 32):
//   bf16 is the top half of an IEEE binary32, so a bf16 pair sits in one dword
//   and the magnitude bits (bits & 0x7FFF) order finite values by |x|;
//   a block's scale byte is S = clamp(floor(log2 amax) - 8 + 127, 0, 254),
//   0xFF for a block holding Inf/NaN (OCP MX v1.0, taken where the pages are
//   silent); elements are e4m3fn(x * 2^(127 - S)), nearest-even, saturating
//   at +-448.
//
// Encoding uses the gfx950 fp8 conversion instructions only in forms that
// were checked exhaustively on the GPU against the rounding rule above
// (every bf16 value times every scale byte):
//   v_cvt_scalef32_pk_fp8_bf16 with scale 2^(S-127) rounds to nearest even
//   and divides by the scale exactly, but turns magnitudes >= 464 into NaN;
//   clamping the bf16 magnitude to 448 * 2^(S-127) first gives the saturating
//   result;
//   v_cvt_pk_fp8_f32 of x * 2^(127-S) clamped to [-448, 448] (v_med3_f32) is
//   exact, subnormals and the sign of zero included.
// Every other step is integer work on bit patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kBlock = 32;          // elements per MX block
constexpr int kChunk = 8;           // bf16 elements per lane per 16-byte load
constexpr int kWave = 64;           // CDNA wavefront

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
      __builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
      __builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}

// Magnitude bits of both halves of a bf16 pair.
__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }

// Largest magnitude key among the 8 bf16 values of a 16-byte chunk.
__device__ __forceinline__ uint32_t chunk_key(const u32x4& v) {
  uint32_t m = pk_max_u16(pk_max_u16(mag2(v.x), mag2(v.y)),
                          pk_max_u16(mag2(v.z), mag2(v.w)));
  return max(m & 0xFFFFu, m >> 16);
}

// Max over the 4 lanes of each aligned lane quad (a 32-element block when
// each lane holds 8 consecutive elements), via DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max(uint32_t k) {
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return k;
}

// E8M0 scale byte from a block's magnitude key.  For a finite key the bf16
// exponent field key >> 7 is floor(log2 amax) + 127 (bf16 subnormals and
// zero have field 0 and land on the clamp), so S = field - 8, clamped at 0.
__device__ __forceinline__ uint32_t scale_byte(uint32_t key) {
  int s = (int)(key >> 7) - 8;
  s = s < 0 ? 0 : s;
  return key >= 0x7F80u ? 0xFFu : (uint32_t)s;
}

// ---- rowwise encode: one scale for the whole chunk ------------------------

struct RowScale {
  float div;      // 2^(S - 127) as float32 (S == 0: the subnormal 2^-127)
  uint32_t lim2;  // bf16 magnitude of 448 * 2^(S - 127), in both halves
  uint32_t nan4;  // 0x7F7F7F7F for a NaN/Inf block, else 0
};

__device__ __forceinline__ RowScale row_scale(uint32_t s) {
  // A NaN/Inf block is converted with the finite stand-in scale 2^0: the
  // clamp below maps NaN/Inf magnitudes to 448 with their own sign, and nan4
  // then turns every byte into sign | 0x7F.
  const uint32_t se = s == 0xFFu ? 127u : s;
  RowScale r;
  r.div = __builtin_bit_cast(float, se ? (se << 23) : 0x00400000u);
  uint32_t lim = ((se + 8u) << 7) | 0x60u;  // 1.75 * 2^(S + 8 - 127) as bf16
  r.lim2 = lim | (lim << 16);
  r.nan4 = s == 0xFFu ? 0x7F7F7F7Fu : 0u;
  return r;
}

// Two e4m3 bytes of a bf16 pair (low byte = low half) in the low 16 bits.
template <bool HI>
__device__ __forceinline__ v2i16 cvt_pair(uint32_t w, const RowScale& rs, v2i16 old) {
  uint32_t clamped = (w & 0x80008000u) | pk_min_u16(mag2(w), rs.lim2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      old, __builtin_bit_cast(v2bf16, clamped), rs.div, HI);
}

// 8 e4m3 bytes of a chunk, in element order.
__device__ __forceinline__ u32x2 encode_chunk_row(const u32x4& v, const RowScale& rs) {
  v2i16 z = {0, 0};
  v2i16 a = cvt_pair<false>(v.x, rs, z);
  a = cvt_pair<true>(v.y, rs, a);
  v2i16 b = cvt_pair<false>(v.z, rs, z);
  b = cvt_pair<true>(v.w, rs, b);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, a) | rs.nan4;
  r.y = __builtin_bit_cast(uint32_t, b) | rs.nan4;
  return r;
}

// ---- columnwise encode: one scale per element column ----------------------

// 2^(127 - S) as float32 (S <= 246 for any finite bf16 block); a NaN/Inf
// column (S = 0xFF) gets 1.0, its elements having been reduced to signed
// zeros by the caller before conversion.
__device__ __forceinline__ float col_mul(uint32_t s) {
  return s == 0xFFu ? 1.0f : __builtin_bit_cast(float, (uint32_t)(254 - (int)s) << 23);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Two e4m3 bytes of a bf16 pair whose halves have their own multipliers.
template <bool HI>
__device__ __forceinline__ int cvt_pair_cols(uint32_t w, float m_lo, float m_hi, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(bf16_lo(w) * m_lo),
                                         clamp448(bf16_hi(w) * m_hi), old, HI);
}

// 8 e4m3 bytes of a chunk whose 8 columns have multipliers m[0..7];
// nan8 holds 0x7F in the byte of every NaN/Inf column, whose input halves
// must already be reduced to their sign bit.
__device__ __forceinline__ u32x2 encode_chunk_cols(const u32x4& v, const float* m,
                                                   u32x2 nan8) {
  int a = cvt_pair_cols<false>(v.x, m[0], m[1], 0);
  a = cvt_pair_cols<true>(v.y, m[2], m[3], a);
  int b = cvt_pair_cols<false>(v.z, m[4], m[5], 0);
  b = cvt_pair_cols<true>(v.w, m[6], m[7], b);
  u32x2 r;
  r.x = (uint32_t)a | nan8.x;
  r.y = (uint32_t)b | nan8.y;
  return r;
}

// ---- decode ----------------------------------------------------------------

// Exact float32 value of e4m3 byte b times 2^(S - 127); NaN for element
// 0x7F / 0xFF or scale 0xFF.
__device__ __forceinline__ float decode_e4m3(uint32_t b, float scale) {
  uint32_t mag = b & 0x7Fu;
  // exponent field >= 1: (1 + m/8) * 2^(e - 7) is float32 bits (mag << 20) + (120 << 23)
  float v = mag >= 8u ? __builtin_bit_cast(float, (mag << 20) + (120u << 23))
                      : (float)mag * 0x1p-9f;  // subnormal m * 2^-9, exact
  v = v * scale;                              // exact: power of two, denormals kept
  uint32_t u = __builtin_bit_cast(uint32_t, v) | ((b & 0x80u) << 24);
  return mag == 0x7Fu ? __builtin_bit_cast(float, 0x7FC00000u | ((b & 0x80u) << 24))
                      : __builtin_bit_cast(float, u);
}

// 2^(S - 127) as float32; NaN for S = 0xFF.
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return s == 0xFFu ? __builtin_bit_cast(float, 0x7FC00000u)
                    : __builtin_bit_cast(float, s ? (s << 23) : 0x00400000u);
}

typedef float v2f32 __attribute__((ext_vector_type(2)));

// Two float32 -> a bf16 pair (lo in the low half) with v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  v2f32 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf16));
}

// float32 -> bf16 bits by integer arithmetic: nearest even, subnormals
// included; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : r;
}

// ---- memory ----------------------------------------------------------------

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void store8(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace mx
