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

constexpr u32x4 kZero4 = {0, 0, 0, 0};

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
      __builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
      __builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}

typedef short v2s16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_min_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
      __builtin_bit_cast(v2s16, a), __builtin_bit_cast(v2s16, b)));
}

// Both bf16 halves of w with their magnitude clamped to the halves of lim
// (each <= 0x7FFF), signs kept; NaN and Inf clamp like large numbers.  As
// unsigned 16-bit values negatives lie above 0x8000, so min_u16 against
// 0x8000 | lim clamps the negatives and passes the positives; as signed
// values the positives are the larger ones, so min_i16 against lim then
// clamps the positives and passes the (clamped) negatives.
__device__ __forceinline__ uint32_t clamp_mag(uint32_t w, uint32_t lim) {
  return pk_min_i16(pk_min_u16(w, lim | 0x80008000u), lim);
}

// float32 values of the low and high bf16 halves of a dword.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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

// ---- rowwise encode: one scale for the whole chunk ------------------------

struct RowScale {
  float div;      // 2^(S - 127) as float32 bits S << 23 (S == 0 gives +0.0, which the
                  // conversion reads, like every scale operand, by its exponent field)
  uint32_t lim2;  // bf16 magnitude of 448 * 2^(S - 127), in both halves
  uint32_t nan4;  // 0x7F7F7F7F for a NaN/Inf block, else 0
  uint32_t sbyte; // the stored scale byte (0xFF for a NaN/Inf block)
};

// Scale parameters of a block from its magnitude key.  A NaN/Inf block is
// converted with the finite stand-in key 0x7F7F: the clamp then maps its
// NaN/Inf magnitudes to 448 with their own sign, and nan4 turns every byte
// into sign | 0x7F.
__device__ __forceinline__ RowScale row_scale_key(uint32_t key) {
  const uint32_t e = min(key, 0x7F7Fu) >> 7;     // bf16 exponent field
  const uint32_t s = e > 8u ? e - 8u : 0u;
  const bool nan = key >= 0x7F80u;
  RowScale r;
  r.div = __builtin_bit_cast(float, s << 23);
  const uint32_t lim = (max(e, 8u) << 7) | 0x60u;  // 1.75 * 2^(S + 8 - 127) as bf16
  r.lim2 = lim | (lim << 16);
  r.nan4 = nan ? 0x7F7F7F7Fu : 0u;
  r.sbyte = nan ? 0xFFu : s;
  return r;
}

// Two e4m3 bytes of a bf16 pair (low byte = low half) in the low 16 bits.
template <bool HI>
__device__ __forceinline__ v2i16 cvt_pair(uint32_t w, const RowScale& rs, v2i16 old) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      old, __builtin_bit_cast(v2bf16, clamp_mag(w, rs.lim2)), rs.div, HI);
}

// Same, for the low half of a fresh dword: the input's own register serves
// as the (fully overwritten) old value, so no zero has to be materialized.
__device__ __forceinline__ v2i16 cvt_pair_first(uint32_t w, const RowScale& rs) {
  const uint32_t c = clamp_mag(w, rs.lim2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(v2i16, c), __builtin_bit_cast(v2bf16, c), rs.div, false);
}

// 8 e4m3 bytes of a chunk, in element order.
__device__ __forceinline__ u32x2 encode_chunk_row(const u32x4& v, const RowScale& rs) {
  v2i16 a = cvt_pair_first(v.x, rs);
  a = cvt_pair<true>(v.y, rs, a);
  v2i16 b = cvt_pair_first(v.z, rs);
  b = cvt_pair<true>(v.w, rs, b);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, a) | rs.nan4;
  r.y = __builtin_bit_cast(uint32_t, b) | rs.nan4;
  return r;
}

// Largest magnitude key among 16 bf16 values (two chunks).
__device__ __forceinline__ uint32_t chunk16_key(const u32x4& a, const u32x4& b) {
  uint32_t m = pk_max_u16(pk_max_u16(pk_max_u16(mag2(a.x), mag2(a.y)),
                                     pk_max_u16(mag2(a.z), mag2(a.w))),
                          pk_max_u16(pk_max_u16(mag2(b.x), mag2(b.y)),
                                     pk_max_u16(mag2(b.z), mag2(b.w))));
  return max(m & 0xFFFFu, m >> 16);
}

// Max over each aligned lane pair (a 32-element block when each lane holds
// 16 consecutive elements), one DPP quad permute.
__device__ __forceinline__ uint32_t pair_max(uint32_t k) {
  return max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
}

// 16 e4m3 bytes of two chunks sharing one block scale.
__device__ __forceinline__ u32x4 encode_chunk16_row(const u32x4& a, const u32x4& b,
                                                    const RowScale& rs) {
  const u32x2 lo = encode_chunk_row(a, rs);
  const u32x2 hi = encode_chunk_row(b, rs);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// ---- columnwise encode on row pairs ----------------------------------------
//
// A lane holds rows r, r+1 of columns 2j, 2j+1 as two bf16-pair dwords.  The
// two rows of one column are gathered into one dword (v_perm_b32), converted
// with that column's scale by v_cvt_scalef32_pk_fp8_bf16, and the resulting
// bytes are permuted back into row order.

// Packed per-column parameters for the two columns of pair-dword j.
struct ColPair {
  uint32_t lim;     // bf16 clamp magnitudes (low half: column 2j, high: 2j+1)
  float div_lo;     // scale operands 2^(S - 127) of the two columns
  float div_hi;
  uint32_t nanff;   // 0x00FF in each half whose column holds a NaN/Inf
  uint32_t sbytes;  // stored scale bytes in each half (0xFF for NaN/Inf)
};

__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(
      __builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b)));
}
__device__ __forceinline__ uint32_t pk_shr_u16(uint32_t a, int n) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, a) >> (unsigned short)n);
}
__device__ __forceinline__ uint32_t pk_shl_u16(uint32_t a, int n) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, a) << (unsigned short)n);
}

// Column parameters from the packed magnitude keys of two columns; the same
// rule as row_scale_key, two columns per operation.
__device__ __forceinline__ ColPair col_pair(uint32_t keys) {
  const uint32_t e = pk_shr_u16(pk_min_u16(keys, 0x7F7F7F7Fu), 7);
  const uint32_t s = pk_sub_sat_u16(e, 0x00080008u);
  ColPair c;
  c.lim = pk_shl_u16(pk_max_u16(e, 0x00080008u), 7) | 0x00600060u;
  c.div_lo = __builtin_bit_cast(float, s << 23);
  c.div_hi = __builtin_bit_cast(float, (s >> 16) << 23);
  // a half is NaN/Inf iff its key exceeds 0x7F7F; such a column is clamped
  // to magnitude 0, leaving each element's sign for the final sign | 0x7F
  c.nanff = pk_min_u16(pk_shl_u16(pk_sub_sat_u16(keys, 0x7F7F7F7Fu), 8), 0x00FF00FFu);
  c.lim &= ~(c.nanff | (c.nanff << 8));
  c.sbytes = pk_max_u16(s, c.nanff);
  return c;
}


// e4m3 bytes of rows r (wr) and r+1 (wr1) for the four columns of pair-dwords
// j and j+1: returns {row r dword, row r+1 dword}.
__device__ __forceinline__ u32x2 encode_col_quad(uint32_t wr_a, uint32_t wr1_a,
                                                 uint32_t wr_b, uint32_t wr1_b,
                                                 const ColPair& pa, const ColPair& pb) {
  const uint32_t ca = clamp_mag(wr_a, pa.lim), ca1 = clamp_mag(wr1_a, pa.lim);
  const uint32_t cb = clamp_mag(wr_b, pb.lim), cb1 = clamp_mag(wr1_b, pb.lim);
  // column 2j: rows r, r+1 (low halves); column 2j+1: high halves
  const uint32_t pa0 = __builtin_amdgcn_perm(ca1, ca, 0x05040100u);
  const uint32_t pb0 = __builtin_amdgcn_perm(cb1, cb, 0x05040100u);
  v2i16 da = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(v2i16, pa0), __builtin_bit_cast(v2bf16, pa0), pa.div_lo, false);
  da = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      da, __builtin_bit_cast(v2bf16, __builtin_amdgcn_perm(ca1, ca, 0x07060302u)), pa.div_hi, true);
  v2i16 db = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(v2i16, pb0), __builtin_bit_cast(v2bf16, pb0), pb.div_lo, false);
  db = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      db, __builtin_bit_cast(v2bf16, __builtin_amdgcn_perm(cb1, cb, 0x07060302u)), pb.div_hi, true);
  // da bytes: (r,c0) (r+1,c0) (r,c1) (r+1,c1); db likewise for c2, c3
  const uint32_t ua = __builtin_bit_cast(uint32_t, da), ub = __builtin_bit_cast(uint32_t, db);
  return u32x2{__builtin_amdgcn_perm(ub, ua, 0x06040200u), __builtin_amdgcn_perm(ub, ua, 0x07050301u)};
}

// e4m3 bytes of rows r (wr) and r+1 (wr1) of the two columns of pair-dword j,
// in column order: (r, 2j), (r+1, 2j), (r, 2j+1), (r+1, 2j+1).
__device__ __forceinline__ uint32_t encode_col_pair(uint32_t wr, uint32_t wr1, const ColPair& pc) {
  const uint32_t c0 = clamp_mag(wr, pc.lim), c1 = clamp_mag(wr1, pc.lim);
  const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x05040100u);
  v2i16 d = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      __builtin_bit_cast(v2i16, lo), __builtin_bit_cast(v2bf16, lo), pc.div_lo, false);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
      d, __builtin_bit_cast(v2bf16, __builtin_amdgcn_perm(c1, c0, 0x07060302u)), pc.div_hi, true);
  return __builtin_bit_cast(uint32_t, d);
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
//
// Every tensor the kernels stream is touched once, so loads and stores carry
// the nontemporal hint (global_load/store ... nt): the lines are not kept in
// the caches for reuse that never comes.  Data that is reused (gamma) goes
// through load16_cached.

// Every tensor the kernels touch lives in global memory; the casts say so,
// so that loads and stores are global_* instructions even where the
// compiler cannot trace a pointer back to the kernel arguments (flat_*
// instructions would otherwise be emitted).
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gload_ptr(const void* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gstore_ptr(void* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return __builtin_nontemporal_load(gload_ptr<u32x4>(p));
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return __builtin_nontemporal_load(gload_ptr<u32x2>(p));
}
__device__ __forceinline__ u32x4 load16_cached(const void* p) {
  return *gload_ptr<u32x4>(p);
}
__device__ __forceinline__ void store8(void* p, u32x2 v) {
  __builtin_nontemporal_store(v, gstore_ptr<u32x2>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, gstore_ptr<u32x4>(p));
}
__device__ __forceinline__ uint32_t load4(const void* p) {
  return __builtin_nontemporal_load(gload_ptr<uint32_t>(p));
}
__device__ __forceinline__ void store4(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, gstore_ptr<uint32_t>(p));
}
// Small reads that neighbouring lanes or workgroups share (scale bytes and
// words), and a scale word written back through the L2.
__device__ __forceinline__ uint32_t load4_cached(const void* p) { return *gload_ptr<uint32_t>(p); }
__device__ __forceinline__ uint32_t load1_cached(const void* p) { return *gload_ptr<uint8_t>(p); }
__device__ __forceinline__ void store4_cached(void* p, uint32_t v) { *gstore_ptr<uint32_t>(p) = v; }
// One scale byte, streamed (nt) or written back through the L2.  A tile owns
// only a few bytes of each rowwise scale line, so those lines are completed
// by several workgroups.  Written back, the pieces can merge before they reach
// HBM, but dirty lines still in the L2 when the kernel ends are written back
// at its end.  The quantize kernel streams them only when its whole grid is
// resident at once, when no later work would hide that write-back.
// (A template parameter: a run-time choice between the two stores is merged
// by the compiler into one plain store.)
template <bool NT>
__device__ __forceinline__ void store_scale(void* p, uint32_t v) {
  if constexpr (NT)
    __builtin_nontemporal_store((uint8_t)v, gstore_ptr<uint8_t>(p));
  else
    *gstore_ptr<uint8_t>(p) = (uint8_t)v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace mx
