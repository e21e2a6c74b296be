// Fused RMSNorm + rowwise MXFP8 quantize.
//
// The fused op of the Mojo DistributedAllGatherRMSNormQuantMXFP8 page
// (execute; "Args": gammas, float32 epsilons, weight_offsets, outputs_normed,
// outputs_quant, outputs_scale [rows, cols/32]) on one GPU's rows:
//   normed = bf16( x / sqrt(mean(x^2) + eps) * (gamma + weight_offset) )
// computed in float32 and rounded once (v_cvt_pk_bf16_f32); the quantize then
// reads the very bf16 words that are stored as normed, so its bytes equal a
// standalone rowwise quantize of normed (the page's execute: the quantize
// rides the epilogue on the same bf16 that lands in outputs_normed).
//
// A row belongs to one wave (rows up to 1024 elements, four rows per
// workgroup) or to all four waves of a workgroup (longer rows).  Its L lanes
// hold NCH 16-byte chunks each in registers: chunk j of lane t is chunk
// t + L j of the row, so every load instruction reads L * 16 contiguous
// bytes.  The sum of squares is a per-lane float32 chain, a fixed butterfly
// over each wave, and a fixed-order sum of the wave totals through LDS, so
// results do not depend on timing.  Rows too long for registers take two
// passes: the sum, then a second read that normalizes and quantizes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

__device__ __forceinline__ int find_desc(const int32_t* start, int n, int32_t task) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= task) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float sumsq_chunk(const u32x4& v, float acc) {
  acc = __builtin_fmaf(bf16_lo(v.x), bf16_lo(v.x), acc);
  acc = __builtin_fmaf(bf16_hi(v.x), bf16_hi(v.x), acc);
  acc = __builtin_fmaf(bf16_lo(v.y), bf16_lo(v.y), acc);
  acc = __builtin_fmaf(bf16_hi(v.y), bf16_hi(v.y), acc);
  acc = __builtin_fmaf(bf16_lo(v.z), bf16_lo(v.z), acc);
  acc = __builtin_fmaf(bf16_hi(v.z), bf16_hi(v.z), acc);
  acc = __builtin_fmaf(bf16_lo(v.w), bf16_lo(v.w), acc);
  acc = __builtin_fmaf(bf16_hi(v.w), bf16_hi(v.w), acc);
  return acc;
}

// Butterfly sum over the 64 lanes; every lane ends with the same value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ uint32_t norm_pair(uint32_t xw, uint32_t gw, float rstd, float off) {
  float lo = bf16_lo(xw) * rstd * (bf16_lo(gw) + off);
  float hi = bf16_hi(xw) * rstd * (bf16_hi(gw) + off);
  return pack_bf16x2(lo, hi);
}

// Normalize one chunk, store normed, quantize the stored words.
__device__ __forceinline__ void finish_chunk(const NormDesc& d, int64_t row, int64_t c,
                                             bool valid, const u32x4& v, float rstd,
                                             int t) {
  u32x4 g = valid ? load16(d.gamma + c * kChunk) : u32x4{0, 0, 0, 0};
  u32x4 y;
  y.x = norm_pair(v.x, g.x, rstd, d.weight_offset);
  y.y = norm_pair(v.y, g.y, rstd, d.weight_offset);
  y.z = norm_pair(v.z, g.z, rstd, d.weight_offset);
  y.w = norm_pair(v.w, g.w, rstd, d.weight_offset);
  uint32_t s = scale_byte(quad_max(chunk_key(y)));
  u32x2 q = encode_chunk_row(y, row_scale(s));
  if (valid) {
    const int64_t e = row * (int64_t)d.cols + c * kChunk;
    store16(d.normed + e, y);
    store8(d.q + e, q);
    if ((t & 3) == 0) d.s[e >> 5] = (uint8_t)s;
  }
}

// Sum of a row's partial sums: wave butterfly, then (WPR > 1) the WPR wave
// totals in wave order through LDS.
template <int WPR>
__device__ __forceinline__ float row_sum(float acc, int sub, int lane, float* part) {
  float w = wave_sum(acc);
  if constexpr (WPR == 1) {
    return w;
  } else {
    if (lane == 0) part[sub] = w;
    __syncthreads();
    float total = part[0];
#pragma unroll
    for (int k = 1; k < WPR; ++k) total += part[k];
    return total;
  }
}

template <int WPR, int NCH>
__device__ void norm_row(const NormDesc& d, int64_t row, int sub, int lane, float* part) {
  constexpr int L = kWave * WPR;           // lanes per row
  const int t = sub * kWave + lane;        // this lane's index within the row
  const int64_t nch = d.cols / kChunk;
  const uint16_t* xr = d.x + row * (int64_t)d.cols;
  const float inv_cols = 1.0f / (float)d.cols;
  if constexpr (NCH > 0) {
    u32x4 v[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      int64_t c = t + (int64_t)j * L;
      v[j] = c < nch ? load16(xr + c * kChunk) : u32x4{0, 0, 0, 0};
    }
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) acc = sumsq_chunk(v[j], acc);
    const float ss = row_sum<WPR>(acc, sub, lane, part);
    const float rstd = 1.0f / __builtin_sqrtf(ss * inv_cols + d.eps);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      int64_t c = t + (int64_t)j * L;
      finish_chunk(d, row, c, c < nch, v[j], rstd, t);
    }
  } else {
    float acc = 0.0f;
    for (int64_t c0 = 0; c0 < nch; c0 += L) {
      int64_t c = c0 + t;
      u32x4 v = c < nch ? load16(xr + c * kChunk) : u32x4{0, 0, 0, 0};
      acc = sumsq_chunk(v, acc);
    }
    const float ss = row_sum<WPR>(acc, sub, lane, part);
    const float rstd = 1.0f / __builtin_sqrtf(ss * inv_cols + d.eps);
    for (int64_t c0 = 0; c0 < nch; c0 += L) {
      int64_t c = c0 + t;
      bool valid = c < nch;
      u32x4 v = valid ? load16(xr + c * kChunk) : u32x4{0, 0, 0, 0};
      finish_chunk(d, row, c, valid, v, rstd, t);
    }
  }
}

// WPR waves per row (1 or 4), NCH chunks per lane (0: two passes).
template <int WPR, int NCH>
__global__ __launch_bounds__(kThreads) void mxfp8_rmsnorm_quantize_kernel(const NormArgs a) {
  __shared__ float part[kWavesPerGroup];
  constexpr int kRowsPerGroup = kWavesPerGroup / WPR;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t task = (int32_t)blockIdx.x * kRowsPerGroup + wave / WPR;
  if (task >= a.task_start[a.n]) return;   // only when WPR == 1: no barrier follows
  const int i = find_desc(a.task_start, a.n, task);
  const NormDesc& d = a.d[i];
  const int64_t row = task - a.task_start[i];
  norm_row<WPR, NCH>(d, row, wave % WPR, lane, part);
}

}  // namespace

int norm_variant(int64_t cols) {
  const int64_t chunks = cols / kChunk;
  if (chunks <= kWave) return 1;           // one wave per row, 1 chunk per lane
  if (chunks <= 2 * kWave) return 2;       // one wave per row, 2 chunks per lane
  if (chunks <= 1 * kThreads) return 11;   // four waves per row, 1..8 chunks per lane
  if (chunks <= 2 * kThreads) return 12;
  if (chunks <= 4 * kThreads) return 14;
  if (chunks <= 8 * kThreads) return 18;
  return 10;                               // four waves per row, two passes
}

hipError_t launch_rmsnorm_quantize(const NormArgs& a, int64_t total_tasks, int variant,
                                   hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  const dim3 block(kThreads);
  const dim3 g1((uint32_t)((total_tasks + kWavesPerGroup - 1) / kWavesPerGroup));
  const dim3 g4((uint32_t)total_tasks);
  switch (variant) {
    case 1: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<1, 1>), g1, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<1, 2>), g1, block, 0, s, a); break;
    case 11: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<4, 1>), g4, block, 0, s, a); break;
    case 12: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<4, 2>), g4, block, 0, s, a); break;
    case 14: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<4, 4>), g4, block, 0, s, a); break;
    case 18: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<4, 8>), g4, block, 0, s, a); break;
    default: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<4, 0>), g4, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace mx
