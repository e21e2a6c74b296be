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
// workgroup) or to all four waves of a workgroup (longer rows); a launch of
// few rows (decode) gives each row a workgroup of 16 waves instead, so each
// lane's serial work is a quarter as long.  Its L lanes
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

// Normalize one chunk with its float32 weights w (gamma + offset), store
// normed, quantize the stored words.
__device__ __forceinline__ void finish_chunk(const NormDesc& d, int64_t s_pitch, int64_t row,
                                             int64_t c, bool valid, const u32x4& v, const float* w,
                                             float rstd, int t) {
  u32x4 y;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    y[k] = pack_bf16x2(bf16_lo(v[k]) * rstd * w[2 * k], bf16_hi(v[k]) * rstd * w[2 * k + 1]);
  const RowScale rs = row_scale_key(quad_max(chunk_key(y)));
  const u32x2 q = encode_chunk_row(y, rs);
  if (valid) {
    const int64_t e = row * (int64_t)d.cols + c * kChunk;
    store16(d.normed + e, y);
    store8(d.q + e, q);
    if ((t & 3) == 0) d.s[row * s_pitch + ((c * kChunk) >> 5)] = (uint8_t)rs.sbyte;
  }
}

__device__ __forceinline__ void load_weights(const NormDesc& d, int64_t c, bool valid, float* w) {
  const u32x4 g = valid ? load16_cached(d.gamma + c * kChunk) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[2 * k] = bf16_lo(g[k]) + d.weight_offset;
    w[2 * k + 1] = bf16_hi(g[k]) + d.weight_offset;
  }
}

// Sum of a row's partial sums: wave butterfly, then (WPR > 1) the WPR wave
// totals in wave order through LDS.  part holds two slots, alternated by row,
// so one barrier per row keeps writers of row k+1 off the values of row k.
template <int WPR>
__device__ __forceinline__ float row_sum(float acc, int sub, int lane, float* part, int slot) {
  float w = wave_sum(acc);
  if constexpr (WPR == 1) {
    return w;
  } else {
    float* p = part + slot * WPR;
    if (lane == 0) p[sub] = w;
    __syncthreads();
    float total = p[0];
#pragma unroll
    for (int k = 1; k < WPR; ++k) total += p[k];
    return total;
  }
}

// Rows first_row, first_row + step, ... (count of them) of one tensor; the
// row's L = 64 * WPR lanes each hold NCH chunks (chunk j of lane t is chunk
// t + L j).  The weights gamma + offset stay in registers across the rows.
template <int WPR, int NCH>
__device__ void norm_rows(const NormDesc& d, int64_t s_pitch, int64_t first_row, int step, int count,
                          int sub, int lane, float* part) {
  constexpr int L = kWave * WPR;           // lanes per row
  const int t = sub * kWave + lane;        // this lane's index within the row
  const int64_t nch = d.cols / kChunk;
  const float inv_cols = 1.0f / (float)d.cols;
  if constexpr (NCH > 0) {
    float w[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int64_t c = t + (int64_t)j * L;
      load_weights(d, c, c < nch, w[j]);
    }
    for (int k = 0; k < count; ++k) {
      const int64_t row = first_row + (int64_t)k * step;
      const uint16_t* xr = d.x + row * (int64_t)d.cols;
      u32x4 v[NCH];
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int64_t c = t + (int64_t)j * L;
        v[j] = c < nch ? load16(xr + c * kChunk) : u32x4{0, 0, 0, 0};
      }
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) acc = sumsq_chunk(v[j], acc);
      const float ss = row_sum<WPR>(acc, sub, lane, part, k & 1);
      const float rstd = 1.0f / __builtin_sqrtf(ss * inv_cols + d.eps);
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int64_t c = t + (int64_t)j * L;
        finish_chunk(d, s_pitch, row, c, c < nch, v[j], w[j], rstd, t);
      }
    }
  } else {
    // rows too long for registers: a cached first pass for the sum, then a
    // second pass over the (now cache-resident) row
    for (int k = 0; k < count; ++k) {
      const int64_t row = first_row + (int64_t)k * step;
      const uint16_t* xr = d.x + row * (int64_t)d.cols;
      float acc = 0.0f;
      for (int64_t c0 = 0; c0 < nch; c0 += L) {
        const int64_t c = c0 + t;
        const u32x4 v = c < nch ? load16_cached(xr + c * kChunk) : u32x4{0, 0, 0, 0};
        acc = sumsq_chunk(v, acc);
      }
      const float ss = row_sum<WPR>(acc, sub, lane, part, k & 1);
      const float rstd = 1.0f / __builtin_sqrtf(ss * inv_cols + d.eps);
      for (int64_t c0 = 0; c0 < nch; c0 += L) {
        const int64_t c = c0 + t;
        const bool valid = c < nch;
        const u32x4 v = valid ? load16_cached(xr + c * kChunk) : u32x4{0, 0, 0, 0};
        float w[8];
        load_weights(d, c, valid, w);
        finish_chunk(d, s_pitch, row, c, valid, v, w, rstd, t);
      }
    }
  }
}

// WAVES waves per workgroup, WPR waves per row (1, 4 or 16), NCH chunks per
// lane (0: two passes).  A task is rows_per_task consecutive rows of one
// tensor: with WPR == WAVES the whole workgroup walks them in order; with
// WPR == 1 wave w takes rows w, w + 4, ...
template <class Args, int WPR, int NCH, int WAVES = kWavesPerGroup>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_rmsnorm_quantize_kernel(const Args a,
                                                                           int rows_per_task) {
  __shared__ float part[2 * WAVES];
  constexpr int kSlots = WAVES / WPR;                   // row slots per workgroup
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int slot = wave / WPR;
  // one tensor: its descriptor is read together with the table size (the
  // empty asm keeps those loads ahead of the branch)
  NormDesc d0 = a.d[0];
  int64_t p0 = 0;
  if constexpr (Args::kPitched) {
    p0 = a.pitch(0);
    asm volatile("" : "+s"(p0));
  }
  asm volatile("" : "+s"(d0.x), "+s"(d0.gamma), "+s"(d0.normed), "+s"(d0.q), "+s"(d0.s),
               "+s"(d0.rows), "+s"(d0.cols), "+s"(d0.weight_offset), "+s"(d0.eps));
  if constexpr (!Args::kPitched) p0 = d0.cols >> 5;
  if (a.n == 1) {
    const int64_t row0 = (int64_t)task * rows_per_task;
    const int64_t left = (int64_t)d0.rows - row0;
    const int in_task = (int)(left < rows_per_task ? left : rows_per_task);
    const int count = (in_task - slot + kSlots - 1) / kSlots;
    norm_rows<WPR, NCH>(d0, p0, row0 + slot, kSlots, count, wave % WPR, lane, part);
    return;
  }
  const int i = find_desc(a.task_start, a.n, task);
  const NormDesc d = a.d[i];
  const int64_t pi = Args::kPitched ? a.pitch(i) : (int64_t)(d.cols >> 5);
  const int64_t row0 = (int64_t)(task - a.task_start[i]) * rows_per_task;
  const int64_t left = (int64_t)d.rows - row0;
  const int in_task = (int)(left < rows_per_task ? left : rows_per_task);
  const int count = (in_task - slot + kSlots - 1) / kSlots;   // rows slot, slot + kSlots, ...
  norm_rows<WPR, NCH>(d, pi, row0 + slot, kSlots, count, wave % WPR, lane, part);
}

}  // namespace

int norm_variant(int64_t cols, int64_t total_rows) {
  const int64_t chunks = cols / kChunk;
  // few rows of at least 4 waves' width: 16 waves per row (measured on the
  // 16 x 7168 decode workload: 4.0 us with 4 waves per row)
  if (total_rows <= kWideNormRows && chunks > 2 * kWave && chunks <= 32 * kWave)
    return chunks <= 16 * kWave ? 161 : 162;
  if (chunks <= kWave) return 1;           // one wave per row, 1 chunk per lane
  if (chunks <= 2 * kWave) return 2;       // one wave per row, 2 chunks per lane
  if (chunks <= 1 * kThreads) return 11;   // four waves per row, 1..8 chunks per lane
  if (chunks <= 2 * kThreads) return 12;
  if (chunks <= 4 * kThreads) return 14;
  if (chunks <= 8 * kThreads) return 18;
  return 10;                               // four waves per row, two passes
}

int norm_rows_per_task(int64_t total_rows, int variant) {
  // Two rows per row slot once the launch has rows to spare: the weights are
  // then loaded once per two rows while the grid still covers every CU many
  // times (measured on the 8192 x 8192 and 65536 x 7168 workloads: 1 and 2
  // rows per task beat 4 and 8).
  const int64_t slots = variant < 10 ? kWavesPerGroup : 1;   // row slots per workgroup
  const int64_t g = total_rows >= slots * 8192 ? 2 : 1;
  return (int)(g * slots);
}

template <class Args>
hipError_t launch_norm(const Args& a, int64_t total_tasks, int variant, int rows_per_task,
                       hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  const dim3 block(kThreads), wide(64 * 16);
  const dim3 grid((uint32_t)total_tasks);
  const int r = rows_per_task;
  switch (variant) {
    case 161: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 16, 1, 16>), grid, wide, 0, s, a, r); break;
    case 162: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 16, 2, 16>), grid, wide, 0, s, a, r); break;
    case 1: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 1, 1>), grid, block, 0, s, a, r); break;
    case 2: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 1, 2>), grid, block, 0, s, a, r); break;
    case 11: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 4, 1>), grid, block, 0, s, a, r); break;
    case 12: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 4, 2>), grid, block, 0, s, a, r); break;
    case 14: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 4, 4>), grid, block, 0, s, a, r); break;
    case 18: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 4, 8>), grid, block, 0, s, a, r); break;
    default: hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, 4, 0>), grid, block, 0, s, a, r); break;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const NormArgs& a, int64_t total_tasks, int variant,
                                   int rows_per_task, hipStream_t s) {
  return launch_norm(a, total_tasks, variant, rows_per_task, s);
}

hipError_t launch_rmsnorm_quantize(const NormArgsPitched& a, int64_t total_tasks, int variant,
                                   int rows_per_task, hipStream_t s) {
  return launch_norm(a, total_tasks, variant, rows_per_task, s);
}

}  // namespace mx
