// MXFP8 dequantize: out = e4m3(q) * 2^(S - 127), float32 or bf16.
//
// Used to compare a dequantized tensor with a fresh quantize (Megatron-Core
// quantization.utils page, _verify_te_to_mcore_mxfp8_conversion).  Both
// scale layouts are read where they lie (rowwise [rows, cols/32], columnwise
// [rows/32, cols]); every float32 result is exact, bf16 results round to
// nearest even only below 2^-133.
//
// Wave tasks: rowwise planes are walked flat (64 x kFlatUnroll chunks of 8
// bytes, scale byte = chunk / 4); columnwise planes by kDeqRows rows x 512
// columns, each lane reading its 8 columns' scale bytes once.
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

// Decode 8 bytes with per-element scales sc[0..7] and store them at element e.
__device__ __forceinline__ void put8(void* out, bool bf16, int64_t e, u32x2 q,
                                     const float* sc) {
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[k] = decode_e4m3((q.x >> (8 * k)) & 0xFFu, sc[k]);
    f[k + 4] = decode_e4m3((q.y >> (8 * k)) & 0xFFu, sc[k + 4]);
  }
  if (bf16) {
    u32x4 w;
    w.x = f32_to_bf16(f[0]) | (f32_to_bf16(f[1]) << 16);
    w.y = f32_to_bf16(f[2]) | (f32_to_bf16(f[3]) << 16);
    w.z = f32_to_bf16(f[4]) | (f32_to_bf16(f[5]) << 16);
    w.w = f32_to_bf16(f[6]) | (f32_to_bf16(f[7]) << 16);
    store16(reinterpret_cast<uint16_t*>(out) + e, w);
  } else {
    u32x4 a, b;
    a.x = __builtin_bit_cast(uint32_t, f[0]); a.y = __builtin_bit_cast(uint32_t, f[1]);
    a.z = __builtin_bit_cast(uint32_t, f[2]); a.w = __builtin_bit_cast(uint32_t, f[3]);
    b.x = __builtin_bit_cast(uint32_t, f[4]); b.y = __builtin_bit_cast(uint32_t, f[5]);
    b.z = __builtin_bit_cast(uint32_t, f[6]); b.w = __builtin_bit_cast(uint32_t, f[7]);
    float* o = reinterpret_cast<float*>(out) + e;
    store16(o, a);
    store16(o + 4, b);
  }
}

__device__ void deq_flat_task(const DeqDesc& d, bool bf16, int64_t task, int lane) {
  const int64_t nchunks = d.rows * d.cols / kChunk;
  const int64_t base = task * (int64_t)(kWave * kFlatUnroll) + lane;
  u32x2 q[kFlatUnroll];
  uint32_t s[kFlatUnroll];
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    int64_t c = base + u * kWave;
    bool ok = c < nchunks;
    q[u] = ok ? load8(d.q + c * kChunk) : u32x2{0, 0};
    s[u] = ok ? d.s[c >> 2] : 0u;
  }
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    int64_t c = base + u * kWave;
    if (c < nchunks) {
      float sv = e8m0_value(s[u]);
      const float sc[8] = {sv, sv, sv, sv, sv, sv, sv, sv};
      put8(d.out, bf16, c * kChunk, q[u], sc);
    }
  }
}

__device__ void deq_col_task(const DeqDesc& d, bool bf16, int64_t task, int lane) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kTileCols - 1) / kTileCols;
  const int64_t r0 = (task / col_tiles) * kDeqRows;
  const int64_t c = (task % col_tiles) * kTileCols + (int64_t)lane * kChunk;
  if (c >= cols) return;
  // rows r0 .. r0 + kDeqRows - 1 lie in one 32-row block (kDeqRows divides 32)
  u32x2 sb = load8(d.s + (r0 / kBlock) * cols + c);
  float sc[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    sc[k] = e8m0_value((sb.x >> (8 * k)) & 0xFFu);
    sc[k + 4] = e8m0_value((sb.y >> (8 * k)) & 0xFFu);
  }
#pragma unroll
  for (int r = 0; r < kDeqRows; ++r) {
    const int64_t e = (r0 + r) * cols + c;
    put8(d.out, bf16, e, load8(d.q + e), sc);
  }
}

__global__ __launch_bounds__(kThreads) void mxfp8_dequantize_kernel(const DeqArgs a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t task = (int32_t)blockIdx.x * kWavesPerGroup + wave;
  if (task >= a.task_start[a.n]) return;
  const int i = find_desc(a.task_start, a.n, task);
  const DeqDesc& d = a.d[i];
  const int64_t local = task - a.task_start[i];
  if (d.axis == 0)
    deq_flat_task(d, a.out_bf16 != 0, local, lane);
  else
    deq_col_task(d, a.out_bf16 != 0, local, lane);
}

}  // namespace

int64_t deq_tasks(const DeqDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (d.axis == 0) {
    const int64_t chunks = d.rows * d.cols / kChunk;
    const int64_t per = (int64_t)kWave * kFlatUnroll;
    return (chunks + per - 1) / per;
  }
  return (d.rows / kDeqRows) * ((d.cols + kTileCols - 1) / kTileCols);
}

hipError_t launch_dequantize(const DeqArgs& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  const int64_t groups = (total_tasks + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL(mxfp8_dequantize_kernel, dim3((uint32_t)groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mx
