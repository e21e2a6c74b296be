// MXFP8 dequantize: out = e4m3(q) * 2^(S - 127), float32 or bf16.
//
// Used to compare a dequantized tensor with a fresh quantize (Megatron-Core
// quantization.utils page, _verify_te_to_mcore_mxfp8_conversion).  Both
// scale layouts are read where they lie (rowwise [rows, cols/32], columnwise
// [rows/32, cols]); every float32 result is exact, bf16 results round to
// nearest even only below 2^-133.
//
// Wave tasks, 4 elements per lane per step so that every load and store
// instruction covers contiguous memory: rowwise planes are walked flat
// (64 x kDeqUnroll units, scale byte = unit / 8); columnwise planes by
// kDeqRows rows x 256 columns, each lane reading its 4 columns' scale bytes
// once.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

// Decode the 4 bytes of q with per-element scales sc[0..3] and store them at
// element e (16 bytes of float32 or 8 bytes of bf16 per lane, so each store
// instruction writes one contiguous span across the wave).
__device__ __forceinline__ void put4(void* out, bool bf16, int64_t e, uint32_t q,
                                     const float* sc) {
  float f[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = decode_e4m3((q >> (8 * k)) & 0xFFu, sc[k]);
  if (bf16) {
    const u32x2 w = {f32_to_bf16(f[0]) | (f32_to_bf16(f[1]) << 16),
                     f32_to_bf16(f[2]) | (f32_to_bf16(f[3]) << 16)};
    store8(reinterpret_cast<uint16_t*>(out) + e, w);
  } else {
    const u32x4 w = {__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                     __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3])};
    store16(reinterpret_cast<float*>(out) + e, w);
  }
}

// Rowwise planes, walked flat in 4-element units: unit u of a wave task is
// lane + 64 u, so every load and store instruction covers contiguous memory.
__device__ void deq_flat_task(const DeqDesc& d, ScaleStride ss, bool bf16, int64_t task, int lane) {
  const int64_t nunits = d.rows * d.cols / 4;
  const int64_t base = task * (int64_t)(kWave * kDeqUnroll) + lane;
  uint32_t q[kDeqUnroll], s[kDeqUnroll];
#pragma unroll
  for (int u = 0; u < kDeqUnroll; ++u) {
    const int64_t p = base + u * kWave;
    const bool ok = p < nunits;
    q[u] = ok ? load4(reinterpret_cast<const uint32_t*>(d.q) + p) : 0u;
    s[u] = ok ? load1_cached(d.s + pitched_block(p >> 3, d.cols >> 5, ss)) : 0u;   // 8 units per block
  }
#pragma unroll
  for (int u = 0; u < kDeqUnroll; ++u) {
    const int64_t p = base + u * kWave;
    if (p < nunits) {
      const float sv = e8m0_value(s[u]);
      const float sc[4] = {sv, sv, sv, sv};
      put4(d.out, bf16, p * 4, q[u], sc);
    }
  }
}

// Columnwise planes: kDeqRows rows x 256 columns per wave task; lane l owns
// columns 4l .. 4l+3 and reads their scale bytes once.
__device__ void deq_col_task(const DeqDesc& d, ScaleStride ss, bool bf16, int64_t task, int lane) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kDeqTileCols - 1) / kDeqTileCols;
  const int64_t r0 = (task / col_tiles) * kDeqRows;
  const int64_t c = (task % col_tiles) * kDeqTileCols + (int64_t)lane * 4;
  if (c >= cols) return;                              // cols % 8 == 0: whole units only
  // rows r0 .. r0 + kDeqRows - 1 lie in one 32-row block (kDeqRows divides 32)
  const uint32_t sb = load4_cached(d.s + (r0 / kBlock) * ss.row + c);
  float sc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sc[k] = e8m0_value((sb >> (8 * k)) & 0xFFu);
  uint32_t q[kDeqRows];
#pragma unroll
  for (int r = 0; r < kDeqRows; ++r)
    q[r] = load4(d.q + (r0 + r) * cols + c);
#pragma unroll
  for (int r = 0; r < kDeqRows; ++r) put4(d.out, bf16, (r0 + r) * cols + c, q[r], sc);
}

// Columnwise planes on the narrow path (narrow_deq): kDeqRows rows x 64
// columns per wave task, one column per lane, element-sized accesses (the
// rows start off the 16-byte grid).
__device__ void deq_col_narrow_task(const DeqDesc& d, ScaleStride ss, bool bf16, int64_t task, int lane) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kWave - 1) / kWave;
  const int64_t r0 = (task / col_tiles) * kDeqRows;
  const int64_t c = (task % col_tiles) * kWave + lane;
  if (c >= cols) return;
  const float sc = e8m0_value(load1_cached(d.s + (r0 / kBlock) * ss.row + c));
#pragma unroll
  for (int r = 0; r < kDeqRows; ++r) {
    const int64_t e = (r0 + r) * cols + c;
    const float f = decode_e4m3(*gload_ptr<uint8_t>(d.q + e), sc);
    if (bf16)
      *gstore_ptr<uint16_t>(reinterpret_cast<uint16_t*>(d.out) + e) = (uint16_t)f32_to_bf16(f);
    else
      *gstore_ptr<float>(reinterpret_cast<float*>(d.out) + e) = f;
  }
}

// NARROW: some tensor of the launch takes the narrow columnwise path.
template <class Args, bool NARROW = false>
__global__ __launch_bounds__(kThreads) void mxfp8_dequantize_kernel(const Args a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t task = (int32_t)blockIdx.x * kWavesPerGroup + wave;
  // one tensor: its descriptor and task count are read together with the
  // table size (the empty asm keeps those loads ahead of the branch)
  DeqDesc d0 = a.d[0];
  int32_t total0 = a.task_start[1];
  ScaleStride p0 = {0, 0};
  if constexpr (Args::kPitched) {
    p0 = a.pitch(0);
    asm volatile("" : "+s"(p0.row), "+s"(p0.grp));
  }
  asm volatile("" : "+s"(d0.q), "+s"(d0.s), "+s"(d0.out), "+s"(d0.rows), "+s"(d0.cols), "+s"(d0.axis),
               "+s"(total0));
  if constexpr (!Args::kPitched) p0 = {d0.axis ? d0.cols : d0.cols >> 5, 16};
  if (a.n == 1) {
    if (task >= total0) return;
    if (d0.axis == 0)
      deq_flat_task(d0, p0, a.out_bf16 != 0, task, lane);
    else if (NARROW && narrow_deq(d0))
      deq_col_narrow_task(d0, p0, a.out_bf16 != 0, task, lane);
    else
      deq_col_task(d0, p0, a.out_bf16 != 0, task, lane);
    return;
  }
  if (task >= a.task_start[a.n]) return;
  const int i = find_desc(a.task_start, a.n, task);
  const DeqDesc d = a.d[i];
  const ScaleStride pi = Args::kPitched ? a.pitch(i) : ScaleStride{d.axis ? d.cols : d.cols >> 5, 16};
  const int64_t local = task - a.task_start[i];
  if (d.axis == 0)
    deq_flat_task(d, pi, a.out_bf16 != 0, local, lane);
  else if (NARROW && narrow_deq(d))
    deq_col_narrow_task(d, pi, a.out_bf16 != 0, local, lane);
  else
    deq_col_task(d, pi, a.out_bf16 != 0, local, lane);
}

template <class Args>
hipError_t launch_deq(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  bool narrow = false;
  for (int i = 0; i < a.n; ++i) narrow |= narrow_deq(a.d[i]);
  const dim3 grid((uint32_t)((total_tasks + kWavesPerGroup - 1) / kWavesPerGroup)), block(kThreads);
  if (narrow)
    hipLaunchKernelGGL((mxfp8_dequantize_kernel<Args, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((mxfp8_dequantize_kernel<Args>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t deq_tasks(const DeqDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (d.axis == 0) {
    const int64_t units = d.rows * d.cols / 4;
    const int64_t per = (int64_t)kWave * kDeqUnroll;
    return (units + per - 1) / per;
  }
  if (narrow_deq(d)) return (d.rows / kDeqRows) * ((d.cols + kWave - 1) / kWave);
  return (d.rows / kDeqRows) * ((d.cols + kDeqTileCols - 1) / kDeqTileCols);
}

hipError_t launch_dequantize(const DeqArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_deq(a, total_tasks, s);
}

hipError_t launch_dequantize(const DeqArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_deq(a, total_tasks, s);
}

}  // namespace mx
