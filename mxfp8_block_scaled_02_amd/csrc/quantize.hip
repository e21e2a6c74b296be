// bf16 -> MXFP8 quantize: rowwise and/or columnwise planes from one read.
//
// Planes (Megatron-Core quantized_dbuffer page, Functions and API; Mojo
// DistributedAllGatherRMSNormQuantMXFP8 page, "Args", outputs_scale):
//   rowwise    q_row [rows, cols], s_row [rows, cols/32], blocks along a row;
//   columnwise q_col [rows, cols], s_col [rows/32, cols], blocks down a column
//              (one scale row per 32-row block, quantized_dbuffer page,
//              _block_atomic_to_flat); q_col keeps x's layout, so the
//              "columnwise" direction is only the direction of the reduction.
//
// Two workgroup-task shapes (4 waves, 256 lanes), both HBM-streaming with
// 16-byte loads per lane:
//   flat  (rowwise only): the tensor is a flat array whose 32-element blocks
//         are contiguous and whose scale array is in block order, so a
//         workgroup walks 256 x kFlatUnroll consecutive 16-byte chunks; a lane
//         quad holds one block and reduces its amax with two DPP steps.
//   tile  (any columnwise request): a workgroup owns a 32 x 512 tile, each
//         wave 8 of its rows, each lane 8 rows x 8 columns in registers.
//         Rowwise blocks are lane quads of one row.  A columnwise block is one
//         lane column across the 4 waves: each wave reduces its 8 rows in
//         registers and the 4 partial maxima meet in 4 KiB of LDS.  The tile
//         is read from HBM once for both planes.
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

__device__ void quant_flat_task(const QuantDesc& d, int64_t task, int tid) {
  const int64_t nchunks = d.rows * d.cols / kChunk;
  const int64_t base = task * (int64_t)(kThreads * kFlatUnroll) + tid;
  u32x4 v[kFlatUnroll];
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    int64_t c = base + u * kThreads;
    v[u] = c < nchunks ? load16(d.x + c * kChunk) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    int64_t c = base + u * kThreads;
    uint32_t s = scale_byte(quad_max(chunk_key(v[u])));
    u32x2 q = encode_chunk_row(v[u], row_scale(s));
    if (c < nchunks) {
      store8(d.q_row + c * kChunk, q);
      if ((tid & 3) == 0) d.s_row[c >> 2] = (uint8_t)s;
    }
  }
}

__device__ void quant_tile_task(const QuantDesc& d, int64_t task, int wave, int lane,
                                u32x4* colmax) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kTileCols - 1) / kTileCols;
  const int64_t rb = task / col_tiles;                       // 32-row block index
  const int64_t r0 = rb * kTileRows + wave * kRowsPerWave;    // this wave's first row
  const int64_t c = (task % col_tiles) * kTileCols + (int64_t)lane * kChunk;
  const bool active = c < cols;
  const uint16_t* xp = d.x + r0 * cols + c;

  u32x4 v[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
    v[r] = active ? load16(xp + r * cols) : u32x4{0, 0, 0, 0};

  if (d.q_row) {
    const int64_t sb_per_row = cols / kBlock;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      uint32_t s = scale_byte(quad_max(chunk_key(v[r])));
      u32x2 q = encode_chunk_row(v[r], row_scale(s));
      if (active) {
        store8(d.q_row + (r0 + r) * cols + c, q);
        if ((lane & 3) == 0) d.s_row[(r0 + r) * sb_per_row + (c >> 5)] = (uint8_t)s;
      }
    }
  }

  if (d.q_col) {
    // packed column maxima: word k holds columns 2k (low half) and 2k+1 (high half)
    u32x4 m = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      m.x = pk_max_u16(m.x, mag2(v[r].x));
      m.y = pk_max_u16(m.y, mag2(v[r].y));
      m.z = pk_max_u16(m.z, mag2(v[r].z));
      m.w = pk_max_u16(m.w, mag2(v[r].w));
    }
    colmax[wave * kWave + lane] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      if (w == wave) continue;
      const u32x4 o = colmax[w * kWave + lane];
      m.x = pk_max_u16(m.x, o.x);
      m.y = pk_max_u16(m.y, o.y);
      m.z = pk_max_u16(m.z, o.z);
      m.w = pk_max_u16(m.w, o.w);
    }
    const uint32_t keys[8] = {m.x & 0xFFFFu, m.x >> 16, m.y & 0xFFFFu, m.y >> 16,
                              m.z & 0xFFFFu, m.z >> 16, m.w & 0xFFFFu, m.w >> 16};
    uint32_t sb[8];
    float mul[8];
    bool any_nan = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sb[k] = scale_byte(keys[k]);
      mul[k] = col_mul(sb[k]);
      any_nan |= sb[k] == 0xFFu;
    }
    u32x2 nan8;
    nan8.x = (sb[0] == 0xFFu ? 0x7Fu : 0u) | (sb[1] == 0xFFu ? 0x7F00u : 0u) |
             (sb[2] == 0xFFu ? 0x7F0000u : 0u) | (sb[3] == 0xFFu ? 0x7F000000u : 0u);
    nan8.y = (sb[4] == 0xFFu ? 0x7Fu : 0u) | (sb[5] == 0xFFu ? 0x7F00u : 0u) |
             (sb[6] == 0xFFu ? 0x7F0000u : 0u) | (sb[7] == 0xFFu ? 0x7F000000u : 0u);
    if (active && wave == 0) {
      u32x2 packed;
      packed.x = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
      packed.y = sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24);
      store8(d.s_col + rb * cols + c, packed);
    }
    if (any_nan) {
      // a NaN/Inf column keeps only each element's sign bit
      u32x4 keep;
      keep.x = (sb[0] == 0xFFu ? 0x8000u : 0xFFFFu) | (sb[1] == 0xFFu ? 0x80000000u : 0xFFFF0000u);
      keep.y = (sb[2] == 0xFFu ? 0x8000u : 0xFFFFu) | (sb[3] == 0xFFu ? 0x80000000u : 0xFFFF0000u);
      keep.z = (sb[4] == 0xFFu ? 0x8000u : 0xFFFFu) | (sb[5] == 0xFFu ? 0x80000000u : 0xFFFF0000u);
      keep.w = (sb[6] == 0xFFu ? 0x8000u : 0xFFFFu) | (sb[7] == 0xFFu ? 0x80000000u : 0xFFFF0000u);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) v[r] &= keep;
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      u32x2 q = encode_chunk_cols(v[r], mul, nan8);
      if (active) store8(d.q_col + (r0 + r) * cols + c, q);
    }
  }
}

__global__ __launch_bounds__(kThreads) void mxfp8_quantize_kernel(const QuantArgs a) {
  __shared__ u32x4 colmax[kThreads];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int i = find_desc(a.task_start, a.n, task);
  const QuantDesc& d = a.d[i];
  const int64_t local = task - a.task_start[i];
  if (d.q_col)
    quant_tile_task(d, local, wave, lane, colmax);
  else
    quant_flat_task(d, local, tid);
}

}  // namespace

int64_t quant_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (d.q_col)
    return (d.rows / kTileRows) * ((d.cols + kTileCols - 1) / kTileCols);
  const int64_t chunks = d.rows * d.cols / kChunk;
  const int64_t per = (int64_t)kThreads * kFlatUnroll;
  return (chunks + per - 1) / per;
}

hipError_t launch_quantize(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((uint32_t)total_tasks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mx
