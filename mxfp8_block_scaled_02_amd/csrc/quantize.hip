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
// Two workgroup-task shapes (4 waves, 256 lanes).  A lane holds kLaneCols = 8
// consecutive elements of a row (one 16-byte load, so every load instruction
// reads 1 KiB of contiguous memory), and a rowwise block is a lane quad whose
// amax takes two DPP steps.
//   flat  (rowwise only): the tensor is a flat array whose 32-element blocks
//         are contiguous and whose scale array is in block order; a workgroup
//         walks 256 x U consecutive 8-element pieces (U = flat_unroll: 1 for
//         small tensors, kFlatUnroll otherwise).
//   tile  (any columnwise request): a workgroup owns a 32 x 512 tile, each
//         wave 8 of its rows, each lane 8 rows x 8 columns in registers.  A
//         columnwise block is one lane column across the 4 waves: each wave
//         reduces its 8 rows in registers and the partial maxima meet in
//         4 KiB of LDS.  The tile is read from HBM once for both planes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kCh = kLaneCols / kChunk;     // 16-byte chunks per lane per row (1 or 2)

// Rowwise scale parameters of the block that holds this lane's kLaneCols
// elements (a lane quad for 8 columns per lane, a lane pair for 16).
__device__ __forceinline__ RowScale lane_row_scale(const u32x4* v) {
  if constexpr (kCh == 1)
    return row_scale_key(quad_max(chunk_key(v[0])));
  else
    return row_scale_key(pair_max(chunk16_key(v[0], v[1])));
}

template <bool NT, int U>
__device__ void quant_flat_pieces(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid,
                                  int64_t npieces) {
  const int64_t base = task * (int64_t)(kThreads * U) + tid;
  u32x4 v[U][kCh];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + u * kThreads;
#pragma unroll
    for (int h = 0; h < kCh; ++h)
      v[u][h] = p < npieces ? load16(d.x + p * kLaneCols + h * kChunk) : kZero4;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + u * kThreads;
    const RowScale rs = lane_row_scale(v[u]);
    if (p < npieces) {
#pragma unroll
      for (int h = 0; h < kCh; ++h)
        store8(d.q_row + p * kLaneCols + h * kChunk, encode_chunk_row(v[u][h], rs));
      if ((tid & (kBlock / kLaneCols - 1)) == 0)
        store_scale<NT>(d.s_row + pitched_block(p * kLaneCols / kBlock, d.cols >> 5, pitch.s_row), rs.sbyte);
    }
  }
}

template <bool NT>
__device__ void quant_flat_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid) {
  const int64_t npieces = d.rows * d.cols / kLaneCols;   // whole blocks: cols % 32 == 0
  if (flat_unroll(npieces) == 1)
    quant_flat_pieces<NT, 1>(d, pitch, task, tid, npieces);
  else
    quant_flat_pieces<NT, kFlatUnroll>(d, pitch, task, tid, npieces);
}

template <bool NT>
__device__ void quant_tile_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task,
                                int wave, int lane, u32x4* colmax) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kTileCols - 1) / kTileCols;
  const int64_t rb = task / col_tiles;                       // 32-row block index
  const int64_t r0 = rb * kTileRows + wave * kRowsPerWave;    // this wave's first row
  const int64_t c = (task % col_tiles) * kTileCols + (int64_t)lane * kLaneCols;
  bool ok[kCh];                                              // chunk h: columns c + 8h ..
#pragma unroll
  for (int h = 0; h < kCh; ++h) ok[h] = c + h * kChunk < cols;
  const uint16_t* xp = d.x + r0 * cols + c;

  u32x4 v[kRowsPerWave][kCh];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int h = 0; h < kCh; ++h)
      v[r][h] = ok[h] ? load16(xp + r * cols + h * kChunk) : kZero4;

  if (d.q_row) {
    // cols % 32 == 0 here, so a block's lanes are either all present or absent
    const int64_t sb_per_row = pitch.s_row;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const RowScale rs = lane_row_scale(v[r]);
      if (ok[0]) {
#pragma unroll
        for (int h = 0; h < kCh; ++h)
          store8(d.q_row + (r0 + r) * cols + c + h * kChunk, encode_chunk_row(v[r][h], rs));
        if ((lane & (kBlock / kLaneCols - 1)) == 0)
          store_scale<NT>(d.s_row + (r0 + r) * sb_per_row + (c >> 5), rs.sbyte);
      }
    }
  }

  if (d.q_col) {
    // packed column maxima: word j of chunk h holds columns c + 8h + 2j, + 1
    u32x4 m[kCh];
#pragma unroll
    for (int h = 0; h < kCh; ++h) {
      m[h] = kZero4;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[h][j] = pk_max_u16(m[h][j], mag2(v[r][h][j]));
      colmax[(wave * kWave + lane) * kCh + h] = m[h];
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      if (w == wave) continue;
#pragma unroll
      for (int h = 0; h < kCh; ++h) {
        const u32x4 o = colmax[(w * kWave + lane) * kCh + h];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[h][j] = pk_max_u16(m[h][j], o[j]);
      }
    }
    ColPair cp[kCh][4];
    u32x2 sb[kCh], nanq[kCh];
#pragma unroll
    for (int h = 0; h < kCh; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) cp[h][j] = col_pair(m[h][j]);
      // scale bytes and NaN bytes of the chunk's 8 columns, in column order
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        sb[h][k] = __builtin_amdgcn_perm(cp[h][2 * k + 1].sbytes, cp[h][2 * k].sbytes, 0x06040200u);
        nanq[h][k] = __builtin_amdgcn_perm(cp[h][2 * k + 1].nanff, cp[h][2 * k].nanff,
                                           0x06040200u) & 0x7F7F7F7Fu;
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int h = 0; h < kCh; ++h)
        if (ok[h]) store8(d.s_col + rb * pitch.s_col + c + h * kChunk, sb[h]);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r += 2) {
      uint8_t* qp = d.q_col + (r0 + r) * cols + c;
#pragma unroll
      for (int h = 0; h < kCh; ++h) {
        u32x2 q0, q1;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const u32x2 o = encode_col_quad(v[r][h][2 * k], v[r + 1][h][2 * k],
                                          v[r][h][2 * k + 1], v[r + 1][h][2 * k + 1],
                                          cp[h][2 * k], cp[h][2 * k + 1]);
          q0[k] = o.x | nanq[h][k];
          q1[k] = o.y | nanq[h][k];
        }
        if (ok[h]) {
          store8(qp + h * kChunk, q0);
          store8(qp + cols + h * kChunk, q1);
        }
      }
    }
  }
}

// NT: stream the rowwise scale bytes (see store_scale and the launcher)
template <class Args, bool NT>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_kernel(const Args a) {
  __shared__ u32x4 colmax[kThreads * kCh];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  // one tensor (the common call): its descriptor is read together with the
  // table size (the empty asm keeps those loads ahead of the branch), so the
  // first global load waits for one scalar round trip instead of two
  QuantDesc d0 = a.d[0];
  QuantPitch p0 = {0, 0};
  if constexpr (Args::kPitched) {
    p0 = a.pitch(0);
    asm volatile("" : "+s"(p0.s_row), "+s"(p0.s_col));
  }
  asm volatile("" : "+s"(d0.x), "+s"(d0.q_row), "+s"(d0.s_row), "+s"(d0.q_col), "+s"(d0.s_col),
               "+s"(d0.rows), "+s"(d0.cols));
  if constexpr (!Args::kPitched) p0 = {d0.cols >> 5, d0.cols};
  if (a.n == 1) {
    if (d0.q_col)
      quant_tile_task<NT>(d0, p0, task, wave, lane, colmax);
    else
      quant_flat_task<NT>(d0, p0, task, tid);
    return;
  }
  const int i = find_desc(a.task_start, a.n, task);
  const QuantDesc d = a.d[i];
  const QuantPitch pi = Args::kPitched ? a.pitch(i) : QuantPitch{d.cols >> 5, d.cols};
  const int64_t local = task - a.task_start[i];
  if (d.q_col)
    quant_tile_task<NT>(d, pi, local, wave, lane, colmax);
  else
    quant_flat_task<NT>(d, pi, local, tid);
}

}  // namespace

int64_t quant_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (d.q_col)
    return (d.rows / kTileRows) * ((d.cols + kTileCols - 1) / kTileCols);
  const int64_t pieces = d.rows * d.cols / kLaneCols;
  const int64_t per = (int64_t)kThreads * flat_unroll(pieces);
  return (pieces + per - 1) / per;
}

// A grid of at most this many workgroups is resident all at once (four per
// CU): its scale bytes are streamed (see store_scale).  Measured: the
// 4096 x 4096 row + column launch (1024 tiles) takes 13.3 us streamed and
// 14.0 us written back; the 64 x 2048 x 7168 grouped launch (57344 tiles)
// 0.73 ms streamed and 0.67 ms written back.
constexpr int64_t kResidentTasks = 4 * 256;

template <class Args>
hipError_t launch_quantize_args(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  if (total_tasks <= kResidentTasks)
    hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, true>), dim3((uint32_t)total_tasks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, false>), dim3((uint32_t)total_tasks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_quantize_args(a, total_tasks, s);
}

hipError_t launch_quantize(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_quantize_args(a, total_tasks, s);
}

}  // namespace mx
