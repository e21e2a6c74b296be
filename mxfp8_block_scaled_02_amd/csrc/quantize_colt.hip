// bf16 -> MXFP8 with the columnwise plane stored transposed.
//
// The columnwise plane's blocks run down the columns of x (Megatron-Core
// quantized_dbuffer page, _block_atomic_to_flat: one columnwise scale row
// per 32-row block).  Stored transposed, q_col [cols, rows] and
// s_col [cols, rows/32], each block's 32 bytes are contiguous: the plane is a
// rowwise plane of x^T, the operand order of the matrix product (see
// include/mxfp8.h, "Transposed columnwise plane").  The bytes are those of
// the untransposed plane: the same block rule and the same encode.
//
// A workgroup owns a 128 x 128 tile, read from HBM once for both planes.
// Wave w takes rows 32 w .. 32 w + 31 of the tile (one columnwise block) and
// all 128 columns; lane l holds the 8 columns 8 (l % 16) .. of rows
// 8 (l / 16) .. 8 (l / 16) + 7 of the wave's block, one 16-byte load per row
// (each load instruction reads 4 rows x 256 contiguous bytes).
//   rowwise    a block is a lane quad (DPP), as in the other tile kernels;
//   columnwise a block is the 4 lanes l, l ^ 16, l ^ 32, l ^ 48: each lane
//              reduces its 8 rows in registers, then two lane exchanges.
// The encoded column bytes go through a 16 KiB transposed tile in LDS
// (column-major, 128 bytes per column), so that each lane then stores 16
// bytes of one output row and each store instruction writes 8 whole 128-byte
// lines of q_col.  The tile's column scale bytes meet in LDS as well: 4 bytes
// per column, one 4-byte store each.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kTRowsPerWave = kTRows / kWavesPerGroup;   // one 32-row column block
constexpr int kTLaneCols = 8;                             // columns a lane holds
constexpr int kTLaneRows = 8;                             // rows a lane holds
static_assert(kTCols == 16 * kTLaneCols && kTRowsPerWave == 4 * kTLaneRows && kTRowsPerWave == kBlock,
              "lane grid of the transposing tile");

// Byte offset of 16-byte chunk k (rows 16 k .. 16 k + 15) of tile column cl in
// the transposed tile: 128-byte columns whose chunks are XOR-swizzled by the
// column's lane (cl / 8), so that the 16 lanes that write one column index
// at a time fall on 8 different chunk positions.
__device__ __forceinline__ int colt_at(int cl, int k) {
  return cl * kTRows + ((k ^ ((cl >> 3) & 7)) << 4);
}

// ROW: the rowwise plane is requested too (then cols % 32 == 0).
template <bool ROW>
__device__ void quant_colt_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid,
                                int wave, uint8_t* tl, uint32_t* ssc) {
  const int lane = tid & (kWave - 1);
  const int64_t rows = d.rows, cols = d.cols;
  const int64_t col_tiles = (cols + kTCols - 1) / kTCols;
  const int64_t r0 = (task / col_tiles) * kTRows, c0 = (task % col_tiles) * kTCols;
  const int cc = lane & 15, rg = lane >> 4;
  // rows % 32 == 0: a wave's block lies wholly inside the tensor or wholly
  // past its end (the last tile of a tensor whose rows are not a multiple of
  // 128); cols % 8 == 0: so does a lane's chunk
  const bool wave_on = r0 + kTRowsPerWave * wave < rows;
  const int64_t c = c0 + kTLaneCols * cc;
  const bool ok = wave_on && c < cols;
  const int ro = kTRowsPerWave * wave + kTLaneRows * rg;   // the lane's first row in the tile
  // Loads are never skipped (a skipped load behind a branch makes the
  // compiler wait on every load before each store): a lane outside the
  // tensor reads rows 0..7 of its first 8 columns (rows >= 32) and stores
  // nothing.  Its columns are its own, so its values reach no block of the
  // tensor; a rowwise quad lies wholly outside with it (cols % 32 == 0).
  const uint16_t* xp = d.x + (ok ? (r0 + ro) * cols + c : 0);
  u32x4 v[kTLaneRows];
#pragma unroll
  for (int r = 0; r < kTLaneRows; ++r) v[r] = load16(xp + r * cols);

  if constexpr (ROW) {
#pragma unroll
    for (int r = 0; r < kTLaneRows; ++r) {
      const RowScale rs = row_scale_key(quad_max(chunk_key(v[r])));
      const u32x2 q = encode_chunk_row(v[r], rs);
      if (ok) {
        const int64_t row = r0 + ro + r;
        store8(d.q_row + row * cols + c, q);
        if ((cc & 3) == 0)
          store_scale<false>(d.s_row + scale_at(row, c >> 5, pitch.s_row, pitch.s_grp), rs.sbyte);
      }
    }
  }

  // column maxima: the lane's 8 rows, then the other 3 lanes of the block
  u32x4 m = kZero4;
#pragma unroll
  for (int r = 0; r < kTLaneRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = pk_max_u16(m[j], mag2(v[r][j]));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = pk_max_u16(m[j], (uint32_t)__shfl_xor((int)m[j], 16));
    m[j] = pk_max_u16(m[j], (uint32_t)__shfl_xor((int)m[j], 32));
  }

  if (wave_on) {
    uint8_t* ssc8 = reinterpret_cast<uint8_t*>(ssc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const ColPair cp = col_pair(m[j]);
      // a NaN/Inf column's bytes become sign | 0x7F (its clamp gave +-0)
      const uint32_t nm = (cp.nanff | (cp.nanff << 8)) & 0x7F7F7F7Fu;
      uint32_t da[kTLaneRows / 2];
#pragma unroll
      for (int p = 0; p < kTLaneRows / 2; ++p) da[p] = encode_col_pair(v[2 * p][j], v[2 * p + 1][j], cp) | nm;
      // 8 rows of column 2j (low bytes of each row pair) and of column 2j + 1
      const u32x2 lo = {__builtin_amdgcn_perm(da[1], da[0], 0x05040100u),
                        __builtin_amdgcn_perm(da[3], da[2], 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(da[1], da[0], 0x07060302u),
                        __builtin_amdgcn_perm(da[3], da[2], 0x07060302u)};
      const int cl = kTLaneCols * cc + 2 * j;
      *reinterpret_cast<u32x2*>(tl + colt_at(cl, ro >> 4) + (ro & 15)) = lo;
      *reinterpret_cast<u32x2*>(tl + colt_at(cl + 1, ro >> 4) + (ro & 15)) = hi;
      if (rg == 0) {
        ssc8[cl * 4 + wave] = (uint8_t)cp.sbytes;
        ssc8[(cl + 1) * 4 + wave] = (uint8_t)(cp.sbytes >> 16);
      }
    }
  }
  __syncthreads();

  // each lane stores 16-byte chunks of the transposed tile: chunk k of tile
  // column cl is rows r0 + 16 k .. of output row c0 + cl
  const int64_t trows = rows - r0 < kTRows ? rows - r0 : kTRows;   // 32, 64, 96 or 128
#pragma unroll
  for (int q = 0; q < kTCols * kTRows / 16 / kThreads; ++q) {
    const int id = tid + kThreads * q, cl = id >> 3, k = id & 7;
    if (c0 + cl < cols && 16 * k < trows)
      store16(d.q_col + (c0 + cl) * rows + r0 + 16 * k, *reinterpret_cast<const u32x4*>(tl + colt_at(cl, k)));
  }
  if (tid < kTCols && c0 + tid < cols) {
    const uint32_t w = ssc[tid];
    uint8_t* sp = d.s_col + (c0 + tid) * (rows / kBlock) + r0 / kBlock;
    if (rows % kTRows == 0) {
      store4_cached(sp, w);                     // 4-byte aligned: rows / 32 % 4 == 0
    } else {
      for (int b = 0; b < trows / kBlock; ++b) *gstore_ptr<uint8_t>(sp + b) = (uint8_t)(w >> (8 * b));
    }
  }
}

template <class Args>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_colt_kernel(const Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t tl[kTCols * kTRows];
  __shared__ uint32_t ssc[kTCols];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int i = a.n == 1 ? 0 : find_desc(a.task_start, a.n, task);
  const QuantDesc d = a.d[i];
  const QuantPitch p = a.pitch(i);
  const int64_t local = task - a.task_start[i];
  if (d.q_row != nullptr)
    quant_colt_task<true>(d, p, local, tid, wave, tl, ssc);
  else
    quant_colt_task<false>(d, p, local, tid, wave, tl, ssc);
}

template <class Args>
hipError_t launch_colt(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  hipLaunchKernelGGL((mxfp8_quantize_colt_kernel<Args>), dim3((uint32_t)total_tasks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t quant_colt_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  return ((d.rows + kTRows - 1) / kTRows) * ((d.cols + kTCols - 1) / kTCols);
}

hipError_t launch_quantize_colt(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_colt(a, total_tasks, s);
}

hipError_t launch_quantize_colt(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_colt(a, total_tasks, s);
}

}  // namespace mx
