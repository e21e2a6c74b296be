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
// A workgroup owns a 128 x 256 tile, read from HBM once for both planes.
// Wave w takes rows 32 w .. 32 w + 31 of the tile (one columnwise block) and
// all 256 columns; lane l holds the 8 columns 8 (l % 32) .. of rows
// 16 (l / 32) .. 16 (l / 32) + 15 of the wave's block, one 16-byte load per
// row (each load instruction reads 2 rows x 512 contiguous bytes).
//   rowwise    a block is a lane quad (DPP), as in the other tile kernels;
//   columnwise a block is the lane pair l, l ^ 32: each lane reduces its 16
//              rows in registers, then one lane exchange.
// The encoded column bytes go through a 32 KiB transposed tile in LDS
// (column-major, 128 bytes per column; each lane writes its 16 rows of a
// column as one 16-byte chunk), so that each lane then stores 16 bytes of
// one output row and each store instruction writes 8 whole 128-byte lines of
// q_col.  The scale bytes meet in LDS as well and leave as one 4-byte store
// per column (its 4 row blocks) and one 8-byte store per row (its 8 column
// blocks).
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kTRowsPerWave = kTRows / kWavesPerGroup;   // one 32-row column block
constexpr int kTLaneCols = 8;                             // columns a lane holds
constexpr int kTLaneRows = 16;                            // rows a lane holds
constexpr int kTColLanes = kTCols / kTLaneCols;           // lanes across the tile's columns
static_assert(kTColLanes == 32 && kTRowsPerWave == 2 * kTLaneRows && kTRowsPerWave == kBlock,
              "lane grid of the transposing tile");
constexpr int kTRowBlocks = kTCols / kBlock;              // rowwise blocks per tile row (8)
constexpr int kTColBlocks = kTRows / kBlock;              // columnwise blocks per tile column (4)

// Byte offset of 16-byte chunk k (rows 16 k .. 16 k + 15) of tile column cl in
// the transposed tile: 128-byte columns whose chunks are XOR-swizzled by the
// column's lane (cl / 8), so that the lanes that write one column index at a
// time fall on 8 different chunk positions.
__device__ __forceinline__ int colt_at(int cl, int k) {
  return cl * kTRows + ((k ^ ((cl >> 3) & 7)) << 4);
}

// LDS of a workgroup: the transposed tile, then the column scale bytes
// (4 per column, one per wave) and the row scale bytes (8 per row).
struct ColtLds {
  uint8_t tile[kTCols * kTRows];
  uint32_t scol[kTCols];
  u32x2 srow[kTRows];
};

// ROW: the rowwise plane is requested too (then cols % 32 == 0).
template <bool ROW>
__device__ void quant_colt_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid,
                                int wave, ColtLds& lds) {
  const int lane = tid & (kWave - 1);
  const int64_t rows = d.rows, cols = d.cols;
  const int64_t col_tiles = (cols + kTCols - 1) / kTCols;
  const int64_t r0 = (task / col_tiles) * kTRows, c0 = (task % col_tiles) * kTCols;
  const int cc = lane & (kTColLanes - 1), rg = lane / kTColLanes;
  const int ro = kTRowsPerWave * wave + kTLaneRows * rg;   // the lane's first row in the tile
  // No load or store before the tile's final stores sits behind a branch
  // (the compiler cannot know whether a store inside an `if` was issued, as
  // stores count in vmcnt, so it would wait on more loads and hold more
  // registers).  Lanes outside the tensor work on a mirror instead:
  //   rows % 32 == 0, so a wave's block lies wholly inside the tensor or
  //   wholly past its end (in the last tile of a tensor whose rows are not a
  //   multiple of 128); a wave past the end takes the tensor's last block;
  //   cols % 8 == 0, so a lane's chunk lies wholly inside or past the end; a
  //   lane past the end takes columns (l % 4) * 8 of its rows.  With the
  //   rowwise plane (cols % 32 == 0) its quad then covers columns 0..31 of
  //   those rows exactly and rewrites the very bytes their owners write;
  //   without it, its rows hold at least 8 columns.
  // A mirror's columnwise results land in LDS rows or columns past the
  // tensor, which the final stores skip.
  const int64_t c = c0 + kTLaneCols * cc;
  const int64_t ce = c < cols ? c : (ROW ? (int64_t)(lane & 3) * kTLaneCols : 0);
  const int64_t rbase = r0 + ro < rows ? r0 + ro : rows - kTRowsPerWave + kTLaneRows * rg;
  const uint16_t* xp = d.x + rbase * cols + ce;
  u32x4 v[kTLaneRows];
#pragma unroll
  for (int r = 0; r < kTLaneRows; ++r) v[r] = load16(xp + r * cols);

  if constexpr (ROW) {
    uint8_t* srow8 = reinterpret_cast<uint8_t*>(lds.srow);
#pragma unroll
    for (int r = 0; r < kTLaneRows; ++r) {
      const RowScale rs = row_scale_key(quad_max(chunk_key(v[r])));
      store8(d.q_row + (rbase + r) * cols + ce, encode_chunk_row(v[r], rs));
      if ((cc & 3) == 0) srow8[(ro + r) * kTRowBlocks + (cc >> 2)] = (uint8_t)rs.sbyte;
    }
  }

  // column maxima: the lane's 16 rows, then the other lane of the block
  u32x4 m = kZero4;
#pragma unroll
  for (int r = 0; r < kTLaneRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = pk_max_u16(m[j], mag2(v[r][j]));
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = pk_max_u16(m[j], (uint32_t)__shfl_xor((int)m[j], kTColLanes));

  {
    uint8_t* scol8 = reinterpret_cast<uint8_t*>(lds.scol);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const ColPair cp = col_pair(m[j]);
      // a NaN/Inf column's bytes become sign | 0x7F (its clamp gave +-0)
      const uint32_t nm = (cp.nanff | (cp.nanff << 8)) & 0x7F7F7F7Fu;
      uint32_t da[kTLaneRows / 2];
#pragma unroll
      for (int p = 0; p < kTLaneRows / 2; ++p) da[p] = encode_col_pair(v[2 * p][j], v[2 * p + 1][j], cp) | nm;
      // 16 rows of column 2j (low bytes of each row pair) and of column 2j + 1
      u32x4 lo, hi;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        lo[h] = __builtin_amdgcn_perm(da[2 * h + 1], da[2 * h], 0x05040100u);
        hi[h] = __builtin_amdgcn_perm(da[2 * h + 1], da[2 * h], 0x07060302u);
      }
      const int cl = kTLaneCols * cc + 2 * j;
      *reinterpret_cast<u32x4*>(lds.tile + colt_at(cl, ro >> 4)) = lo;
      *reinterpret_cast<u32x4*>(lds.tile + colt_at(cl + 1, ro >> 4)) = hi;
      if (rg == 0) {
        scol8[cl * kTColBlocks + wave] = (uint8_t)cp.sbytes;
        scol8[(cl + 1) * kTColBlocks + wave] = (uint8_t)(cp.sbytes >> 16);
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
      store16(d.q_col + (c0 + cl) * rows + r0 + 16 * k, *reinterpret_cast<const u32x4*>(lds.tile + colt_at(cl, k)));
  }
  // column scales: thread t takes tile column t
  static_assert(kThreads == kTCols, "one thread per tile column");
  if (c0 + tid < cols) {
    const uint32_t w = lds.scol[tid];
    uint8_t* sp = d.s_col + (c0 + tid) * (rows / kBlock) + r0 / kBlock;
    if (rows % kTRows == 0) {
      store4_cached(sp, w);                     // 4-byte aligned: rows / 32 % 4 == 0
    } else {
      for (int b = 0; b < trows / kBlock; ++b) *gstore_ptr<uint8_t>(sp + b) = (uint8_t)(w >> (8 * b));
    }
  }
  // row scales: thread t < 128 takes tile row t
  if constexpr (ROW) {
    if (tid < trows) {
      const int64_t row = r0 + tid, b0 = c0 / kBlock;
      const u32x2 w = lds.srow[tid];
      // 8 blocks in a row of the plane (8-byte aligned: b0 % 8 == 0, and in
      // the MFMA order b0 % 16 is 0 or 8) when the tile is whole
      if (pitch.s_row % 8 == 0 && c0 + kTCols <= cols) {
        *gstore_ptr<u32x2>(d.s_row + scale_at(row, b0, pitch.s_row, pitch.s_grp)) = w;
      } else {
        for (int b = 0; b < kTRowBlocks && (b0 + b) * kBlock < cols; ++b)
          *gstore_ptr<uint8_t>(d.s_row + scale_at(row, b0 + b, pitch.s_row, pitch.s_grp)) =
              (uint8_t)((b < 4 ? w.x : w.y) >> (8 * (b & 3)));
      }
    }
  }
}

template <class Args>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_colt_kernel(const Args a) {
  __shared__ __attribute__((aligned(16))) ColtLds lds;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int i = a.n == 1 ? 0 : find_desc(a.task_start, a.n, task);
  const QuantDesc d = a.d[i];
  const QuantPitch p = a.pitch(i);
  const int64_t local = task - a.task_start[i];
  if (d.q_row != nullptr)
    quant_colt_task<true>(d, p, local, tid, wave, lds);
  else
    quant_colt_task<false>(d, p, local, tid, wave, lds);
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
