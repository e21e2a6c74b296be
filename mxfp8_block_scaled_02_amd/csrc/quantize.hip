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
        store_scale<NT>(d.s_row + pitched_block(p * kLaneCols / kBlock, d.cols >> 5,
                                                ScaleStride{pitch.s_row, pitch.s_grp}),
                        rs.sbyte);
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

// The narrow columnwise path (narrow_col): the workgroup takes 256 columns of
// one 32-row block, one column per thread.  A column's 32 values are packed
// into four 8-value chunks and scaled and encoded by the rowwise block code,
// which computes the same rule on any 32 values.  Loads and stores are
// element-sized, so every access is aligned whatever the row length; across a
// wave they cover 64 consecutive columns of one row.
template <bool NT>
__device__ void quant_col_narrow_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid) {
  const int64_t cols = d.cols;
  const int64_t col_tasks = (cols + kThreads - 1) / kThreads;
  const int64_t rb = task / col_tasks;
  const int64_t c = (task % col_tasks) * kThreads + tid;
  if (c >= cols) return;                                   // no barrier follows
  const uint16_t* xp = d.x + rb * kBlock * cols + c;
  u32x4 v[kBlock / kChunk];
#pragma unroll
  for (int j = 0; j < kBlock / kChunk; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = *gload_ptr<uint16_t>(xp + (8 * j + 2 * k) * cols);
      const uint32_t hi = *gload_ptr<uint16_t>(xp + (8 * j + 2 * k + 1) * cols);
      v[j][k] = lo | (hi << 16);
    }
  uint32_t key = 0;
#pragma unroll
  for (int j = 0; j < kBlock / kChunk; ++j) key = max(key, chunk_key(v[j]));
  const RowScale rs = row_scale_key(key);
  uint8_t* qp = d.q_col + rb * kBlock * cols + c;
#pragma unroll
  for (int j = 0; j < kBlock / kChunk; ++j) {
    const u32x2 e = encode_chunk_row(v[j], rs);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *gstore_ptr<uint8_t>(qp + (8 * j + k) * cols) = (uint8_t)((k < 4 ? e.x : e.y) >> (8 * (k & 3)));
  }
  store_scale<NT>(d.s_col + rb * pitch.s_col + c, rs.sbyte);
}

// Packed magnitude maxima of the lane's 8 columns over the wave's rows (word j
// holds columns 2j, 2j + 1), also written to the lane's LDS slot.
__device__ __forceinline__ u32x4 wave_col_max(const u32x4 (&v)[kRowsPerWave][kCh], u32x4* slot) {
  u32x4 m = kZero4;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = pk_max_u16(m[j], mag2(v[r][0][j]));
  *slot = m;
  return m;
}

// ROW: the rowwise plane is requested too (then cols % 32 == 0).
template <bool NT, bool ROW>
__device__ void quant_tile_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task,
                                int wave, int lane, u32x4* colmax) {
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kTileCols - 1) / kTileCols;
  if constexpr (ROW) {
    // The column tiles of a row block share its rowwise scale lines.
    // Workgroup ids are spread over the 8 XCDs in turn, so tiles whose ids
    // are 8 apart run on one XCD and their pieces meet in its L2.  Tile
    // (rb, ct) takes id 8 (col_tiles (rb / 8) + ct) + rb % 8, a permutation
    // whenever the row blocks are a multiple of 8.  A resident grid whose
    // column tiles are a multiple of 8 keeps the plain order, where each XCD
    // holds whole column strips: measured faster there (4096 x 4096: 13.3
    // against 13.6 us), slower everywhere else.
    if ((d.rows / kTileRows) % 8 == 0 && !(NT && col_tiles % 8 == 0)) {
      const int64_t j = task >> 3;
      task = ((j / col_tiles) * 8 + (task & 7)) * col_tiles + j % col_tiles;
    }
  }
  const int64_t rb = task / col_tiles;                       // 32-row block index
  const int64_t r0 = rb * kTileRows + wave * kRowsPerWave;    // this wave's first row
  const int64_t c = (task % col_tiles) * kTileCols + (int64_t)lane * kLaneCols;
  // Lanes past the row's end (only in a last, partial column tile) never load
  // or store behind a branch: the compiler cannot know whether a store inside
  // an `if` was issued (stores count in vmcnt), so it would wait for more
  // loads, and finally for the wave's own earlier stores, before each row.
  //   ROW (cols % 32 == 0): such a lane takes column (lane % 4) * 8 of the
  //   same rows instead.  Its lane quad then covers columns 0..31 of the
  //   tile's 32 rows exactly, so it computes the very bytes, row scales and
  //   column scales that the lanes owning those columns compute, and its
  //   stores rewrite identical bytes.
  //   !ROW (columnwise only; cols % 8 == 0): such a lane reads columns 0..7
  //   of its rows (always inside the tensor) and its stores are skipped;
  //   what it computes reaches no output, since a column's maximum is its
  //   own lane's.
  static_assert(kCh == 1, "lane mirroring assumes one chunk per lane");
  const bool ok = c < cols;
  const int64_t ce = ok ? c : (ROW ? (int64_t)(lane & 3) * kLaneCols : 0);
  const bool st = ROW || ok;
  const uint16_t* xp = d.x + r0 * cols + ce;

  u32x4 v[kRowsPerWave][kCh];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) v[r][0] = load16(xp + r * cols);

  // A resident grid (NT) runs one tile per workgroup: every wave there waits
  // for all its loads before its first store (the column maxima need them
  // all, and the empty asm keeps the stores behind them), so the chip reads
  // first and then writes.  A streaming grid stores each row as its load
  // lands, which overlaps other workgroups' loads.  Measured both ways:
  // 4096 x 4096 13.3 against 13.6 us, 8192 x 7168 42.0 against 42.6 us.
  u32x4 m = kZero4;
  if constexpr (NT) {
    m = wave_col_max(v, colmax + wave * kWave + lane);
    asm volatile("" ::"v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]));
  }

  // rowwise scale bytes of the wave's rows, stored after every data store of
  // the tile, packed four to a dword: row r in byte r % 4 of word r / 4
  uint32_t row_sb[kRowsPerWave / 4] = {};
  if constexpr (ROW) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const RowScale rs = lane_row_scale(v[r]);
      row_sb[r / 4] |= rs.sbyte << (8 * (r % 4));
      store8(d.q_row + (r0 + r) * cols + ce, encode_chunk_row(v[r][0], rs));
    }
  }

  if constexpr (!NT) m = wave_col_max(v, colmax + wave * kWave + lane);
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWavesPerGroup; ++w) {
    if (w == wave) continue;
    const u32x4 o = colmax[w * kWave + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = pk_max_u16(m[j], o[j]);
  }
  ColPair cp[4];
  u32x2 sb, nanq;
#pragma unroll
  for (int j = 0; j < 4; ++j) cp[j] = col_pair(m[j]);
  // scale bytes and NaN bytes of the chunk's 8 columns, in column order
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    sb[k] = __builtin_amdgcn_perm(cp[2 * k + 1].sbytes, cp[2 * k].sbytes, 0x06040200u);
    nanq[k] = __builtin_amdgcn_perm(cp[2 * k + 1].nanff, cp[2 * k].nanff, 0x06040200u) & 0x7F7F7F7Fu;
  }
  if (st && wave == 0) store8(d.s_col + rb * pitch.s_col + ce, sb);
#pragma unroll
  for (int r = 0; r < kRowsPerWave; r += 2) {
    uint8_t* qp = d.q_col + (r0 + r) * cols + ce;
    u32x2 q0, q1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x2 o = encode_col_quad(v[r][0][2 * k], v[r + 1][0][2 * k], v[r][0][2 * k + 1],
                                      v[r + 1][0][2 * k + 1], cp[2 * k], cp[2 * k + 1]);
      q0[k] = o.x | nanq[k];
      q1[k] = o.y | nanq[k];
    }
    if (st) {
      store8(qp, q0);
      store8(qp + cols, q1);
    }
  }

  if (ROW && (lane & (kBlock / kLaneCols - 1)) == 0) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
      store_scale<NT>(d.s_row + scale_at(r0 + r, ce >> 5, pitch.s_row, pitch.s_grp),
                      row_sb[r / 4] >> (8 * (r % 4)));
  }
}

// NT: stream the rowwise scale bytes (see store_scale and the launcher).
// ROWCOL: every tensor of the launch requests both planes (the launcher
// checks), so only that tile path is compiled in; compiled together with the
// other paths, it would share their code and registers.  NARROW: some tensor
// takes the narrow columnwise path (only such launches carry its code).
template <class Args, bool NT, bool ROWCOL, bool NARROW = false>
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
  QuantPitch p0 = {0, 0, 0};
  if constexpr (Args::kPitched) {
    p0 = a.pitch(0);
    asm volatile("" : "+s"(p0.s_row), "+s"(p0.s_col), "+s"(p0.s_grp));
  }
  asm volatile("" : "+s"(d0.x), "+s"(d0.q_row), "+s"(d0.s_row), "+s"(d0.q_col), "+s"(d0.s_col),
               "+s"(d0.rows), "+s"(d0.cols));
  if constexpr (!Args::kPitched) p0 = {d0.cols >> 5, d0.cols, 16};
  // a grouped launch replaces it with the task's own tensor
  int64_t local = task;
  if (a.n != 1) {
    const int i = find_desc(a.task_start, a.n, task);
    d0 = a.d[i];
    p0 = Args::kPitched ? a.pitch(i) : QuantPitch{d0.cols >> 5, d0.cols, 16};
    local = task - a.task_start[i];
  }
  if constexpr (ROWCOL) {
    quant_tile_task<NT, true>(d0, p0, local, wave, lane, colmax);
  } else {
    if (d0.q_col) {
      if (d0.q_row)
        quant_tile_task<NT, true>(d0, p0, local, wave, lane, colmax);
      else if (NARROW && narrow_col(d0))
        quant_col_narrow_task<NT>(d0, p0, local, tid);
      else
        quant_tile_task<NT, false>(d0, p0, local, wave, lane, colmax);
    } else {
      quant_flat_task<NT>(d0, p0, local, tid);
    }
  }
}

}  // namespace

int64_t quant_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (narrow_col(d)) return (d.rows / kBlock) * ((d.cols + kThreads - 1) / kThreads);
  if (d.q_col)
    return (d.rows / kTileRows) * ((d.cols + kTileCols - 1) / kTileCols);
  const int64_t pieces = d.rows * d.cols / kLaneCols;
  const int64_t per = (int64_t)kThreads * flat_unroll(pieces);
  return (pieces + per - 1) / per;
}

// A grid of at most this many workgroups is resident all at once (four per
// CU): its scale bytes are streamed (see store_scale) and its waves load
// everything before they store.  Measured: the 4096 x 4096 row + column
// launch (1024 tiles) takes 13.3 us so and 13.8 us as a streaming grid; the
// 64 x 2048 x 7168 grouped launch (57344 tiles) 0.73 ms with streamed scale
// bytes and 0.67 ms written back.
constexpr int64_t kResidentTasks = 4 * 256;

template <class Args>
hipError_t launch_quantize_args(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  bool rowcol = true, narrow = false;
  for (int i = 0; i < a.n; ++i) {
    rowcol &= a.d[i].q_row != nullptr && a.d[i].q_col != nullptr;
    narrow |= narrow_col(a.d[i]);
  }
  const dim3 grid((uint32_t)total_tasks), block(kThreads);
  if (total_tasks <= kResidentTasks) {
    if (rowcol)
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, true, true>), grid, block, 0, s, a);
    else if (narrow)
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, true, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, true, false>), grid, block, 0, s, a);
  } else {
    if (rowcol)
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, false, true>), grid, block, 0, s, a);
    else if (narrow)
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, false, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((mxfp8_quantize_kernel<Args, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_quantize_args(a, total_tasks, s);
}

hipError_t launch_quantize(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_quantize_args(a, total_tasks, s);
}

}  // namespace mx
