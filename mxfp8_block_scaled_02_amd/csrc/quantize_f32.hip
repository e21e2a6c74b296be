// float32 -> MXFP8 quantize: the planes of a float32 master weight.
//
// The same planes and rule as the bf16 quantize (quantize.hip), applied to
// float32 values: quantizing a local float32 master shard into its planes is
// the Megatron-Core quantized_dbuffer page's QuantizedDBuffer.quantize_.
//
// A lane holds 4 consecutive float32 of a row (one 16-byte load, so every
// load instruction reads 1 KiB of contiguous memory); a rowwise block is 8
// lanes and its amax takes three DPP steps.  Tile tasks (any columnwise
// request) are 32 rows x 256 columns per workgroup, 8 rows per wave; flat
// tasks (rowwise only) walk 256 x kFlatUnroll pieces of 4 elements.
//
// The columnwise plane stored transposed (q_col [cols, rows], see
// quantize_colt.hip for the bf16 form) comes from 128 x 128 tiles: wave w
// takes rows 32 w .. 32 w + 31, lane l holds 4 columns of 16 rows (each load
// instruction reads 2 rows x 512 contiguous bytes), a rowwise block is 8
// lanes, a columnwise block the lane pair l, l ^ 32.  Each lane converts its
// 16 rows of a column into one 16-byte chunk of a column-major tile in LDS,
// which the workgroup then stores as whole 128-byte lines of q_col.
//
// Scaling and rounding use v_cvt_scalef32_pk_fp8_f32 with scale operand
// 2^(S-127), which divides by the scale and rounds to nearest even; like the
// bf16 form it turns magnitudes >= 464 into NaN, so every input is first
// clamped to +-448 * 2^(S-127) with v_med3_f32.  A NaN/Inf block or column is
// reduced to signed zeros before the clamp (so med3 never sees a NaN) and
// its bytes become sign | 0x7F.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kF32Lane = 4;                       // float32 per lane per row
constexpr int kF32TileCols = kWave * kF32Lane;    // 256

__device__ __forceinline__ uint32_t f32_key4(const u32x4& v) {
  return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

// Max over each aligned group of 8 lanes: two quad permutes, then the mirror
// within 8 lanes, which pairs lane i with lane 7 - i.
__device__ __forceinline__ uint32_t oct_max(uint32_t k) {
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x141, 0xF, 0xF, true));  // half mirror
  return k;
}

// Scale parameters of a float32 block from its magnitude key (float32 bits
// & 0x7FFFFFFF).  S = exponent field - 8, clamped at 0; NaN/Inf -> 0xFF.
struct F32Scale {
  float div;       // scale operand 2^(S-127) (S == 0: the subnormal 2^-127)
  float lim;       // 448 * 2^(S-127)
  uint32_t nan;    // 1 for a NaN/Inf block
  uint32_t sbyte;  // stored scale byte
};

__device__ __forceinline__ F32Scale f32_scale_key(uint32_t key) {
  const uint32_t e = min(key, 0x7F7FFFFFu) >> 23;
  const uint32_t s = e > 8u ? e - 8u : 0u;
  F32Scale r;
  r.div = __builtin_bit_cast(float, s ? (s << 23) : 0x00400000u);
  r.lim = __builtin_bit_cast(float, (max(e, 8u) << 23) | 0x00600000u);  // 1.75 * 2^(S+8-127)
  r.nan = key >= 0x7F800000u ? 1u : 0u;
  r.sbyte = r.nan ? 0xFFu : s;
  return r;
}

__device__ __forceinline__ float med(uint32_t bits, float lim) {
  return __builtin_amdgcn_fmed3f(__builtin_bit_cast(float, bits), -lim, lim);
}

// 4 e4m3 bytes of 4 float32 sharing one block scale.
__device__ __forceinline__ uint32_t encode4_row(u32x4 v, const F32Scale& sc) {
  if (sc.nan) v &= 0x80000000u;   // keep only the signs; the bytes become sign | 0x7F
  v2i16 a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
      __builtin_bit_cast(v2i16, v.x), med(v.x, sc.lim), med(v.y, sc.lim), sc.div, false);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, med(v.z, sc.lim), med(v.w, sc.lim), sc.div, true);
  return __builtin_bit_cast(uint32_t, a) | (sc.nan ? 0x7F7F7F7Fu : 0u);
}

// The narrow columnwise path (narrow_col), as for bf16: one column of a
// 32-row block per thread, element-sized accesses, the rowwise block code on
// the column's 32 values.
__device__ void quant_f32_col_narrow_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid) {
  const int64_t cols = d.cols;
  const int64_t col_tasks = (cols + kThreads - 1) / kThreads;
  const int64_t rb = task / col_tasks;
  const int64_t c = (task % col_tasks) * kThreads + tid;
  if (c >= cols) return;                                   // no barrier follows
  const float* xp = reinterpret_cast<const float*>(d.x) + rb * kBlock * cols + c;
  u32x4 v[kBlock / 4];
  uint32_t key = 0;
#pragma unroll
  for (int j = 0; j < kBlock / 4; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[j][k] = *gload_ptr<uint32_t>(xp + (4 * j + k) * cols);
    key = max(key, f32_key4(v[j]));
  }
  const F32Scale sc = f32_scale_key(key);
  uint8_t* qp = d.q_col + rb * kBlock * cols + c;
#pragma unroll
  for (int j = 0; j < kBlock / 4; ++j) {
    const uint32_t e = encode4_row(v[j], sc);
#pragma unroll
    for (int k = 0; k < 4; ++k) *gstore_ptr<uint8_t>(qp + (4 * j + k) * cols) = (uint8_t)(e >> (8 * k));
  }
  store_scale<false>(d.s_col + rb * pitch.s_col + c, sc.sbyte);
}

__device__ void quant_f32_flat_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid) {
  const float* x = reinterpret_cast<const float*>(d.x);
  const int64_t npieces = d.rows * d.cols / kF32Lane;    // whole blocks: cols % 32 == 0
  const int64_t base = task * (int64_t)(kThreads * kFlatUnroll) + tid;
  u32x4 v[kFlatUnroll];
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    const int64_t p = base + u * kThreads;
    v[u] = p < npieces ? load16(x + p * kF32Lane) : kZero4;
  }
#pragma unroll
  for (int u = 0; u < kFlatUnroll; ++u) {
    const int64_t p = base + u * kThreads;
    const F32Scale sc = f32_scale_key(oct_max(f32_key4(v[u])));
    const uint32_t q = encode4_row(v[u], sc);
    if (p < npieces) {
      store4(reinterpret_cast<uint32_t*>(d.q_row) + p, q);
      if ((tid & 7) == 0)
        store_scale<false>(d.s_row + pitched_block(p >> 3, d.cols >> 5, ScaleStride{pitch.s_row, pitch.s_grp}),
                           sc.sbyte);
    }
  }
}

// ROW: the rowwise plane is requested too.  The two cases are separate code
// so that neither path's waits for its loads are merged with the other's (a
// shared columnwise part made the rowwise path wait for its own rowwise
// stores before the column maxima).
template <bool ROW>
__device__ void quant_f32_tile_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int wave, int lane,
                                    u32x4* colmax) {
  const float* x = reinterpret_cast<const float*>(d.x);
  const int64_t cols = d.cols;
  const int64_t col_tiles = (cols + kF32TileCols - 1) / kF32TileCols;
  if constexpr (ROW) {
    // The column tiles of a row block share its rowwise scale lines (8 bytes
    // each of every 128-byte line).  Workgroup ids are spread over the 8 XCDs
    // in turn, so tiles whose ids are 8 apart run on one XCD, and their pieces
    // meet in its L2.  Tile (rb, ct) takes id 8 (col_tiles (rb / 8) + ct) +
    // rb % 8, a permutation whenever the row blocks are a multiple of 8.
    // Measured on the 4096 x 4096 weight, with the scale bytes stored last:
    // 18.6 us, against 19.0 us in row-major order.
    if ((d.rows / kTileRows) % 8 == 0) {
      const int64_t j = task >> 3;
      task = ((j / col_tiles) * 8 + (task & 7)) * col_tiles + j % col_tiles;
    }
  }
  const int64_t rb = task / col_tiles;
  const int64_t r0 = rb * kTileRows + wave * kRowsPerWave;
  const int64_t c = (task % col_tiles) * kF32TileCols + (int64_t)lane * kF32Lane;
  // Lanes past the row's end (only in a last, partial column tile) never load
  // or store behind a branch: the compiler cannot know whether a store inside
  // an `if` was issued, so it then waits for more loads, and finally for the
  // wave's earlier stores, before each row (measured on the 4096 x 4096
  // weight: 21.4 us with guarded stores, 20.0 us without).
  //   ROW (both planes; cols % 32 == 0): such a lane takes column
  //   (lane % 8) * 4 of the same rows instead.  Its aligned group of 8 lanes
  //   then covers columns 0..31 of the tile's 32 rows exactly, so it computes
  //   the very bytes, row scales and column scales that the lanes owning
  //   those columns compute, and its stores rewrite identical bytes.
  //   !ROW (columnwise only; cols % 8 == 0): such a lane reads columns 0..3
  //   (always inside the tensor), and its stores are skipped; what it
  //   computes reaches no output, since a column's maximum is its own lane's.
  const bool ok = c < cols;
  const int64_t ce = ok ? c : (ROW ? (int64_t)(lane & 7) * kF32Lane : 0);
  const float* xp = x + r0 * cols + ce;
  const bool st = ROW || ok;

  u32x4 v[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) v[r] = load16(xp + r * cols);

  // rowwise scale bytes, packed four to a dword (row r in byte r % 4 of word
  // r / 4) and stored after every data store of the tile: 19.0 us against
  // 20.1 us with each byte next to its row's data
  uint32_t row_sb[kRowsPerWave / 4] = {};
  if constexpr (ROW) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const F32Scale sc = f32_scale_key(oct_max(f32_key4(v[r])));
      const uint32_t q = encode4_row(v[r], sc);
      row_sb[r / 4] |= sc.sbyte << (8 * (r % 4));
      store4_cached(d.q_row + (r0 + r) * cols + ce, q);
    }
  }

  {
    u32x4 m = kZero4;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) m = __builtin_elementwise_max(m, v[r] & 0x7FFFFFFFu);
    colmax[wave * kWave + lane] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w)
      if (w != wave) m = __builtin_elementwise_max(m, colmax[w * kWave + lane]);
    F32Scale sc[kF32Lane];
    uint32_t any_nan = 0, nanq = 0, sbytes = 0;
#pragma unroll
    for (int k = 0; k < kF32Lane; ++k) {
      sc[k] = f32_scale_key(m[k]);
      any_nan |= sc[k].nan;
      nanq |= (sc[k].nan ? 0x7Fu : 0u) << (8 * k);
      sbytes |= sc[k].sbyte << (8 * k);
    }
    if (st && wave == 0)
      store4_cached(d.s_col + rb * pitch.s_col + ce, sbytes);
    if (any_nan) {
      // a NaN/Inf column keeps only each element's sign bit
      u32x4 keep;
#pragma unroll
      for (int k = 0; k < kF32Lane; ++k) keep[k] = sc[k].nan ? 0x80000000u : 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) v[r] &= keep;
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r += 2) {
      // columns k = 0..3 of rows r, r+1: one conversion per column (two rows)
      uint32_t dd[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k0 = 2 * h, k1 = 2 * h + 1;
        v2i16 t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
            __builtin_bit_cast(v2i16, v[r][k0]), med(v[r][k0], sc[k0].lim),
            med(v[r + 1][k0], sc[k0].lim), sc[k0].div, false);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, med(v[r][k1], sc[k1].lim),
                                                     med(v[r + 1][k1], sc[k1].lim), sc[k1].div, true);
        dd[h] = __builtin_bit_cast(uint32_t, t);   // bytes (r,k0) (r+1,k0) (r,k1) (r+1,k1)
      }
      const uint32_t q0 = __builtin_amdgcn_perm(dd[1], dd[0], 0x06040200u) | nanq;
      const uint32_t q1 = __builtin_amdgcn_perm(dd[1], dd[0], 0x07050301u) | nanq;
      if (st) {
        uint8_t* qp = d.q_col + (r0 + r) * cols + ce;
        store4(qp, q0);
        store4(qp + cols, q1);
      }
    }
  }

  if (ROW && (lane & 7) == 0) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
      store_scale<false>(d.s_row + scale_at(r0 + r, ce >> 5, pitch.s_row, pitch.s_grp),
                         row_sb[r / 4] >> (8 * (r % 4)));
  }
}

// ---- transposed columnwise plane -------------------------------------------

constexpr int kF32TRowsPerWave = kTRows / kWavesPerGroup;   // one 32-row column block
constexpr int kF32TLaneRows = 16;                            // rows a lane holds
constexpr int kF32TCols = 32 * kF32Lane;                     // 128: 32 lanes x 4 columns
static_assert(kF32TRowsPerWave == 2 * kF32TLaneRows && kF32TRowsPerWave == kBlock, "lane grid");

// chunk k (rows 16 k ..) of tile column cl: 128-byte columns, chunks
// XOR-swizzled by the column's lane (cl / 4)
__device__ __forceinline__ int f32_colt_at(int cl, int k) {
  return cl * kTRows + ((k ^ ((cl >> 2) & 7)) << 4);
}

struct F32ColtLds {
  uint8_t tile[kF32TCols * kTRows];
  uint32_t scol[kF32TCols];   // 4 column scale bytes per column (one per wave)
  uint32_t srow[kTRows];      // 4 row scale bytes per row (one per 32 columns)
};

// ROW: the rowwise plane is requested too (then cols % 32 == 0).  Lanes and
// waves outside the tensor work on mirrors, as in the bf16 form: a wave past
// the end takes the tensor's last block; a lane past the end takes columns
// (l % 8) * 4 of its rows (ROW: its 8-lane group then covers columns 0..31
// exactly and rewrites its owners' bytes) or 0..3 (columnwise only, cols % 8
// == 0).  Their columnwise results land in LDS rows or columns past the
// tensor, which the final stores skip.
template <bool ROW>
__device__ void quant_f32_colt_task(const QuantDesc& d, const QuantPitch& pitch, int64_t task, int tid, int wave,
                                    F32ColtLds& lds) {
  const float* x = reinterpret_cast<const float*>(d.x);
  const int lane = tid & (kWave - 1);
  const int64_t rows = d.rows, cols = d.cols;
  const int64_t col_tiles = (cols + kF32TCols - 1) / kF32TCols;
  const int64_t r0 = (task / col_tiles) * kTRows, c0 = (task % col_tiles) * kF32TCols;
  const int cc = lane & 31, rg = lane >> 5;
  const int ro = kF32TRowsPerWave * wave + kF32TLaneRows * rg;   // the lane's first row in the tile
  const int64_t c = c0 + kF32Lane * cc;
  const int64_t ce = c < cols ? c : (ROW ? (int64_t)(lane & 7) * kF32Lane : 0);
  const int64_t rbase = r0 + ro < rows ? r0 + ro : rows - kF32TRowsPerWave + kF32TLaneRows * rg;
  const float* xp = x + rbase * cols + ce;
  u32x4 v[kF32TLaneRows];
#pragma unroll
  for (int r = 0; r < kF32TLaneRows; ++r) v[r] = load16(xp + r * cols);

  if constexpr (ROW) {
    uint8_t* srow8 = reinterpret_cast<uint8_t*>(lds.srow);
#pragma unroll
    for (int r = 0; r < kF32TLaneRows; ++r) {
      const F32Scale sc = f32_scale_key(oct_max(f32_key4(v[r])));
      // written back, as in the 32 x 256 tiles (4096 x 4096: 23.1 against 23.4 us
      // streamed; 8192 x 7168: 67.1 against 71.9 us)
      store4_cached(d.q_row + (rbase + r) * cols + ce, encode4_row(v[r], sc));
      if ((cc & 7) == 0) srow8[(ro + r) * 4 + (cc >> 3)] = (uint8_t)sc.sbyte;
    }
  }

  // column maxima: the lane's 16 rows, then the other lane of the block
  u32x4 m = kZero4;
#pragma unroll
  for (int r = 0; r < kF32TLaneRows; ++r) m = __builtin_elementwise_max(m, v[r] & 0x7FFFFFFFu);
#pragma unroll
  for (int k = 0; k < kF32Lane; ++k) m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], 32));

  uint8_t* scol8 = reinterpret_cast<uint8_t*>(lds.scol);
#pragma unroll
  for (int k = 0; k < kF32Lane; ++k) {
    const F32Scale sc = f32_scale_key(m[k]);
    // a NaN/Inf column keeps only each element's sign bit; its bytes become sign | 0x7F
    const uint32_t keep = sc.nan ? 0x80000000u : 0xFFFFFFFFu, nanq = sc.nan ? 0x7F7F7F7Fu : 0u;
    u32x4 col;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t a0 = v[4 * h][k] & keep, a1 = v[4 * h + 1][k] & keep;
      const uint32_t a2 = v[4 * h + 2][k] & keep, a3 = v[4 * h + 3][k] & keep;
      v2i16 t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2i16, a0), med(a0, sc.lim),
                                                         med(a1, sc.lim), sc.div, false);
      t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, med(a2, sc.lim), med(a3, sc.lim), sc.div, true);
      col[h] = __builtin_bit_cast(uint32_t, t) | nanq;   // rows 4h .. 4h + 3 of the column
    }
    const int cl = kF32Lane * cc + k;
    *reinterpret_cast<u32x4*>(lds.tile + f32_colt_at(cl, ro >> 4)) = col;
    if (rg == 0) scol8[cl * 4 + wave] = (uint8_t)sc.sbyte;
  }
  __syncthreads();

  const int64_t trows = rows - r0 < kTRows ? rows - r0 : kTRows;   // 32, 64, 96 or 128
#pragma unroll
  for (int q = 0; q < kF32TCols * kTRows / 16 / kThreads; ++q) {
    const int id = tid + kThreads * q, cl = id >> 3, k = id & 7;
    if (c0 + cl < cols && 16 * k < trows)
      store16(d.q_col + (c0 + cl) * rows + r0 + 16 * k, *reinterpret_cast<const u32x4*>(lds.tile + f32_colt_at(cl, k)));
  }
  if (tid < kF32TCols) {
    // column scales: thread t takes tile column t (4 row blocks)
    if (c0 + tid < cols) {
      const uint32_t w = lds.scol[tid];
      uint8_t* sp = d.s_col + (c0 + tid) * (rows / kBlock) + r0 / kBlock;
      if (rows % kTRows == 0) {
        store4_cached(sp, w);                   // 4-byte aligned: rows / 32 % 4 == 0
      } else {
        for (int b = 0; b < trows / kBlock; ++b) *gstore_ptr<uint8_t>(sp + b) = (uint8_t)(w >> (8 * b));
      }
    }
  } else if (ROW) {
    // row scales: thread 128 + t takes tile row t (4 column blocks; 4-byte
    // aligned where the tile is whole: b0 % 4 == 0, also in the MFMA order)
    const int t = tid - kF32TCols;
    if (t < trows) {
      const int64_t row = r0 + t, b0 = c0 / kBlock;
      const uint32_t w = lds.srow[t];
      if (pitch.s_row % 4 == 0 && c0 + kF32TCols <= cols) {
        store4_cached(d.s_row + scale_at(row, b0, pitch.s_row, pitch.s_grp), w);
      } else {
        for (int b = 0; b < 4 && (b0 + b) * kBlock < cols; ++b)
          *gstore_ptr<uint8_t>(d.s_row + scale_at(row, b0 + b, pitch.s_row, pitch.s_grp)) = (uint8_t)(w >> (8 * b));
      }
    }
  }
}

template <class Args>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_f32_colt_kernel(const Args a) {
  __shared__ __attribute__((aligned(16))) F32ColtLds lds;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int i = a.n == 1 ? 0 : find_desc(a.task_start, a.n, task);
  const QuantDesc d = a.d[i];
  const QuantPitch p = a.pitch(i);
  const int64_t local = task - a.task_start[i];
  if (d.q_row != nullptr)
    quant_f32_colt_task<true>(d, p, local, tid, wave, lds);
  else
    quant_f32_colt_task<false>(d, p, local, tid, wave, lds);
}

// ROWCOL: every tensor of the launch requests both planes (the launcher
// checks), so only that tile path is compiled in.  Compiled together, the two
// tile paths share their loads and columnwise part and need 79 VGPRs against
// 47 for this one, which would cut the waves a SIMD holds from 8 to 5.
// ROWCOL: every tensor requests both planes; NARROW: some tensor takes the
// narrow columnwise path (only such launches carry its code).
template <class Args, bool ROWCOL, bool NARROW = false>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_f32_kernel(const Args a) {
  __shared__ u32x4 colmax[kThreads];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  // one tensor: its descriptor is read together with the table size (the
  // empty asm keeps those loads ahead of the branch)
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
    quant_f32_tile_task<true>(d0, p0, local, wave, lane, colmax);
  } else {
    if (d0.q_col) {
      if (d0.q_row)
        quant_f32_tile_task<true>(d0, p0, local, wave, lane, colmax);
      else if (NARROW && narrow_col(d0))
        quant_f32_col_narrow_task(d0, p0, local, tid);
      else
        quant_f32_tile_task<false>(d0, p0, local, wave, lane, colmax);
    } else {
      quant_f32_flat_task(d0, p0, local, tid);
    }
  }
}

}  // namespace

int64_t quant_f32_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  if (narrow_col(d)) return (d.rows / kBlock) * ((d.cols + kThreads - 1) / kThreads);
  if (d.q_col)
    return (d.rows / kTileRows) * ((d.cols + kF32TileCols - 1) / kF32TileCols);
  const int64_t pieces = d.rows * d.cols / kF32Lane;
  const int64_t per = (int64_t)kThreads * kFlatUnroll;
  return (pieces + per - 1) / per;
}

template <class Args>
hipError_t launch_f32(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  bool rowcol = true, narrow = false;
  for (int i = 0; i < a.n; ++i) {
    rowcol &= a.d[i].q_row != nullptr && a.d[i].q_col != nullptr;
    narrow |= narrow_col(a.d[i]);
  }
  const dim3 grid((uint32_t)total_tasks), block(kThreads);
  if (rowcol)
    hipLaunchKernelGGL((mxfp8_quantize_f32_kernel<Args, true>), grid, block, 0, s, a);
  else if (narrow)
    hipLaunchKernelGGL((mxfp8_quantize_f32_kernel<Args, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((mxfp8_quantize_f32_kernel<Args, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_f32(a, total_tasks, s);
}

int64_t quant_f32_colt_tasks(const QuantDesc& d) {
  if (d.rows == 0 || d.cols == 0) return 0;
  return ((d.rows + kTRows - 1) / kTRows) * ((d.cols + kF32TCols - 1) / kF32TCols);
}

template <class Args>
hipError_t launch_f32_colt(const Args& a, int64_t total_tasks, hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  hipLaunchKernelGGL((mxfp8_quantize_f32_colt_kernel<Args>), dim3((uint32_t)total_tasks), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_quantize_f32_colt(const QuantArgs& a, int64_t total_tasks, hipStream_t s) {
  return launch_f32_colt(a, total_tasks, s);
}

hipError_t launch_quantize_f32_colt(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_f32_colt(a, total_tasks, s);
}

hipError_t launch_quantize_f32(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s) {
  return launch_f32(a, total_tasks, s);
}

}  // namespace mx
