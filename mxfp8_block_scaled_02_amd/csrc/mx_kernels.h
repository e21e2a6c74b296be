// Kernel argument blocks and launchers shared by the C ABI and the kernels.
//
// Every launch takes a small table of tensors (one entry for the single-
// tensor calls, up to kGroupMax for the grouped calls) passed by value in the
// kernel argument segment, plus a prefix sum of per-tensor wave tasks.  A
// wave finds its tensor by binary search over that prefix sum, so tensors of
// any mix of shapes share one launch (Megatron-Core quantized_dbuffer page:
// QuantizedDBuffer.empty builds one layout from a list of logical 2D shapes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kGroupMax = 64;        // tensors per launch (argument block < 4 KiB)
constexpr int kPitchedGroupMax = 32; // the same with per-tensor scale pitches
constexpr int kWavesPerGroup = 4;    // waves per workgroup
constexpr int kThreads = 64 * kWavesPerGroup;
constexpr int kLaneCols = 8;         // consecutive row elements a lane holds (8 or 16)
constexpr int kFlatUnroll = 4;       // kLaneCols-element pieces per lane per flat task
// A bf16 rowwise-only tensor of fewer pieces than this (fewer than 1024
// workgroups at kFlatUnroll pieces a lane) takes one piece a lane instead:
// four times the workgroups, each with a quarter of the serial work
// (measured on the 256 x 1024 workload: 2.56 us at 4 pieces a lane, 2.07 us
// at 1, against 1.53 us for an empty launch).
constexpr int64_t kSmallFlatPieces = (int64_t)1024 * kThreads * kFlatUnroll;
__host__ __device__ constexpr int flat_unroll(int64_t pieces) {
  return pieces < kSmallFlatPieces ? 1 : kFlatUnroll;
}
constexpr int kTileRows = 32;        // rows of a row+column tile (one MX block)
constexpr int kRowsPerWave = kTileRows / kWavesPerGroup;
constexpr int kTileCols = 64 * kLaneCols;  // columns of a tile
constexpr int kDeqUnroll = 8;        // 4-element units per lane per flat dequantize task
constexpr int kDeqRows = 4;          // rows per columnwise dequantize task
constexpr int kDeqTileCols = 256;    // columns per columnwise dequantize task: 64 lanes x 4

// ---- quantize ------------------------------------------------------------
struct QuantDesc {
  const uint16_t* x;
  uint8_t* q_row;
  uint8_t* s_row;  // NULL: rowwise plane not requested
  uint8_t* q_col;
  uint8_t* s_col;  // NULL: columnwise plane not requested
  int64_t rows, cols;
};
// Where a rowwise scale byte lives: block b of row r at
// r * row + (b / 16) * grp + b % 16 (see scale_at).  Compact planes have
// row = the plane's width and grp = 16; a padded allocation (a consumer's
// layout) has a larger row; the MFMA order has row = 16 and grp = rows * 16.
struct ScaleStride {
  int64_t row, grp;
};
// Scale strides of a quantize call: rowwise (row, grp) and the columnwise
// plane's row pitch (its rows are always contiguous).
struct QuantPitch {
  int64_t s_row, s_col, s_grp;
};
// Compact planes: the pitch follows from the shape.
struct QuantArgs {
  static constexpr int kMax = kGroupMax;
  static constexpr bool kPitched = false;
  int32_t n;
  int32_t task_start[kMax + 1];
  QuantDesc d[kMax];
  __device__ QuantPitch pitch(int i) const { return {d[i].cols >> 5, d[i].cols, 16}; }
};
// Planes with pitches of their own (fewer tensors per launch: the argument
// block stays under 4 KiB).
struct QuantArgsPitched {
  static constexpr int kMax = kPitchedGroupMax;
  static constexpr bool kPitched = true;
  int32_t n;
  int32_t task_start[kMax + 1];
  QuantDesc d[kMax];
  QuantPitch p[kMax];
  __device__ QuantPitch pitch(int i) const { return p[i]; }
};
// A columnwise-only request whose rows are not a multiple of 8 elements: its
// rows start off the 16-byte grid, so it takes the narrow path (one thread per
// column of a 32-row block, element-sized accesses) instead of the tiles.
__host__ __device__ inline bool narrow_col(const QuantDesc& d) {
  return d.q_col != nullptr && d.q_row == nullptr && (d.cols & 7) != 0;
}
// Workgroup tasks a tensor needs: 32 x 512 tiles when a columnwise plane is
// requested (32-row blocks of 256 columns on the narrow path), otherwise
// 256 x flat_unroll 8-element pieces of the flattened tensor.
int64_t quant_tasks(const QuantDesc& d);
hipError_t launch_quantize(const QuantArgs& a, int64_t total_tasks, hipStream_t s);
hipError_t launch_quantize(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s);
// The same for float32 input (QuantDesc::x points to float): 32 x 256 tiles
// or 256 x kFlatUnroll 4-element pieces.
int64_t quant_f32_tasks(const QuantDesc& d);
hipError_t launch_quantize_f32(const QuantArgs& a, int64_t total_tasks, hipStream_t s);
hipError_t launch_quantize_f32(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s);

// Transposed columnwise plane (a quantize descriptor whose columnwise scale
// pitch is MXFP8_COLUMNWISE_T): q_col [cols, rows], s_col [cols, rows/32],
// written from 128 x 256 tiles (rows % 32 == 0, cols % 8 == 0); the rowwise
// plane, when requested, as usual.  Workgroup tasks: one per tile.
constexpr int kTRows = 128;          // rows of a transposing tile (4 waves x one 32-row block)
constexpr int kTCols = 256;          // columns of a transposing tile (32 lanes x 8)
int64_t quant_colt_tasks(const QuantDesc& d);
hipError_t launch_quantize_colt(const QuantArgs& a, int64_t total_tasks, hipStream_t s);
hipError_t launch_quantize_colt(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s);
// The same for float32 input: 128 x 128 tiles.
int64_t quant_f32_colt_tasks(const QuantDesc& d);
hipError_t launch_quantize_f32_colt(const QuantArgs& a, int64_t total_tasks, hipStream_t s);
hipError_t launch_quantize_f32_colt(const QuantArgsPitched& a, int64_t total_tasks, hipStream_t s);

// ---- RMSNorm + rowwise quantize ------------------------------------------
struct NormDesc {
  const uint16_t* x;
  const uint16_t* gamma;
  uint16_t* normed;
  uint8_t* q;
  uint8_t* s;
  int32_t rows, cols;
  float weight_offset, eps;
};
struct NormArgs {
  static constexpr int kMax = kGroupMax;
  static constexpr bool kPitched = false;
  int32_t n;
  int32_t task_start[kMax + 1];
  NormDesc d[kMax];
  __device__ ScaleStride pitch(int i) const { return {d[i].cols >> 5, 16}; }
};
struct NormArgsPitched {
  static constexpr int kMax = kPitchedGroupMax;
  static constexpr bool kPitched = true;
  int32_t n;
  int32_t task_start[kMax + 1];
  NormDesc d[kMax];
  ScaleStride p[kMax];
  __device__ ScaleStride pitch(int i) const { return p[i]; }
};
// Kernel shape from the longest row of a launch and its total row count:
// waves per row and chunks per lane (see rmsnorm_quantize.hip).  A task is
// rows_per_task consecutive rows of one tensor, also chosen from the total
// row count.  Launches of at most kWideNormRows rows use 16 waves per row.
constexpr int64_t kWideNormRows = 256;
int norm_variant(int64_t cols, int64_t total_rows);
int norm_rows_per_task(int64_t total_rows, int variant);
hipError_t launch_rmsnorm_quantize(const NormArgs& a, int64_t total_tasks, int variant,
                                   int rows_per_task, hipStream_t s);
hipError_t launch_rmsnorm_quantize(const NormArgsPitched& a, int64_t total_tasks, int variant,
                                   int rows_per_task, hipStream_t s);

// ---- dequantize ----------------------------------------------------------
struct DeqDesc {
  const uint8_t* q;
  const uint8_t* s;
  void* out;
  int64_t rows, cols;
  int32_t axis;  // 0 rowwise scales, 1 columnwise scales
};
struct DeqArgs {
  static constexpr int kMax = kGroupMax;
  static constexpr bool kPitched = false;
  int32_t n;
  int32_t out_bf16;
  int32_t task_start[kMax + 1];
  DeqDesc d[kMax];
  __device__ ScaleStride pitch(int i) const { return {d[i].axis ? d[i].cols : d[i].cols >> 5, 16}; }
};
struct DeqArgsPitched {
  static constexpr int kMax = kPitchedGroupMax;
  static constexpr bool kPitched = true;
  int32_t n;
  int32_t out_bf16;
  int32_t task_start[kMax + 1];
  DeqDesc d[kMax];
  ScaleStride p[kMax];   // columnwise planes: p.row is the row pitch
  __device__ ScaleStride pitch(int i) const { return p[i]; }
};
// Columnwise planes whose rows are not a multiple of 8 elements take a
// narrow path: one lane per column, element-sized accesses.
__host__ __device__ inline bool narrow_deq(const DeqDesc& d) { return d.axis == 1 && (d.cols & 7) != 0; }
int64_t deq_tasks(const DeqDesc& d);
hipError_t launch_dequantize(const DeqArgs& a, int64_t total_tasks, hipStream_t s);
hipError_t launch_dequantize(const DeqArgsPitched& a, int64_t total_tasks, hipStream_t s);

// ---- MXFP8 matrix product -------------------------------------------------
// out[M, N] (float32, or bf16 if out_bf16) = A . B^T for rowwise planes
// A = (qa [M, K], sa [M, K/32]), B = (qb [N, K], sb [N, K/32]); K % 128 == 0.
// The scale planes' strides are sa and sb (row strides multiples of 4; the
// MFMA order only with K % 512 == 0); output rows are out_ld elements apart.
hipError_t launch_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, ScaleStride sa_stride, ScaleStride sb_stride,
                       void* out, int64_t out_ld, bool out_bf16, hipStream_t s);
// A list of products (MoE experts), in shared launches: products of up to
// kGroupSkinnyRows rows (or up to kGemmGroupRows with K < 512) run the
// skinny kernel, one workgroup per 32 output columns with one, two or four
// 32-row A tiles; the others with K >= 512 run ring tiles, each product with
// its own tile size; a table of up to 32 products per launch, one table for
// each kernel variant.  Products of more than kGemmGroupRows rows with
// K < 512 take launch_gemm's route one by one.
struct GemmDesc {
  const uint8_t *qa, *sa, *qb, *sb;
  int64_t M, N, K;
  ScaleStride sa_stride, sb_stride;
  void* out;
  int64_t out_ld;
};
constexpr int64_t kGemmGroupRows = 128;
constexpr int64_t kGroupSkinnyRows = 32;
hipError_t launch_gemm_grouped(const GemmDesc* d, int n, bool out_bf16, hipStream_t s);

// The tensor of a launch's table that task belongs to: the last i with
// start[i] <= task, by binary search over the prefix sum of task counts.
__device__ __forceinline__ int find_desc(const int32_t* start, int n, int32_t task) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= task) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Byte offset of the scale of block b of row r (see ScaleStride):
// r * row + (b / 16) * grp + b % 16, written so that a grp known to be 16
// leaves r * row + b.
__device__ __forceinline__ int64_t scale_at(int64_t r, int64_t b, int64_t row, int64_t grp) {
  return r * row + b + (b >> 4) * (grp - 16);
}

// Scale offset of flat block b of a plane with bpr blocks per row
// (b < 2^32 whenever the plane is not compact).
__device__ __forceinline__ int64_t pitched_block(int64_t b, int64_t bpr, ScaleStride st) {
  if (st.row == bpr && st.grp == 16) return b;
  const uint32_t ub = (uint32_t)b, ubpr = (uint32_t)bpr;
  const uint32_t r = ub / ubpr;
  return scale_at(r, ub - r * ubpr, st.row, st.grp);
}

}  // namespace mx
