// Fused RMSNorm + rowwise MXFP8 quantize.
//
// The fused op of the Mojo DistributedAllGatherRMSNormQuantMXFP8 page
// (execute; "Args": gammas, float32 epsilons, weight_offsets, outputs_normed,
// outputs_quant, outputs_scale [rows, cols/32]) on one GPU's rows:
//   normed = bf16( x / sqrt(mean(x^2) + eps) * (gamma + weight_offset) )
// rounded once (v_cvt_pk_bf16_f32); the quantize then reads the very bf16
// words that are stored as normed, so its bytes equal a standalone rowwise
// quantize of normed (the page's execute: the quantize rides the epilogue on
// the same bf16 that lands in outputs_normed).
//
// Range.  A row's sum of squares is first accumulated in float32.  When that
// sum lies in [2^-60, 2^120], float32 is exact enough (nothing overflows, and
// squares lost below float32's range are negligible), and rstd is its
// reciprocal square root.  Otherwise (rows of huge or tiny values, Inf, NaN;
// the branch is the same for every lane of the row) the squares are summed
// again in float64: the square of a bf16 value has at most 16 significant
// bits and lies between 2^-266 and 2^256, so every square is exact and no row
// sum (fewer than 2^31 elements) can overflow or underflow.  The mean square
// is formed in float64 and its reciprocal square root taken in float32 after
// an exact power-of-two range reduction.  Either way rstd is applied in
// float32 as (x * rstd) * w, the order the formula is written in;
// |x * rstd| <= sqrt(cols), so that product cannot overflow.  rstd exceeds
// float32's range only when the mean square is below about 2^-250, which
// needs eps == 0 and a row whose values all lie below 2^-124 * sqrt(cols);
// such a row is scaled by 2^64 first (exact) and rstd by 2^-64.  The IEEE
// cases follow from the formula: a zero row with eps == 0 is 0 / 0 (NaN
// everywhere); a row holding an infinity has rstd = 0 (its finite values give
// +-0, its infinities NaN); a row holding a NaN is NaN.
//
// A row belongs to one wave (rows up to 1024 elements, four rows per
// workgroup) or to all four waves of a workgroup (longer rows); a launch of
// few rows (decode) gives each row a workgroup of 16 waves instead, so each
// lane's serial work is a quarter as long.  Its L lanes
// hold NCH 16-byte chunks each in registers: chunk j of lane t is chunk
// t + L j of the row, so every load instruction reads L * 16 contiguous
// bytes.  The sum of squares is a per-lane chain, a fixed DPP reduction over
// each wave, and a fixed tree over the wave totals through LDS, so results do
// not depend on timing.  Rows too long for registers take two
// passes: the sum, then a second read that normalizes and quantizes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

// Adds the squares of a chunk's 8 values to a float32 or float64 sum (in
// float64 each square is exact).
template <class T>
__device__ __forceinline__ T sumsq_chunk(const u32x4& v, T acc) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const T lo = bf16_lo(v[k]), hi = bf16_hi(v[k]);
    acc = __builtin_fma(lo, lo, acc);
    acc = __builtin_fma(hi, hi, acc);
  }
  return acc;
}

// Sum over the 64 lanes.  Within each row of 16 lanes, four DPP steps pair
// lane i with lane i ^ 1, i ^ 2 (quad permutes), then with its mirror in the
// half row and in the row; each step adds the same two values in both
// partners (IEEE addition is commutative), so all 16 lanes hold the same row
// sum.  The four row sums are then read into scalars and added in one fixed
// order, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const u32x2 h = __builtin_bit_cast(u32x2, v);
  return __builtin_bit_cast(double, u32x2{(uint32_t)__builtin_amdgcn_mov_dpp((int)h.x, CTRL, 0xF, 0xF, true),
                                          (uint32_t)__builtin_amdgcn_mov_dpp((int)h.y, CTRL, 0xF, 0xF, true)});
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ double lane_value(double v, int lane) {
  const u32x2 h = __builtin_bit_cast(u32x2, v);
  return __builtin_bit_cast(double, u32x2{(uint32_t)__builtin_amdgcn_readlane((int)h.x, lane),
                                          (uint32_t)__builtin_amdgcn_readlane((int)h.y, lane)});
}

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
  v += dpp<0xB1>(v);    // quad [1, 0, 3, 2]
  v += dpp<0x4E>(v);    // quad [2, 3, 0, 1]
  v += dpp<0x141>(v);   // mirror within 8 lanes
  v += dpp<0x140>(v);   // mirror within 16 lanes
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// How a row's rstd is applied in float32 (see the file comment): rstd itself,
// or, for the rows whose rstd lies past float32's range, x * 2^64 times
// rstd * 2^-64.  The flag is the same in every lane of the row.
struct RowRstd {
  float r;
  bool pre;
};

// rstd = 1 / sqrt(ms), ms = ss / cols + eps formed in float64.  ms = m * 2^E
// with m in [0.5, 2) and E even (frexp, one exponent step moved into m when
// odd) is exact; rstd = rsq(m) * 2^(-E/2), with rsq(m) taken in float32
// (v_rsq_f32, within 1 ulp, after rounding m to float32), so the float32
// result is within a few 2^-24 of the exact one.  ms = 0 gives m = 0 and
// rstd = inf; ms = inf or NaN gives m = ms and rstd = 0 or NaN.
__device__ __forceinline__ RowRstd row_rstd(double ss, double inv_cols, float eps) {
  const double ms = __builtin_fma(ss, inv_cols, (double)eps);
  const double f = __builtin_amdgcn_frexp_mant(ms);   // [0.5, 1), or ms itself if 0 / inf / NaN
  const int e = __builtin_amdgcn_frexp_exp(ms);
  const int odd = e & 1;
  const float m = (float)(odd ? f * 2.0 : f);
  const float rm = __builtin_amdgcn_rsqf(m);
  const int k = -((e - odd) >> 1);                     // rstd = rm * 2^k
  const bool pre = k > 125;
  return RowRstd{__builtin_ldexpf(rm, pre ? k - 64 : k), pre};
}

// Normalize one chunk with its float32 weights w (gamma + offset), store
// normed, quantize the stored words.  y = ((x * pre) * rstd) * w, where pre
// is 1 except for the rows whose rstd lies past float32's range (2^64 there).
// ALLQ: all four lanes of the block store its scale byte (the same byte to
// the same address), so that no store sits behind a per-lane branch.
template <bool ALLQ = false>
__device__ __forceinline__ void finish_chunk(const NormDesc& d, ScaleStride ss, int64_t row,
                                             int64_t c, bool valid, const u32x4& v, const float* w,
                                             float rstd, float pre, int t) {
  u32x4 y;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    y[k] = pack_bf16x2(bf16_lo(v[k]) * pre * rstd * w[2 * k], bf16_hi(v[k]) * pre * rstd * w[2 * k + 1]);
  const RowScale rs = row_scale_key(quad_max(chunk_key(y)));
  const u32x2 q = encode_chunk_row(y, rs);
  if (valid) {
    const int64_t e = row * (int64_t)d.cols + c * kChunk;
    store16(d.normed + e, y);
    store8(d.q + e, q);
    if (ALLQ || (t & 3) == 0)
      store_scale<false>(d.s + scale_at(row, (c * kChunk) >> 5, ss.row, ss.grp), rs.sbyte);
  }
}

// gamma's 8 values of chunk c (zeros past the row), and the weights
// gamma + offset as float32.
__device__ __forceinline__ u32x4 load_gamma(const NormDesc& d, int64_t c, bool valid) {
  return valid ? load16_cached(d.gamma + c * kChunk) : u32x4{0, 0, 0, 0};
}

__device__ __forceinline__ void weights(const NormDesc& d, const u32x4& g, float* w) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[2 * k] = bf16_lo(g[k]) + d.weight_offset;
    w[2 * k + 1] = bf16_hi(g[k]) + d.weight_offset;
  }
}

// Sum of a row's partial sums: wave reduction, then (WPR > 1) the WPR wave
// totals through LDS in a fixed pairwise tree.  p holds the row's WPR slots;
// the float32 sums alternate between two such regions by row, so one barrier
// per row keeps writers of row k+1 off the values of row k.
template <int WPR, class T>
__device__ __forceinline__ T row_sum(T acc, int sub, int lane, T* p) {
  T w = wave_sum(acc);
  if constexpr (WPR == 1) {
    return w;
  } else {
    if (lane == 0) p[sub] = w;
    __syncthreads();
    T t[WPR];
#pragma unroll
    for (int k = 0; k < WPR; ++k) t[k] = p[k];
#pragma unroll
    for (int n = WPR; n > 1; n >>= 1)
#pragma unroll
      for (int k = 0; k < n / 2; ++k) t[k] = t[2 * k] + t[2 * k + 1];
    return t[0];
  }
}

// LDS of a workgroup: float32 row sums in two alternating regions, and one
// region for the float64 sums of the rare rows that need them.  A wave can
// write the float64 region for row k + 1 only after the float32 barrier of
// row k + 1, which every wave reaches after reading row k's float64 sums.
template <int WAVES>
struct RowParts {
  float f[2 * WAVES];
  double d[WAVES];
};

// Whether a row's float32 sum of squares ss32 can be used (the same answer
// in every lane of the row).  Inside [2^-60, 2^120] float32 is exact enough:
// no square or partial sum can overflow, squares lost below float32's range
// change the sum by less than 2^-35 of itself, and the sum's rounding error
// stays below 2^-17.  Otherwise (huge or tiny rows, Inf, NaN) the row's
// squares are summed again in float64.
__device__ __forceinline__ bool sum32_ok(float ss32) {
  return __builtin_amdgcn_readfirstlane((int)(ss32 >= 0x1p-60f && ss32 <= 0x1p120f));
}

__device__ __forceinline__ float rstd32(float ss32, float inv_cols32, float eps) {
  return __builtin_amdgcn_rsqf(__builtin_fmaf(ss32, inv_cols32, eps));
}

// rstd and the prescale of a row from its float64 sum of squares ss.  The
// empty asm keeps 1 / cols (a float64 division) inside the rare branch that
// calls this; the compiler would otherwise compute it for every row.
template <int WPR>
__device__ __forceinline__ void rstd64(double acc, int32_t cols, float eps, int sub, int lane,
                                       double* part64, float& r, float& pre) {
  asm volatile("" : "+s"(cols));
  const RowRstd rr = row_rstd(row_sum<WPR>(acc, sub, lane, part64), 1.0 / (double)cols, eps);
  r = rr.r;
  pre = rr.pre ? 0x1p64f : 1.0f;
}

// Rows first_row, first_row + step, ... (count of them) of one tensor; the
// row's L = 64 * WPR lanes each hold NCH chunks (chunk j of lane t is chunk
// t + L j).  The weights gamma + offset stay in registers across the rows.
// FULL: every chunk lies inside the row (cols == 8 L NCH), so no load or
// store waits behind a per-lane branch; the compiler cannot tell how many
// stores a branch issued, and would then wait for the wave's own stores.
// PF: the next row's loads go out before this row's stores (measured on
// 65536 x 7168: 392 against 406 us; launches with one row per slot do
// without: 16 x 7168 took 3.54 against 3.33 us with it).
template <int WPR, int NCH, bool FULL, bool PF, class Parts>
__device__ void norm_rows(const NormDesc& d, ScaleStride ss, int64_t first_row, int step, int count,
                          int sub, int lane, Parts* part) {
  constexpr int L = kWave * WPR;           // lanes per row
  const int t = sub * kWave + lane;        // this lane's index within the row
  const int64_t nch = d.cols / kChunk;
  // 1 / cols within 1 ulp (v_rcp_f32): the mean square needs no more
  const float inv_cols32 = __builtin_amdgcn_rcpf((float)d.cols);
  if constexpr (NCH > 0) {
    // gamma's loads, then the first row's, are issued before any arithmetic
    // waits on them
    u32x4 g[NCH], v[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int64_t c = t + (int64_t)j * L;
      g[j] = load_gamma(d, c, FULL || c < nch);
    }
    auto load_row = [&](int64_t row, u32x4 (&dst)[NCH]) {
      const uint16_t* xr = d.x + row * (int64_t)d.cols;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int64_t c = t + (int64_t)j * L;
        dst[j] = (FULL || c < nch) ? load16(xr + c * kChunk) : u32x4{0, 0, 0, 0};
      }
    };
    if (count > 0) load_row(first_row, v);
    float w[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) weights(d, g[j], w[j]);
    for (int k = 0; k < count; ++k) {
      const int64_t row = first_row + (int64_t)k * step;
      if (!PF && k > 0) load_row(row, v);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) acc = sumsq_chunk(v[j], acc);
      const float ss32 = row_sum<WPR>(acc, sub, lane, part->f + (k & 1) * WPR);
      float r, pre = 1.0f;
      if (sum32_ok(ss32)) {
        r = rstd32(ss32, inv_cols32, d.eps);
      } else {
        // the empty asm keeps this float64 work inside the branch (the
        // compiler would otherwise compute it for every row, ahead of the test)
        double a = 0.0;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          u32x4 x = v[j];
          asm volatile("" : "+v"(x));
          a = sumsq_chunk(x, a);
        }
        rstd64<WPR>(a, d.cols, d.eps, sub, lane, part->d, r, pre);
      }
      u32x4 vn[NCH];
      const bool more = PF && k + 1 < count;
      if (more) load_row(row + step, vn);
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int64_t c = t + (int64_t)j * L;
        finish_chunk<FULL>(d, ss, row, c, FULL || c < nch, v[j], w[j], r, pre, t);
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) v[j] = vn[j];
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
      const float ss32 = row_sum<WPR>(acc, sub, lane, part->f + (k & 1) * WPR);
      float r, pre = 1.0f;
      if (sum32_ok(ss32)) {
        r = rstd32(ss32, inv_cols32, d.eps);
      } else {
        double a = 0.0;
        for (int64_t c0 = 0; c0 < nch; c0 += L) {
          const int64_t c = c0 + t;
          const u32x4 v = c < nch ? load16_cached(xr + c * kChunk) : u32x4{0, 0, 0, 0};
          a = sumsq_chunk(v, a);
        }
        rstd64<WPR>(a, d.cols, d.eps, sub, lane, part->d, r, pre);
      }
      for (int64_t c0 = 0; c0 < nch; c0 += L) {
        const int64_t c = c0 + t;
        const bool valid = c < nch;
        const u32x4 v = valid ? load16_cached(xr + c * kChunk) : u32x4{0, 0, 0, 0};
        float w[8];
        weights(d, load_gamma(d, c, valid), w);
        finish_chunk(d, ss, row, c, valid, v, w, r, pre, t);
      }
    }
  }
}

// WAVES waves per workgroup, WPR waves per row (1, 4 or 16), NCH chunks per
// lane (0: two passes).  A task is rows_per_task consecutive rows of one
// tensor: with WPR == WAVES the whole workgroup walks them in order; with
// WPR == 1 wave w takes rows w, w + 4, ...
template <class Args, int WPR, int NCH, int WAVES = kWavesPerGroup, bool PF = false>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_rmsnorm_quantize_kernel(const Args a,
                                                                           int rows_per_task) {
  __shared__ RowParts<WAVES> part;
  constexpr int kSlots = WAVES / WPR;                   // row slots per workgroup
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t task = (int32_t)blockIdx.x;
  const int slot = wave / WPR;
  // one tensor: its descriptor is read together with the table size (the
  // empty asm keeps those loads ahead of the branch)
  NormDesc d0 = a.d[0];
  ScaleStride p0 = {0, 0};
  if constexpr (Args::kPitched) {
    p0 = a.pitch(0);
    asm volatile("" : "+s"(p0.row), "+s"(p0.grp));
  }
  asm volatile("" : "+s"(d0.x), "+s"(d0.gamma), "+s"(d0.normed), "+s"(d0.q), "+s"(d0.s),
               "+s"(d0.rows), "+s"(d0.cols), "+s"(d0.weight_offset), "+s"(d0.eps));
  if constexpr (!Args::kPitched) p0 = {d0.cols >> 5, 16};
  // a grouped launch replaces it with the task's own tensor
  int64_t row0 = (int64_t)task * rows_per_task;
  if (a.n != 1) {
    const int i = find_desc(a.task_start, a.n, task);
    d0 = a.d[i];
    p0 = Args::kPitched ? a.pitch(i) : ScaleStride{d0.cols >> 5, 16};
    row0 = (int64_t)(task - a.task_start[i]) * rows_per_task;
  }
  const int64_t left = (int64_t)d0.rows - row0;
  const int in_task = (int)(left < rows_per_task ? left : rows_per_task);
  const int count = (in_task - slot + kSlots - 1) / kSlots;   // rows slot, slot + kSlots, ...
  if (NCH > 0 && d0.cols == NCH * kWave * WPR * kChunk)
    norm_rows<WPR, NCH, true, PF>(d0, p0, row0 + slot, kSlots, count, wave % WPR, lane, &part);
  else
    norm_rows<WPR, NCH, false, PF>(d0, p0, row0 + slot, kSlots, count, wave % WPR, lane, &part);
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

// One kernel shape; the prefetching instantiation exists only where a slot
// can hold two rows (CAN_PF).
template <class Args, int WPR, int NCH, int WAVES = kWavesPerGroup, bool CAN_PF = true>
void launch_shape(const Args& a, dim3 grid, int rows_per_task, bool pf, hipStream_t s) {
  const dim3 block(64 * WAVES);
  if constexpr (CAN_PF) {
    if (pf) {
      hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, WPR, NCH, WAVES, true>), grid, block, 0, s, a,
                         rows_per_task);
      return;
    }
  }
  hipLaunchKernelGGL((mxfp8_rmsnorm_quantize_kernel<Args, WPR, NCH, WAVES, false>), grid, block, 0, s, a,
                     rows_per_task);
}

template <class Args>
hipError_t launch_norm(const Args& a, int64_t total_tasks, int variant, int rows_per_task,
                       hipStream_t s) {
  if (total_tasks <= 0) return hipSuccess;
  const dim3 grid((uint32_t)total_tasks);
  const int r = rows_per_task;
  // two rows a slot: prefetch the second (see norm_rows)
  const bool pf = rows_per_task > (variant < 10 ? kWavesPerGroup : 1);
  switch (variant) {
    case 161: launch_shape<Args, 16, 1, 16, false>(a, grid, r, pf, s); break;
    case 162: launch_shape<Args, 16, 2, 16, false>(a, grid, r, pf, s); break;
    case 1: launch_shape<Args, 1, 1>(a, grid, r, pf, s); break;
    case 2: launch_shape<Args, 1, 2>(a, grid, r, pf, s); break;
    case 11: launch_shape<Args, 4, 1>(a, grid, r, pf, s); break;
    case 12: launch_shape<Args, 4, 2>(a, grid, r, pf, s); break;
    case 14: launch_shape<Args, 4, 4>(a, grid, r, pf, s); break;
    case 18: launch_shape<Args, 4, 8>(a, grid, r, pf, s); break;
    default: launch_shape<Args, 4, 0, kWavesPerGroup, false>(a, grid, r, pf, s); break;
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
