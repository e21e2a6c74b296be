// C ABI of libmxfp8 (declared in include/mxfp8.h): argument checks, tensor
// tables and launches.  Every check runs before the first launch, so a call
// that fails has enqueued nothing.  The library holds no state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <vector>

#include "mx_kernels.h"
#include "mxfp8.h"

namespace {


bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Largest task count one launch (and so one tensor) may carry.
constexpr int64_t kMaxTasksPerLaunch = (int64_t)1 << 30;
// Largest count of 64 x 32 output tiles of a matrix product.
constexpr int64_t kMaxGemmTiles = (int64_t)1 << 28;

bool fits(int64_t rows, int64_t cols) {
  return rows >= 0 && cols >= 0 && (cols == 0 || rows <= INT64_MAX / 4 / cols);
}

// A flat (rowwise-only) task finds a block's scale row by 32-bit division
// when its plane has a pitch of its own.
bool flat_blocks_fit(int64_t rows, int64_t cols) { return rows * (cols / MXFP8_BLOCK) <= (int64_t)UINT32_MAX; }

// A rowwise scale plane in the MFMA order needs whole 512-element groups.
bool mfma_order_ok(int64_t pitch, int64_t cols) { return pitch != MXFP8_SCALES_MFMA || cols % 512 == 0; }

// The columnwise plane of d is requested and stored transposed.
bool col_t(const mxfp8_quant_desc& d) {
  return d.s_col_pitch == MXFP8_COLUMNWISE_T && (d.q_col != nullptr || d.s_col != nullptr);
}

mxfp8_status check_quant(const mxfp8_quant_desc& d) {
  if (d.rows < 0 || d.cols < 0 || !fits(d.rows, d.cols)) return MXFP8_ERR_SHAPE;
  if ((d.s_row_pitch < 0 && d.s_row_pitch != MXFP8_SCALES_MFMA) ||
      (d.s_col_pitch < 0 && d.s_col_pitch != MXFP8_COLUMNWISE_T))
    return MXFP8_ERR_SHAPE;
  if (!mfma_order_ok(d.s_row_pitch, d.cols)) return MXFP8_ERR_SHAPE;
  if (d.rows == 0 || d.cols == 0) return MXFP8_OK;
  const bool row = d.q_row || d.s_row, col = d.q_col || d.s_col;
  if ((d.q_row == nullptr) != (d.s_row == nullptr)) return MXFP8_ERR_NULL;
  if ((d.q_col == nullptr) != (d.s_col == nullptr)) return MXFP8_ERR_NULL;
  if (!row && !col) return MXFP8_ERR_NO_OUTPUT;
  if (d.x == nullptr) return MXFP8_ERR_NULL;
  if (row && d.cols % MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
  if (col && d.rows % MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
  if (misaligned(d.x) || misaligned(d.q_row) || misaligned(d.s_row) ||
      misaligned(d.q_col) || misaligned(d.s_col))
    return MXFP8_ERR_ALIGN;
  if (row && d.s_row_pitch == MXFP8_SCALES_MFMA) {
    if (!col && !flat_blocks_fit(d.rows, d.cols)) return MXFP8_ERR_SHAPE;
  } else if (row && d.s_row_pitch) {
    if (d.s_row_pitch < d.cols / MXFP8_BLOCK || !fits(d.rows, d.s_row_pitch)) return MXFP8_ERR_SHAPE;
    if (!col && d.s_row_pitch != d.cols / MXFP8_BLOCK && !flat_blocks_fit(d.rows, d.cols))
      return MXFP8_ERR_SHAPE;
  }
  if (col && d.s_col_pitch == MXFP8_COLUMNWISE_T) {
    // the transposing tiles read 16-byte chunks of a row (no narrow path)
    if (d.cols % 8) return MXFP8_ERR_SHAPE;
  } else if (col && d.s_col_pitch) {
    if (d.s_col_pitch < d.cols || !fits(d.rows / MXFP8_BLOCK, d.s_col_pitch)) return MXFP8_ERR_SHAPE;
    // the tiles store 8 scale bytes at a time; rows of other lengths store bytes
    if (d.cols % 8 == 0 && d.s_col_pitch % 8) return MXFP8_ERR_ALIGN;
  }
  return MXFP8_OK;
}

mxfp8_status check_norm(const mxfp8_norm_desc& d) {
  if (d.rows < 0 || d.cols < 0 || d.rows > INT32_MAX || d.cols > INT32_MAX)
    return MXFP8_ERR_SHAPE;
  if (!isfinite(d.eps) || d.eps < 0.0f) return MXFP8_ERR_ARG;
  if (d.s_row_pitch < 0 && d.s_row_pitch != MXFP8_SCALES_MFMA) return MXFP8_ERR_SHAPE;
  if (!mfma_order_ok(d.s_row_pitch, d.cols)) return MXFP8_ERR_SHAPE;
  if (d.rows == 0 || d.cols == 0) return MXFP8_OK;
  if (!d.x || !d.gamma || !d.normed || !d.q_row || !d.s_row) return MXFP8_ERR_NULL;
  if (d.cols % MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
  if (misaligned(d.x) || misaligned(d.gamma) || misaligned(d.normed) ||
      misaligned(d.q_row) || misaligned(d.s_row))
    return MXFP8_ERR_ALIGN;
  if (d.s_row_pitch > 0 && (d.s_row_pitch < d.cols / MXFP8_BLOCK || !fits(d.rows, d.s_row_pitch)))
    return MXFP8_ERR_SHAPE;
  return MXFP8_OK;
}

mxfp8_status check_deq(const mxfp8_deq_desc& d) {
  if (d.axis != MXFP8_ROWWISE && d.axis != MXFP8_COLUMNWISE) return MXFP8_ERR_ARG;
  if (d.rows < 0 || d.cols < 0 || !fits(d.rows, d.cols)) return MXFP8_ERR_SHAPE;
  if (d.s_pitch < 0 && (d.s_pitch != MXFP8_SCALES_MFMA || d.axis != MXFP8_ROWWISE)) return MXFP8_ERR_SHAPE;
  if (!mfma_order_ok(d.s_pitch, d.cols)) return MXFP8_ERR_SHAPE;
  if (d.rows == 0 || d.cols == 0) return MXFP8_OK;
  if (!d.q || !d.s || !d.out) return MXFP8_ERR_NULL;
  if (d.axis == MXFP8_ROWWISE && d.cols % MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
  if (d.axis == MXFP8_COLUMNWISE && d.rows % MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
  if (misaligned(d.q) || misaligned(d.s) || misaligned(d.out)) return MXFP8_ERR_ALIGN;
  if (d.s_pitch == MXFP8_SCALES_MFMA) {
    if (!flat_blocks_fit(d.rows, d.cols)) return MXFP8_ERR_SHAPE;
  } else if (d.s_pitch) {
    const int64_t srows = d.axis == MXFP8_ROWWISE ? d.rows : d.rows / MXFP8_BLOCK;
    if (!fits(srows, d.s_pitch)) return MXFP8_ERR_SHAPE;
    if (d.axis == MXFP8_ROWWISE) {
      if (d.s_pitch < d.cols / MXFP8_BLOCK) return MXFP8_ERR_SHAPE;
      if (d.s_pitch != d.cols / MXFP8_BLOCK && !flat_blocks_fit(d.rows, d.cols)) return MXFP8_ERR_SHAPE;
    } else {
      if (d.s_pitch < d.cols) return MXFP8_ERR_SHAPE;
      if (d.cols % 8 == 0 && d.s_pitch % 8) return MXFP8_ERR_ALIGN;
    }
  }
  return MXFP8_OK;
}

mx::ScaleStride row_scale_stride(int64_t pitch, int64_t rows, int64_t w);

// Checks one product and fills its internal descriptor.
mxfp8_status check_gemm(const mxfp8_gemm_desc& d, mx::GemmDesc& g) {
  const int64_t M = d.M, N = d.N, K = d.K;
  if (M < 0 || N < 0 || K < 0 || !fits(M, K) || !fits(N, K) || !fits(M, N)) return MXFP8_ERR_SHAPE;
  if (d.out_pitch < 0 || (d.out_pitch && (d.out_pitch < N || !fits(M, d.out_pitch)))) return MXFP8_ERR_SHAPE;
  if ((d.sa_pitch < 0 && d.sa_pitch != MXFP8_SCALES_MFMA) || (d.sb_pitch < 0 && d.sb_pitch != MXFP8_SCALES_MFMA))
    return MXFP8_ERR_SHAPE;
  if (!mfma_order_ok(d.sa_pitch, K) || !mfma_order_ok(d.sb_pitch, K)) return MXFP8_ERR_SHAPE;
  g = mx::GemmDesc{};
  g.M = M;
  g.N = N;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (K == 0 || K % 128) return MXFP8_ERR_SHAPE;
  if (!d.qa || !d.sa || !d.qb || !d.sb || !d.out) return MXFP8_ERR_NULL;
  if (misaligned(d.qa) || misaligned(d.sa) || misaligned(d.qb) || misaligned(d.sb) || misaligned(d.out))
    return MXFP8_ERR_ALIGN;
  const int64_t kb = K / MXFP8_BLOCK;
  if (d.sa_pitch > 0 && (d.sa_pitch < kb || !fits(M, d.sa_pitch))) return MXFP8_ERR_SHAPE;
  if (d.sb_pitch > 0 && (d.sb_pitch < kb || !fits(N, d.sb_pitch))) return MXFP8_ERR_SHAPE;
  if ((d.sa_pitch > 0 && d.sa_pitch % 4) || (d.sb_pitch > 0 && d.sb_pitch % 4)) return MXFP8_ERR_ALIGN;
  // 64 x 32 outputs bound the smallest workgroup tile of every route, so this
  // keeps grid sizes and tile indices within 32 bits
  if (((M + 63) / 64) * ((N + 31) / 32) > kMaxGemmTiles) return MXFP8_ERR_SHAPE;
  g.qa = static_cast<const uint8_t*>(d.qa);
  g.sa = static_cast<const uint8_t*>(d.sa);
  g.qb = static_cast<const uint8_t*>(d.qb);
  g.sb = static_cast<const uint8_t*>(d.sb);
  g.K = K;
  g.sa_stride = row_scale_stride(d.sa_pitch, M, kb);
  g.sb_stride = row_scale_stride(d.sb_pitch, N, kb);
  g.out = d.out;
  g.out_ld = d.out_pitch ? d.out_pitch : N;
  return MXFP8_OK;
}

mxfp8_status hip_status(hipError_t e) { return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_HIP; }

// A tensor of a launch with the pitches of its scale planes.
template <class Desc, class Pitch>
struct Item {
  Desc d;
  Pitch p;
  bool pitched;  // some pitch differs from the compact one
};

template <class Args, class It>
void put(Args& a, int i, const It& it) {
  a.d[i] = it.d;
  if constexpr (Args::kPitched) a.p[i] = it.p;
}

// Packs non-empty tensors into argument blocks of at most Args::kMax entries
// and kMaxTasksPerLaunch tasks, launching each block as it fills.
template <class Args, class It, class TaskFn, class LaunchFn>
mxfp8_status run_groups(const std::vector<It>& items, TaskFn tasks, LaunchFn launch, Args& a) {
  a.n = 0;
  a.task_start[0] = 0;
  int64_t total = 0;
  bool cleared = false;
  for (const It& it : items) {
    const int64_t t = tasks(it.d);
    if (t == 0) continue;
    if (!cleared) {
      (void)hipGetLastError();  // report only errors raised by this call's launches
      cleared = true;
    }
    if (a.n == Args::kMax || total + t > kMaxTasksPerLaunch) {
      if (mxfp8_status st = hip_status(launch(a, total))) return st;
      a.n = 0;
      total = 0;
    }
    put(a, a.n, it);
    total += t;
    a.task_start[++a.n] = (int32_t)total;
  }
  if (a.n) return hip_status(launch(a, total));
  return MXFP8_OK;
}

// Runs the items through the compact argument block, or through the pitched
// one when any plane has a pitch of its own; a tensor with more tasks than
// one launch carries fails the call first.
template <class Compact, class Pitched, class It, class TaskFn, class LaunchFn>
mxfp8_status run_items(const std::vector<It>& items, TaskFn tasks, LaunchFn launch) {
  bool pitched = false;
  for (const It& it : items) {
    if (tasks(it.d) > kMaxTasksPerLaunch) return MXFP8_ERR_SHAPE;  // before any launch
    pitched |= it.pitched;
  }
  if (pitched) {
    Pitched a;
    return run_groups(items, tasks, [&](const Pitched& args, int64_t t) { return launch(args, t); }, a);
  }
  Compact a;
  return run_groups(items, tasks, [&](const Compact& args, int64_t t) { return launch(args, t); }, a);
}

mx::QuantDesc to_internal(const mxfp8_quant_desc& d) {
  mx::QuantDesc q;
  q.x = static_cast<const uint16_t*>(d.x);
  q.q_row = static_cast<uint8_t*>(d.q_row);
  q.s_row = static_cast<uint8_t*>(d.s_row);
  q.q_col = static_cast<uint8_t*>(d.q_col);
  q.s_col = static_cast<uint8_t*>(d.s_col);
  q.rows = d.rows;
  q.cols = d.cols;
  return q;
}

mx::NormDesc to_internal(const mxfp8_norm_desc& d) {
  mx::NormDesc n;
  n.x = static_cast<const uint16_t*>(d.x);
  n.gamma = static_cast<const uint16_t*>(d.gamma);
  n.normed = static_cast<uint16_t*>(d.normed);
  n.q = static_cast<uint8_t*>(d.q_row);
  n.s = static_cast<uint8_t*>(d.s_row);
  n.rows = (int32_t)d.rows;
  n.cols = (int32_t)d.cols;
  n.weight_offset = d.weight_offset;
  n.eps = d.eps;
  return n;
}

mx::DeqDesc to_internal(const mxfp8_deq_desc& d) {
  mx::DeqDesc q;
  q.q = static_cast<const uint8_t*>(d.q);
  q.s = static_cast<const uint8_t*>(d.s);
  q.out = d.out;
  q.rows = d.rows;
  q.cols = d.cols;
  q.axis = d.axis == MXFP8_COLUMNWISE ? 1 : 0;
  return q;
}

using QuantItem = Item<mx::QuantDesc, mx::QuantPitch>;
using NormItem = Item<mx::NormDesc, mx::ScaleStride>;
using DeqItem = Item<mx::DeqDesc, mx::ScaleStride>;

// Strides of a rowwise scale plane of `rows` rows and width w from its pitch
// argument (0 compact, MXFP8_SCALES_MFMA, or a row pitch).
mx::ScaleStride row_scale_stride(int64_t pitch, int64_t rows, int64_t w) {
  if (pitch == MXFP8_SCALES_MFMA) return {16, rows * 16};
  return {pitch ? pitch : w, 16};
}

bool compact(mx::ScaleStride st, int64_t w) { return st.row == w && st.grp == 16; }

QuantItem to_item(const mxfp8_quant_desc& d) {
  QuantItem it;
  it.d = to_internal(d);
  const int64_t wr = d.cols / MXFP8_BLOCK, wc = d.cols;
  const mx::ScaleStride sr = row_scale_stride(d.s_row_pitch, d.rows, wr);
  it.p.s_row = sr.row;
  it.p.s_grp = sr.grp;
  it.p.s_col = d.s_col_pitch > 0 ? d.s_col_pitch : wc;   // unused by the transposing tiles
  it.pitched = (d.s_row && !compact(sr, wr)) || (d.s_col && it.p.s_col != wc);
  return it;
}

NormItem to_item(const mxfp8_norm_desc& d) {
  NormItem it;
  it.d = to_internal(d);
  const int64_t w = d.cols / MXFP8_BLOCK;
  it.p = row_scale_stride(d.s_row_pitch, d.rows, w);
  it.pitched = !compact(it.p, w);
  return it;
}

DeqItem to_item(const mxfp8_deq_desc& d) {
  DeqItem it;
  it.d = to_internal(d);
  if (d.axis == MXFP8_COLUMNWISE) {
    it.p = {d.s_pitch ? d.s_pitch : d.cols, 16};
    it.pitched = it.p.row != d.cols;
  } else {
    const int64_t w = d.cols / MXFP8_BLOCK;
    it.p = row_scale_stride(d.s_pitch, d.rows, w);
    it.pitched = !compact(it.p, w);
  }
  return it;
}

// A grouped quantize: every descriptor, and every tensor's task count, is
// checked before the first launch; tensors whose columnwise plane is stored
// transposed go to their own tiles.
template <class TaskFn, class TaskFnT, class LaunchFn, class LaunchFnT>
mxfp8_status quantize_lists(const mxfp8_quant_desc* descs, int32_t n, void* stream, TaskFn tasks,
                            TaskFnT tasks_t, LaunchFn launch, LaunchFnT launch_t) {
  if (n < 0) return MXFP8_ERR_ARG;
  if (n == 0) return MXFP8_OK;
  if (!descs) return MXFP8_ERR_NULL;
  std::vector<QuantItem> v, vt;
  v.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    if (mxfp8_status st = check_quant(descs[i])) return st;
    (col_t(descs[i]) ? vt : v).push_back(to_item(descs[i]));
  }
  for (const QuantItem& it : vt)
    if (tasks_t(it.d) > kMaxTasksPerLaunch) return MXFP8_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mxfp8_status st = run_items<mx::QuantArgs, mx::QuantArgsPitched>(
          v, tasks, [&](const auto& args, int64_t t) { return launch(args, t, s); }))
    return st;
  return run_items<mx::QuantArgs, mx::QuantArgsPitched>(
      vt, tasks_t, [&](const auto& args, int64_t t) { return launch_t(args, t, s); });
}

}  // namespace

extern "C" {

int mxfp8_abi_version(void) { return MXFP8_ABI_VERSION; }

const char* mxfp8_status_string(mxfp8_status status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_ERR_NULL: return "a required pointer is NULL or a plane is half specified";
    case MXFP8_ERR_SHAPE: return "bad shape: negative size, partial 32-element block or size limit";
    case MXFP8_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MXFP8_ERR_NO_OUTPUT: return "neither the rowwise nor the columnwise plane was requested";
    case MXFP8_ERR_ARG: return "bad argument: enum value, group count or eps";
    case MXFP8_ERR_HIP: return "the HIP runtime refused the launch";
  }
  return "unknown status";
}

mxfp8_status mxfp8_quantize_grouped(const mxfp8_quant_desc* descs, int32_t n, void* stream) {
  return quantize_lists(descs, n, stream, mx::quant_tasks, mx::quant_colt_tasks,
                        [](const auto& args, int64_t t, hipStream_t s) { return mx::launch_quantize(args, t, s); },
                        [](const auto& args, int64_t t, hipStream_t s) { return mx::launch_quantize_colt(args, t, s); });
}

mxfp8_status mxfp8_quantize_f32_grouped(const mxfp8_quant_desc* descs, int32_t n,
                                        void* stream) {
  return quantize_lists(
      descs, n, stream, mx::quant_f32_tasks, mx::quant_f32_colt_tasks,
      [](const auto& args, int64_t t, hipStream_t s) { return mx::launch_quantize_f32(args, t, s); },
      [](const auto& args, int64_t t, hipStream_t s) { return mx::launch_quantize_f32_colt(args, t, s); });
}

mxfp8_status mxfp8_quantize_f32(const void* x, int64_t rows, int64_t cols, void* q_row,
                                void* s_row, void* q_col, void* s_col, void* stream) {
  mxfp8_quant_desc d = {x, rows, cols, q_row, s_row, q_col, s_col, 0, 0};
  return mxfp8_quantize_f32_grouped(&d, 1, stream);
}

mxfp8_status mxfp8_quantize(const void* x, int64_t rows, int64_t cols, void* q_row,
                            void* s_row, void* q_col, void* s_col, void* stream) {
  mxfp8_quant_desc d = {x, rows, cols, q_row, s_row, q_col, s_col, 0, 0};
  return mxfp8_quantize_grouped(&d, 1, stream);
}

mxfp8_status mxfp8_rmsnorm_quantize_grouped(const mxfp8_norm_desc* descs, int32_t n,
                                            void* stream) {
  if (n < 0) return MXFP8_ERR_ARG;
  if (n == 0) return MXFP8_OK;
  if (!descs) return MXFP8_ERR_NULL;
  std::vector<NormItem> v;
  v.reserve(n);
  int64_t max_cols = 0, total_rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (mxfp8_status st = check_norm(descs[i])) return st;
    v.push_back(to_item(descs[i]));
    if (descs[i].rows > 0 && descs[i].cols > 0) {
      if (descs[i].cols > max_cols) max_cols = descs[i].cols;
      total_rows += descs[i].rows;
    }
  }
  const int variant = mx::norm_variant(max_cols, total_rows);
  const int rpt = mx::norm_rows_per_task(total_rows, variant);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run_items<mx::NormArgs, mx::NormArgsPitched>(
      v, [rpt](const mx::NormDesc& d) -> int64_t { return d.cols ? (d.rows + rpt - 1) / rpt : 0; },
      [&](const auto& args, int64_t t) { return mx::launch_rmsnorm_quantize(args, t, variant, rpt, s); });
}

mxfp8_status mxfp8_rmsnorm_quantize(const void* x, const void* gamma, float weight_offset,
                                    float eps, int64_t rows, int64_t cols, void* normed,
                                    void* q_row, void* s_row, void* stream) {
  mxfp8_norm_desc d = {x, gamma, weight_offset, eps, rows, cols, normed, q_row, s_row, 0};
  return mxfp8_rmsnorm_quantize_grouped(&d, 1, stream);
}

mxfp8_status mxfp8_dequantize_grouped(const mxfp8_deq_desc* descs, int32_t n,
                                      mxfp8_out_dtype out_dtype, void* stream) {
  if (n < 0) return MXFP8_ERR_ARG;
  if (out_dtype != MXFP8_OUT_F32 && out_dtype != MXFP8_OUT_BF16) return MXFP8_ERR_ARG;
  if (n == 0) return MXFP8_OK;
  if (!descs) return MXFP8_ERR_NULL;
  std::vector<DeqItem> v;
  v.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    if (mxfp8_status st = check_deq(descs[i])) return st;
    v.push_back(to_item(descs[i]));
  }
  const int32_t bf16 = out_dtype == MXFP8_OUT_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run_items<mx::DeqArgs, mx::DeqArgsPitched>(v, mx::deq_tasks, [&](auto args, int64_t t) {
    args.out_bf16 = bf16;
    return mx::launch_dequantize(args, t, s);
  });
}

mxfp8_status mxfp8_gemm(const void* qa, const void* sa, const void* qb, const void* sb,
                        int64_t M, int64_t N, int64_t K, int64_t sa_pitch, int64_t sb_pitch,
                        void* out, int64_t out_pitch, mxfp8_out_dtype out_dtype, void* stream) {
  if (out_dtype != MXFP8_OUT_F32 && out_dtype != MXFP8_OUT_BF16) return MXFP8_ERR_ARG;
  const mxfp8_gemm_desc d = {qa, sa, qb, sb, M, N, K, sa_pitch, sb_pitch, out, out_pitch};
  mx::GemmDesc g;
  if (mxfp8_status st = check_gemm(d, g)) return st;
  if (M == 0 || N == 0) return MXFP8_OK;
  (void)hipGetLastError();
  return hip_status(mx::launch_gemm(g.qa, g.sa, g.qb, g.sb, g.M, g.N, g.K, g.sa_stride, g.sb_stride, g.out,
                                    g.out_ld, out_dtype == MXFP8_OUT_BF16, static_cast<hipStream_t>(stream)));
}

mxfp8_status mxfp8_gemm_grouped(const mxfp8_gemm_desc* descs, int32_t n, mxfp8_out_dtype out_dtype,
                                void* stream) {
  if (n < 0 || (out_dtype != MXFP8_OUT_F32 && out_dtype != MXFP8_OUT_BF16)) return MXFP8_ERR_ARG;
  if (n == 0) return MXFP8_OK;
  if (!descs) return MXFP8_ERR_NULL;
  std::vector<mx::GemmDesc> v(n);
  for (int32_t i = 0; i < n; ++i)
    if (mxfp8_status st = check_gemm(descs[i], v[i])) return st;
  (void)hipGetLastError();
  return hip_status(mx::launch_gemm_grouped(v.data(), n, out_dtype == MXFP8_OUT_BF16,
                                            static_cast<hipStream_t>(stream)));
}

mxfp8_status mxfp8_dequantize(const void* q, const void* s, int64_t rows, int64_t cols,
                              mxfp8_axis axis, void* out, mxfp8_out_dtype out_dtype,
                              void* stream) {
  mxfp8_deq_desc d = {q, s, rows, cols, axis, out, 0};
  return mxfp8_dequantize_grouped(&d, 1, out_dtype, stream);
}

}  // extern "C"
