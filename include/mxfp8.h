/*
 * mxfp8.h - C ABI of libmxfp8, an MXFP8 block-quantization library for AMD
 * Instinct MI355X (gfx950).
 *
 * What the library computes.  A bf16 tensor is cut into blocks of 32 elements
 * (Megatron-Core quantized_dbuffer page, "Data", _MXFP8_BLOCK_SIZE).  Each
 * block gets one float8_e8m0fnu scale byte S and each element one
 * float8_e4m3fn byte (Mojo DistributedAllGatherRMSNormQuantMXFP8 page,
 * "Parameters", quant_dtype and scales_dtype).  The pages leave the scale
 * rule and the rounding open; the library follows OCP MX v1.0:
 *
 *     S = clamp(floor(log2(amax)) - 8 + 127, 0, 254)   (amax: block max |x|)
 *     S = 0x00 for an all-zero block, 0xFF for a block holding a NaN or an
 *         infinity (then every element byte is sign | 0x7F)
 *     q = e4m3fn(x * 2^(127 - S)), round to nearest even, saturate at +-448,
 *         sign of zero kept.
 *
 * Two planes can be produced from one read of the input:
 *   rowwise:    blocks x[r, 32j .. 32j+31]; scales [rows, cols/32]
 *               (Mojo page, "Args", outputs_scale);
 *   columnwise: blocks x[32i .. 32i+31, c]; scales [rows/32, cols] (one
 *               columnwise scale row covers a 32-row block: quantized_dbuffer
 *               page, API, _block_atomic_to_flat).
 * Both data planes are [rows, cols] row-major, the input's own layout, not
 * transposed (quantized_dbuffer page, Functions: _rowwise_scale_layout and
 * _columnwise_scale_layout derive both scale layouts from one data layout).
 * By default every plane is compact and unswizzled, with no padding
 * (quantized_dbuffer page, API: QuantizedDBuffer and get_tensor_view).  A
 * scale plane may instead be written into, and read from, a padded
 * allocation whose rows are a caller-chosen pitch apart (see "Scale pitches"
 * below).
 *
 * Conventions shared by every entry point:
 *   - Tensors are 2D, row-major and contiguous.  rows and cols count
 *     elements.  Element types: bf16 for x / gamma / normed, uint8 for e4m3
 *     and e8m0 bytes, float32 or bf16 for dequantized output.
 *   - Every pointer is a device pointer (hipMalloc or equivalent) and must be
 *     16-byte aligned.  The caller owns all memory.  The library never
 *     allocates, frees or synchronizes; outputs are written in place into the
 *     caller's persistent buffers, so captured HIP graphs keep valid
 *     pointers (Megatron-Core quantization.utils page, quantize_params_to_mxfp8:
 *     results are copied into persistent buffers for graph captures).
 *     Inputs are read only.
 *   - stream is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *     it and the call returns at once; results are ready when the stream is.
 *   - Every argument is checked before anything is launched, so a call that
 *     returns an argument error has enqueued nothing.  (MXFP8_ERR_HIP from a
 *     grouped call long enough to need several launches can follow launches
 *     already enqueued.)  rows == 0 or cols == 0 is a no-op that returns
 *     MXFP8_OK.  Device faults surface at the caller's
 *     next synchronization, as with any HIP work.
 *   - The library keeps no state: calls may come from any thread.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP8_ABI_VERSION 4
#define MXFP8_BLOCK 32
/* Descriptors handled by one kernel launch in the grouped calls; longer
 * lists are processed in consecutive launches of at most this many.  A list
 * in which any scale plane has a pitch of its own goes in launches of at most
 * MXFP8_PITCHED_GROUP_PER_LAUNCH. */
#define MXFP8_GROUP_PER_LAUNCH 64
#define MXFP8_PITCHED_GROUP_PER_LAUNCH 32
/* A rowwise scale pitch of this value selects the MFMA order (see "Scale
 * pitches"). */
#define MXFP8_SCALES_MFMA ((int64_t)-1)
/* A columnwise scale pitch of this value in a quantize descriptor stores the
 * columnwise plane transposed (see "Transposed columnwise plane"). */
#define MXFP8_COLUMNWISE_T ((int64_t)-2)

typedef enum {
    MXFP8_OK = 0,
    MXFP8_ERR_NULL = 1,      /* a required pointer is NULL, or a plane's data /
                                scale pointers are not both set or both NULL */
    MXFP8_ERR_SHAPE = 2,     /* negative size, partial block, or size limit
                                (a byte count above 2^61; a tensor needing
                                more than the 2^30 tasks of one launch, which
                                takes 2^40 elements or more; a product of
                                more than 2^28 tiles of 64 x 32 outputs) */
    MXFP8_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
    MXFP8_ERR_NO_OUTPUT = 4, /* neither plane requested */
    MXFP8_ERR_ARG = 5,       /* bad enum value, n < 0, or a non-finite eps */
    MXFP8_ERR_HIP = 6        /* the HIP runtime refused the launch */
} mxfp8_status;

typedef enum { MXFP8_ROWWISE = 0, MXFP8_COLUMNWISE = 1 } mxfp8_axis;
typedef enum { MXFP8_OUT_F32 = 0, MXFP8_OUT_BF16 = 1 } mxfp8_out_dtype;

/* MXFP8_ABI_VERSION of the built library. */
int mxfp8_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *mxfp8_status_string(mxfp8_status status);

/*
 * mxfp8_quantize - one read of x, one or both planes written.
 *
 * Quantizes a local weight or activation shard into its planes
 * (quantized_dbuffer page, API, QuantizedDBuffer.quantize_; quantization.utils
 * page, mm_mxfp8 quantizes the bf16 activation on the fly).  The pair
 * (q_row, s_row) selects the rowwise plane and (q_col, s_col) the columnwise
 * plane, like the rowwise / columnwise usages of the quantizer
 * (quantized_dbuffer page, _get_quantizer and planes_for).
 *
 *   x      bf16 [rows, cols]
 *   q_row  uint8 e4m3 [rows, cols]     s_row  uint8 e8m0 [rows, cols/32]
 *   q_col  uint8 e4m3 [rows, cols]     s_col  uint8 e8m0 [rows/32, cols]
 *
 * A plane whose two pointers are NULL is not requested; one NULL and one set
 * is MXFP8_ERR_NULL; both planes NULL is MXFP8_ERR_NO_OUTPUT.  A rowwise
 * request needs cols % 32 == 0, a columnwise request rows % 32 == 0
 * (MXFP8_ERR_SHAPE otherwise).  A columnwise-only request with cols % 8 != 0
 * runs a narrow path of element-sized accesses (the same bytes, at a fraction
 * of the tiles' bandwidth).
 */
mxfp8_status mxfp8_quantize(const void *x, int64_t rows, int64_t cols,
                            void *q_row, void *s_row, void *q_col, void *s_col,
                            void *stream);

/*
 * mxfp8_quantize_f32 - mxfp8_quantize for a float32 tensor.
 *
 * Quantizes a float32 master weight straight into its planes
 * (quantized_dbuffer page, QuantizedDBuffer.quantize_ on a local master
 * shard): the same blocks, scale rule, rounding and plane layouts as
 * mxfp8_quantize, applied to the float32 values.  x is float32 [rows, cols];
 * every other argument and rule is mxfp8_quantize's.
 */
mxfp8_status mxfp8_quantize_f32(const void *x, int64_t rows, int64_t cols,
                                void *q_row, void *s_row, void *q_col,
                                void *s_col, void *stream);

/*
 * mxfp8_rmsnorm_quantize - RMSNorm, then the rowwise plane of its bf16 output.
 *
 * The fused norm-and-quantize of the Mojo DistributedAllGatherRMSNormQuantMXFP8
 * page (execute; "Args": outputs_normed, outputs_quant, outputs_scale, gammas,
 * epsilons, weight_offsets) on one GPU's rows, without the all-gather:
 *
 *   normed[r, c] = bf16( x[r, c] / sqrt(mean_c(x[r, :]^2) + eps)
 *                        * (gamma[c] + weight_offset) )
 *
 * rounded once to bf16 (nearest even); (q_row, s_row) is then exactly
 * mxfp8_quantize's rowwise plane of those normed bf16 values (the page's
 * execute: the quantize reads the same bf16 that lands in outputs_normed, so
 * it is byte-identical to a standalone quantize).
 *
 *   x, normed  bf16 [rows, cols]     gamma  bf16 [cols]
 *   q_row      uint8 [rows, cols]    s_row  uint8 [rows, cols/32]
 *
 * Precision and range.  sum_c x[r, c]^2 is accumulated in float32 when that
 * sum lies in [2^-60, 2^120], and otherwise again in float64, where the
 * square of every bf16 value is exact and no row sum can overflow or
 * underflow; rstd = 1 / sqrt(sum / cols + eps) is then within a few float32
 * roundings of exact.  The product x * rstd * (gamma + weight_offset) is
 * taken in float32 (gamma + weight_offset is one float32 addition).  Every finite bf16 row, from
 * subnormals to the largest finite values, with any finite eps >= 0, gives
 * normed values within one bf16 rounding (plus a few float32 roundings) of
 * the exact formula.  Rows the formula leaves undefined follow IEEE
 * arithmetic:
 *   - a row of zeros with eps == 0 is 0 / 0: every normed value is NaN, so
 *     every scale byte of the row is 0xFF and every element byte sign | 0x7F;
 *     with eps > 0 a row of zeros gives zeros (with x's sign);
 *   - a row holding +-Inf and no NaN has rstd = 0: its finite values give
 *     +-0, its infinities NaN;
 *   - a row holding a NaN is NaN everywhere.
 * The sign bit of a NaN produced this way is not specified.  A result whose
 * magnitude exceeds bf16's range (a huge gamma) is +-Inf.
 *
 * All pointers are required; cols % 32 == 0; eps must be finite and >= 0.
 */
mxfp8_status mxfp8_rmsnorm_quantize(const void *x, const void *gamma,
                                    float weight_offset, float eps,
                                    int64_t rows, int64_t cols, void *normed,
                                    void *q_row, void *s_row, void *stream);

/*
 * mxfp8_dequantize - values of one plane: out = e4m3(q) * 2^(S - 127).
 *
 * The check that compares a dequantized tensor with a fresh quantize
 * (quantization.utils page, _verify_te_to_mcore_mxfp8_conversion) needs it.
 * axis picks the scale layout: MXFP8_ROWWISE s [rows, cols/32] (cols % 32 ==
 * 0), MXFP8_COLUMNWISE s [rows/32, cols] (rows % 32 == 0; cols % 8 != 0
 * takes a narrow path of element-sized accesses).
 * out is float32 or bf16 [rows, cols]: the exact value rounded to nearest
 * even.  Float32 results are exact (values from 2^-136 up), except that
 * scale bytes above 246, which no quantize of bf16 input produces, can push a
 * value past float32's range, giving +-inf; bf16 results are exact except
 * below 2^-133.  Scale 0xFF or element 0x7F / 0xFF gives NaN.
 */
mxfp8_status mxfp8_dequantize(const void *q, const void *s, int64_t rows,
                              int64_t cols, mxfp8_axis axis, void *out,
                              mxfp8_out_dtype out_dtype, void *stream);

/*
 * Scale pitches - scale planes in a consumer's padded allocation.
 *
 * Consumers may keep scales in a larger, padded allocation ("TE's physical
 * allocation shape": quantized_dbuffer page, _pad_rowwise_scale and
 * _pad_columnwise_scale; TE-only padding is added when a wrapper for compute
 * is materialized).  The pages give neither the padded shape nor any other
 * consumer order, so the library takes the plainest reading that covers
 * them: the scale plane's rows are `pitch` bytes apart instead of the plane's
 * width, and the kernels write (or read) the scale bytes there directly, in
 * the same pass, with no extra copy.  Bytes between the end of a scale row and
 * the next row's start, and rows past the plane, are never written or read.
 * A pitch of 0 means compact.  Required:
 *
 *   rowwise scales     pitch >= cols/32 (any value), and rows * cols/32 < 2^32
 *                      when the rowwise plane is the only one requested;
 *   columnwise scales  pitch >= cols, and a multiple of 8 when cols % 8 == 0
 *                      (MXFP8_ERR_ALIGN);
 *   matrix product     pitch >= K/32 and a multiple of 4.
 *
 * A pitch below the plane's width is MXFP8_ERR_SHAPE.
 *
 * The MFMA order (rowwise scale planes only; pitch MXFP8_SCALES_MFMA).  The
 * Mojo page's Limitations name a preshuffled scale order that one AMD matrix
 * kernel needs, without defining it; the library's reading is the order in
 * which its own matrix product feeds the scale operand of the block-scaled
 * MFMA.  A [rows, cols] tensor's scales are cut into groups of 512 columns (16
 * blocks); group g holds, row after row, each row's 16 scale bytes of that
 * group: block b of row r sits at byte (b / 16) * rows * 16 + r * 16 + b % 16.
 * The plane has the compact plane's size, rows * cols/32 bytes.  Required:
 * cols % 512 == 0 (for the matrix product, K % 512 == 0), else
 * MXFP8_ERR_SHAPE; a columnwise plane with this pitch is MXFP8_ERR_SHAPE.
 * Quantize, the fused RMSNorm and dequantize write or read it in their one
 * pass; the matrix product loads each 512-deep group's scales of 64 rows as
 * one contiguous 1 KiB run instead of 64 separate 16-byte pieces.
 */

/*
 * Transposed columnwise plane (quantize descriptors only; s_col_pitch
 * MXFP8_COLUMNWISE_T).  The columnwise plane's blocks run down the columns of
 * x (quantized_dbuffer page, _block_atomic_to_flat), and the pages store it
 * in x's layout.  Each training phase installs the planes it uses
 * (quantized_dbuffer page, update_mxfp8_tensor); the library's reading is
 * the usual one, the columnwise planes serve the backward products, which
 * contract over the rows of x: the input gradient takes the weight's
 * columnwise plane, the weight gradient both activations'.  mxfp8_gemm, like
 * gfx950's block-scaled MFMA whose operand fragments hold consecutive k of
 * one row, reads operands whose 32-element blocks are contiguous.  With this
 * pitch the quantize writes the columnwise plane in that order, in the same
 * pass, with the same bytes:
 *
 *   q_col  uint8 e4m3 [cols, rows]   q_col[c, r] = the e4m3 byte of x[r, c]
 *   s_col  uint8 e8m0 [cols, rows/32] s_col[c, b] = the scale of rows
 *                                     32 b .. 32 b + 31 of column c
 *
 * so (q_col, s_col) is a rowwise plane of x^T, ready to be an operand of
 * mxfp8_gemm (K = rows) or to be dequantized as a rowwise plane of
 * [cols, rows].  Required: rows % 32 == 0 and cols % 8 == 0
 * (MXFP8_ERR_SHAPE otherwise); the rowwise plane, if requested, follows its
 * usual rules, pitches and MFMA order included.  mxfp8_quantize_grouped and
 * mxfp8_quantize_f32_grouped (a single tensor is a grouped call with
 * n == 1; a float32 master weight's transposed plane serves the input
 * gradient).  A grouped list that mixes
 * transposed and untransposed columnwise planes takes one launch sequence for
 * each kind.
 */

/*
 * mxfp8_gemm - out[M, N] = A . B^T from two rowwise planes.
 *
 * The consumer the planes exist for: a linear layer that quantizes its bf16
 * activation on the fly and multiplies it by a pre-quantized weight
 * (quantization.utils page, mm_mxfp8), on gfx950's block-scaled MFMA, which
 * takes the plain rank-2 scale layout (Mojo page, Limitations: the scale
 * layout block_scaled_matmul_amd takes as a_scales).
 *
 *   qa  uint8 e4m3 [M, K]   sa  uint8 e8m0 [M, K/32]   (A rowwise plane)
 *   qb  uint8 e4m3 [N, K]   sb  uint8 e8m0 [N, K/32]   (B rowwise plane, e.g.
 *                                                        a weight [out, in])
 *   out float32 or bf16 [M, N]
 *
 * out[m, n] = sum_k A[m, k] B[n, k] with the element and scale values of the
 * planes, accumulated by the matrix cores, then rounded to the output type.
 * Each 64-deep step cuts the products of every group of 8 consecutive k
 * toward zero 13 bits below the group's largest exponent sum, and rounds the
 * group sums and the running sum 24 bits below the largest of them, then to
 * float32.  The float32 result is within
 *   sum_g sum_{k in g} min(|p_k|, 2^(E_g - 13)) + (11 n + 3) 2^-24 sum_k |p_k|
 * of the exact sum, p_k = A[m, k] B[n, k], 2^E_g the group's largest
 * exponent sum, n = K / 64 rounded up to a multiple of 8.  K must be a
 * positive multiple of 128 (MXFP8_ERR_SHAPE otherwise); M == 0 or N == 0 is
 * a no-op.  sa_pitch and sb_pitch are the bytes between scale rows of A and
 * of B (0: compact, K/32), or MXFP8_SCALES_MFMA for a plane in the MFMA order
 * (see "Scale pitches").  out_pitch is the number of elements between output
 * rows (0: N; else at least N, MXFP8_ERR_SHAPE otherwise), so the product can
 * fill a column slice of a wider matrix; elements past column N of a row are
 * never written.
 */
mxfp8_status mxfp8_gemm(const void *qa, const void *sa, const void *qb,
                        const void *sb, int64_t M, int64_t N, int64_t K,
                        int64_t sa_pitch, int64_t sb_pitch, void *out,
                        int64_t out_pitch, mxfp8_out_dtype out_dtype,
                        void *stream);

/*
 * Grouped calls: one launch over a list of independent 2D tensors of any
 * shapes, such as the experts of an MoE layer (quantized_dbuffer page,
 * QuantizedDBuffer.empty takes a list of logical 2D shapes; quantization.utils
 * page, resolve_mxfp8_backend serves grouped-MoE GEMMs).  Each descriptor
 * follows the rules of the matching single call and the results equal n
 * single calls.  descs is a host array of n entries, read before the call
 * returns.  n == 0 is a no-op; n < 0 is MXFP8_ERR_ARG.  Each launch takes at
 * most MXFP8_GROUP_PER_LAUNCH descriptors.  The descriptors also carry scale
 * pitches (0: compact; see "Scale pitches"), so a single tensor with padded
 * scale planes is a grouped call with n == 1.
 */
typedef struct {
    const void *x;
    int64_t rows, cols;
    void *q_row, *s_row; /* both NULL: rowwise plane not requested */
    void *q_col, *s_col; /* both NULL: columnwise plane not requested */
    int64_t s_row_pitch, s_col_pitch; /* bytes between scale rows; 0: compact */
} mxfp8_quant_desc;

typedef struct {
    const void *x, *gamma;
    float weight_offset, eps;
    int64_t rows, cols;
    void *normed, *q_row, *s_row;
    int64_t s_row_pitch; /* bytes between scale rows; 0: compact */
} mxfp8_norm_desc;

typedef struct {
    const void *q, *s;
    int64_t rows, cols;
    mxfp8_axis axis;
    void *out;
    int64_t s_pitch; /* bytes between scale rows; 0: compact */
} mxfp8_deq_desc;

typedef struct {
    const void *qa, *sa; /* A rowwise plane [M, K], scales [M, K/32] */
    const void *qb, *sb; /* B rowwise plane [N, K], scales [N, K/32] */
    int64_t M, N, K;
    int64_t sa_pitch, sb_pitch; /* as in mxfp8_gemm */
    void *out;                  /* [M, N] */
    int64_t out_pitch;          /* elements between output rows; 0: N */
} mxfp8_gemm_desc;

mxfp8_status mxfp8_quantize_grouped(const mxfp8_quant_desc *descs, int32_t n,
                                    void *stream);
/* Grouped mxfp8_quantize_f32: each descriptor's x points to float32. */
mxfp8_status mxfp8_quantize_f32_grouped(const mxfp8_quant_desc *descs, int32_t n,
                                        void *stream);
mxfp8_status mxfp8_rmsnorm_quantize_grouped(const mxfp8_norm_desc *descs,
                                            int32_t n, void *stream);
mxfp8_status mxfp8_dequantize_grouped(const mxfp8_deq_desc *descs, int32_t n,
                                      mxfp8_out_dtype out_dtype, void *stream);

/*
 * mxfp8_gemm_grouped - n independent products out = A . B^T, such as the
 * experts of an MoE layer, each with its own activation rows, weight,
 * shape and output (quantization.utils page, resolve_mxfp8_backend: grouped
 * MoE products take MXFP8 expert weights).  Each descriptor follows
 * mxfp8_gemm's rules and its result meets mxfp8_gemm's accuracy statement;
 * out_dtype applies to all.  The products share launches, so even a list of
 * one-token products fills the GPU: products of at most 32 rows (and of at
 * most 128 with K < 512) one workgroup per 32 output columns, their results
 * equal to mxfp8_gemm's bit for bit; larger ones ring tiles, whose 64-deep
 * steps may be summed in another order than mxfp8_gemm's; more than 128
 * rows with K < 512 run as single calls.  Every descriptor is checked
 * before the first launch; n == 0 is a no-op, n < 0 is MXFP8_ERR_ARG.
 */
mxfp8_status mxfp8_gemm_grouped(const mxfp8_gemm_desc *descs, int32_t n,
                                mxfp8_out_dtype out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
