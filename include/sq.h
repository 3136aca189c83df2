/*
 * sq.h -- C ABI of libsq.so: the SmoothQuant W8A8 quantized linear
 * Y = X W^T on MI355X (gfx950).
 *
 * The method is the one of the page "w8a8_smoothquant.py" (BiGRU_T_version,
 * src/bigru_t/quantization): activations X (M x K) and weights W (N x K, the
 * nn.Linear layout) are rebalanced per input channel j by a smoothing factor
 *     s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)        (module docstring,
 *                                                        calibrate_smoothquant)
 * so that X~ = X / s and W~ = W * s give the same product. W~ is quantised
 * to int8 once with one scale per output channel, X~ is quantised to int8 per
 * token on every call, and the integer product is scaled back:
 *     y[t, o] = acc[t, o] * scale_x[t] * scale_w[o] + bias[o],
 *     acc[t, o] = sum_j xq[t, j] * wq[o, j]  (int32).
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers owned by the caller. The
 *     library allocates nothing, frees nothing and never synchronises: work
 *     is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     the call returns at once. Outputs are valid when the stream reaches
 *     that point. Calls on different streams that write the same buffer race.
 *   - Row-major, dense: X is [m][k], W and wq are [n][k], Y is [m][n]
 *     (wq and xq may instead be tiled, below).
 *   - k must be a positive multiple of 16. Every pointer to a [.][k] array
 *     must be 16-byte aligned. m and n may be any size from 1 to
 *     SQ_MAX_ROWS (a call with m == 0 is a no-op that touches nothing); the
 *     products (sq_w8a8_gemm*, sq_w8a8_linear, sq_reference_linear) also
 *     return SQ_ERR_SHAPE when ceil(m / 128) * ceil(n / 128) exceeds
 *     SQ_MAX_TILES (an output of more than about 1.4e11 elements).
 *   - Floating-point input types: SQ_F32 or SQ_BF16 (widened exactly to
 *     fp32). All scale and code arithmetic is IEEE binary32 with
 *     round-to-nearest-even, every quotient one correctly rounded division
 *     (or a scheme proven to give the same result); codes are
 *     round-half-to-even of that quotient, clamped to [-128, 127].
 *   - The floor 1e-8 (the binary32 value 0x322BCC77) is applied to every
 *     maximum that is divided by, and to s.
 *   - Inputs (activations, weights, bias) must be finite, and every
 *     quotient x / s finite; the method is not defined on infinities or
 *     NaNs (their maxima and codes are left unspecified here).
 *   - Layout: the [.][k] int8 code arrays are row-major, or in 16 x 64
 *     tiles for the entry points named *_tiled (see sq_tiled_bytes).
 *   - Errors: arguments are checked before anything is enqueued; a negative
 *     status means nothing was enqueued. SQ_ERR_HIP means a launch failed
 *     (earlier launches of the same call may have run). No exception or
 *     abort ever crosses this ABI.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_WARN_UNCALIBRATED = 1, /* success; s was set to 1 (no calibration data) */
    SQ_ERR_ARG = -1,          /* null pointer, alpha outside [0, 1], bad enum */
    SQ_ERR_SHAPE = -2,        /* negative / zero size where one is required, or too large */
    SQ_ERR_DTYPE = -3,        /* unsupported input or output type */
    SQ_ERR_ALIGN = -4,        /* k not a multiple of 16, or a pointer not 16-byte aligned */
    SQ_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
    SQ_ERR_HIP = -6           /* a HIP launch reported an error */
} sq_status;

typedef enum {
    SQ_F32 = 0,   /* IEEE binary32 */
    SQ_BF16 = 1,  /* bfloat16 */
    SQ_I32 = 2    /* int32: output only, the raw integer accumulators */
} sq_dtype;

/* Largest k the kernels accept (one token row of X~ is held on chip). */
#define SQ_MAX_K 16384
/* Largest row count (m, n, rows) any entry point accepts: the kernels count
 * rows, tiles and row groups in 32-bit integers. */
#define SQ_MAX_ROWS (1LL << 30)
/* Largest number of 128 x 128 output tiles of one product. */
#define SQ_MAX_TILES ((1LL << 23) - 1)
/* Most calibration batches one sq_calibrate_batches call takes. */
#define SQ_MAX_CALIB_BATCHES 8

/*
 * sq_calibrate -- running per-input-channel max of |X| over calibration rows.
 * Follows SmoothQuantW8A8.calibrate (page "w8a8_smoothquant.py"): the buffer
 * starts at zero once and every batch folds max_r |x[r][j]| into it; the
 * result is independent of how the rows are split into batches or ordered.
 *   x               [rows][k] in xt (F32 or BF16), 16-byte aligned
 *   running_max_abs [k] fp32, in/out; caller zero-fills it before the first
 *                   batch; values stay non-negative (no floor is applied here)
 * Returns SQ_OK, or SQ_ERR_* before launching. rows == 0 is a no-op.
 */
sq_status sq_calibrate(const void* x, sq_dtype xt, int64_t rows, int64_t k,
                       float* running_max_abs, void* stream);

/*
 * sq_calibrate_first -- the first batch of a calibration: the running max
 * starts from this batch alone, whatever the buffer held,
 *   running_max_abs[j] = max_r |x[r][j]|       (0 for rows == 0)
 * i.e. sq_calibrate on a zero-filled buffer, without the caller's fill
 * (one launch when the batch fits one row group of the column max, up to
 * 128 rows). Later batches go through sq_calibrate. Arguments as
 * sq_calibrate; x may be NULL when rows == 0.
 */
sq_status sq_calibrate_first(const void* x, sq_dtype xt, int64_t rows, int64_t k,
                             float* running_max_abs, void* stream);

/*
 * sq_calibrate_batches -- several calibration batches at once. The running
 * max of SmoothQuantW8A8.calibrate (page "w8a8_smoothquant.py") is a max
 * over every calibration row, so batches already resident on the device can
 * be folded in together, with the same result bits as one sq_calibrate per
 * batch in any order:
 *   running_max_abs[j] = max(start_j, max_b max_r |x[b][r][j]|)
 * where start_j is the buffer's value (first == 0, as sq_calibrate) or 0
 * (first != 0, as sq_calibrate_first on the first batch: no zero fill).
 *   x               HOST array of nbatch DEVICE pointers, batch b [rows[b]][k]
 *                   in xt, each 16-byte aligned (may be NULL where rows[b] == 0)
 *   rows            HOST array of nbatch row counts, each >= 0, summing to at
 *                   most SQ_MAX_ROWS
 *   nbatch          1 .. SQ_MAX_CALIB_BATCHES
 *   running_max_abs [k] fp32, in/out as in sq_calibrate
 * Both host arrays are read before the call returns. One launch over all
 * the rows (the row groups of a column max over that many rows), after a
 * zero fill when first != 0 and the rows make more than one row group (more
 * than 128 rows).
 * Returns SQ_OK, or SQ_ERR_* before launching. No rows at all: a no-op, or
 * the buffer set to 0 when first != 0.
 */
sq_status sq_calibrate_batches(const void* const* x, const int64_t* rows, int nbatch, sq_dtype xt,
                               int64_t k, float* running_max_abs, int first, void* stream);

/*
 * sq_prepare_weight -- the smoothing factor s and the int8 weights.
 * Follows calibrate_smoothquant + SmoothQuantW8A8.freeze_quantization
 * (page "w8a8_smoothquant.py"); calling it again with another alpha is
 * recompute_smooth_scale.
 *   mw_j     = max(max_o |w[o][j]|, 1e-8)
 *   mx_j     = max(x_max_abs[j], 1e-8)
 *   s_j      = max(f32(P(mx_j, alpha)) / f32(P(mw_j, 1 - alpha)), 1e-8)
 *              with P(x, a) = x^a through binary64 (exact sqrt-based forms
 *              for a in {0, 1/4, 1/2, 3/4, 1}, binary64 pow otherwise) and
 *              1 - alpha formed in binary64
 *   w~[o][j] = f32(w[o][j] * s_j)
 *   w_scale[o] = max(max_j |w~[o][j]|, 1e-8) / 127
 *   w_q[o][j]  = clamp(round_half_even(w~[o][j] / w_scale[o]), -128, 127)
 *   w         [n][k] in wt (F32 or BF16), 16-byte aligned
 *   x_max_abs [k] fp32 from sq_calibrate, or NULL: never calibrated, s = 1
 *             and the call returns SQ_WARN_UNCALIBRATED (the page's warning
 *             for that case announces a fallback to s = 1)
 *   alpha     in [0, 1]
 *   smooth    [k] fp32 out (also used as scratch during the call)
 *   w_q       [n][k] int8 out, 16-byte aligned (also used as scratch for
 *             the per-row-group column maxima before the codes are written)
 *   w_scale   [n] fp32 out
 * n must be >= 1.
 */
sq_status sq_prepare_weight(const void* w, sq_dtype wt, int64_t n, int64_t k,
                            const float* x_max_abs, float alpha, float* smooth,
                            int8_t* w_q, float* w_scale, void* stream);

/*
 * sq_quantize_act -- dynamic per-token int8 of X / s.
 * Follows SmoothQuantW8A8.forward (X_smooth = X / s, then
 * quantize_per_token_symmetric), page "w8a8_smoothquant.py":
 *   x~[t][j]   = f32(x[t][j] / smooth[j])
 *   x_scale[t] = max(max_j |x~[t][j]|, 1e-8) / 127
 *   x_q[t][j]  = clamp(round_half_even(x~[t][j] / x_scale[t]), -128, 127)
 *   x       [m][k] in xt (F32 or BF16), 16-byte aligned
 *   smooth  [k] fp32 from sq_prepare_weight (every s_j > 0)
 *   x_q     [m][k] int8 out, 16-byte aligned
 *   x_scale [m] fp32 out
 */
sq_status sq_quantize_act(const void* x, sq_dtype xt, int64_t m, int64_t k,
                          const float* smooth, int8_t* x_q, float* x_scale,
                          void* stream);

/*
 * sq_w8a8_gemm -- the INT8 x INT8 -> INT32 product and its dequantisation.
 * The page's forward multiplies the dequantised operands in fp32 and notes
 * that real hardware does INT8 x INT8 -> INT32 -> fp32; this is that route:
 *   acc[t][o] = sum_j x_q[t][j] * w_q[o][j]          (exact, int32)
 *   y[t][o]   = acc[t][o] * x_scale[t] * w_scale[o] + bias[o]   (fp32, then
 *               rounded to yt); the bias is added after the product
 *   x_q     [m][k] int8, w_q [n][k] int8 (both 16-byte aligned)
 *   x_scale [m] fp32, w_scale [n] fp32 (ignored when yt == SQ_I32)
 *   bias    [n] in bias_t (F32 or BF16), or NULL for none
 *   y       [m][n] in yt: SQ_F32, SQ_BF16 (round to nearest even) or SQ_I32
 *           (raw acc; scales and bias are not applied), 16-byte aligned
 */
sq_status sq_w8a8_gemm(const int8_t* x_q, const float* x_scale, int64_t m,
                       const int8_t* w_q, const float* w_scale, int64_t n,
                       int64_t k, const void* bias, sq_dtype bias_t, void* y,
                       sq_dtype yt, void* stream);

/*
 * sq_w8a8_linear -- one frozen forward: sq_quantize_act then sq_w8a8_gemm.
 * Follows SmoothQuantW8A8.forward, quantized branch (page
 * "w8a8_smoothquant.py"). The activation codes and scales are written to
 * the caller's workspace, laid out as
 *   [0, m*k)                      x_q  int8 [m][k]
 *   [round_up(m*k, 256), +4*m)    x_scale fp32 [m]
 * so they can be inspected after the call.
 *   x         [m][k] in xt; bias [n] in xt or NULL; y [m][n] in yt
 *   workspace device memory of at least sq_w8a8_linear_workspace_bytes(m, k)
 *             bytes, 256-byte aligned
 */
sq_status sq_w8a8_linear(const void* x, sq_dtype xt, int64_t m, int64_t k,
                         const float* smooth, const int8_t* w_q,
                         const float* w_scale, int64_t n, const void* bias,
                         void* y, sq_dtype yt, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * sq_quantize_tensor -- per-tensor symmetric int8 (the per-tensor variant).
 * Follows quantize_tensor (num_bits = 8) of the page "quantized_linear.py":
 * one scale for the whole tensor,
 *   scale = f32(max_i |x_i| / 127), replaced by 1 when below 1e-8
 *   q_i   = clamp(round_half_even(f32(x_i / scale)), -128, 127)
 * (the page returns q * scale; the codes and the scale are returned here).
 *   x      [count] in xt (F32 or BF16), 16-byte aligned
 *   count  >= 1, a multiple of 16
 *   q      [count] int8 out, 16-byte aligned (also scratch during the call:
 *          it holds per-block maxima until the codes overwrite them)
 *   scale  [1] fp32 out, device memory
 */
sq_status sq_quantize_tensor(const void* x, sq_dtype xt, int64_t count, int8_t* q,
                             float* scale, void* stream);

/*
 * sq_w8a8_gemm_per_tensor -- sq_w8a8_gemm with one activation scale and one
 * weight scale (the per-tensor variant): the page "quantized_linear.py",
 * QuantizedLinear.forward, multiplies the per-tensor dequantised input and
 * weight and adds the bias; on the integer route that is
 *   y[t][o] = f32(acc[t][o]) * x_scale[0] * w_scale[0] + bias[o].
 * Arguments as sq_w8a8_gemm, except x_scale and w_scale point to a single
 * fp32 value each (device memory, e.g. from sq_quantize_tensor).
 */
sq_status sq_w8a8_gemm_per_tensor(const int8_t* x_q, const float* x_scale, int64_t m,
                                  const int8_t* w_q, const float* w_scale, int64_t n,
                                  int64_t k, const void* bias, sq_dtype bias_t, void* y,
                                  sq_dtype yt, void* stream);

/*
 * sq_quantize_tensor_tiled -- sq_quantize_tensor of a [rows][k] matrix with
 * the codes in the 16 x 64 tiled layout (see sq_tiled_bytes): the same one
 * scale and the same codes, the padding columns of every row zero.
 *   x      [rows][k] in xt (F32 or BF16), 16-byte aligned; k a multiple of 16
 *   q      sq_tiled_bytes(rows, k) bytes, 16-byte aligned (also scratch
 *          during the call, as in sq_quantize_tensor)
 *   scale  [1] fp32 out, device memory
 */
sq_status sq_quantize_tensor_tiled(const void* x, sq_dtype xt, int64_t rows, int64_t k,
                                   int8_t* q, float* scale, void* stream);

/*
 * sq_w8a8_gemm_per_tensor_tiled -- sq_w8a8_gemm_per_tensor with both codes
 * in the tiled layout (from sq_quantize_tensor_tiled); the arithmetic and
 * the output as sq_w8a8_gemm_per_tensor, bit-identical to it.
 */
sq_status sq_w8a8_gemm_per_tensor_tiled(const int8_t* x_q, const float* x_scale, int64_t m,
                                        const int8_t* w_q, const float* w_scale, int64_t n,
                                        int64_t k, const void* bias, sq_dtype bias_t, void* y,
                                        sq_dtype yt, void* stream);

/*
 * sq_wo_linear -- weight-only int8 linear: bf16 activations, int8 weights.
 * Follows Int8WeightOnlyQuantizedLinearWeight._quantized_op of the torchao
 * page "quantization/subclass.py": the int8 weights are converted to the
 * activations' type, multiplied with them, scaled per output channel, and
 * the bias is added:
 *   y[t][o] = f32(sum_j x[t][j] * w_q[o][j]) * w_scale[o] + bias[o]
 * with every bf16 x int8 product exact and the sum accumulated in fp32
 * (order unspecified), then rounded to yt. The weights are those of
 * sq_prepare_weight; with SmoothQuant weights (W * s) the activations must be
 * the smoothed X / s (as when s is folded into the preceding layer), with
 * uncalibrated weights (s = 1) they are plain per-channel int8 weights.
 * Built for the decode shape: tokens are processed in chunks of 64, each
 * chunk streaming the weights once.
 *   x       [m][k] bf16 (SQ_BF16 only), 16-byte aligned
 *   w_q     [n][k] int8, 16-byte aligned; w_scale [n] fp32
 *   bias    [n] in bias_t (F32 or BF16), or NULL
 *   y       [m][n] in yt (SQ_F32 or SQ_BF16, round to nearest even),
 *           4-byte aligned
 */
sq_status sq_wo_linear(const void* x, sq_dtype xt, int64_t m, int64_t k,
                       const int8_t* w_q, const float* w_scale, int64_t n,
                       const void* bias, sq_dtype bias_t, void* y, sq_dtype yt,
                       void* stream);

/*
 * sq_wo_linear_tiled -- sq_wo_linear with w_q in the 16 x 64 tiled layout
 * (from sq_prepare_weight_tiled; sq_tiled_bytes(n, k) bytes, 16-byte
 * aligned). Each weight load then reads one 1 KiB tile contiguously. The
 * other arguments, the arithmetic and the output as sq_wo_linear.
 */
sq_status sq_wo_linear_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k,
                             const int8_t* w_q, const float* w_scale, int64_t n,
                             const void* bias, sq_dtype bias_t, void* y, sq_dtype yt,
                             void* stream);

/*
 * sq_selfcheck_reciprocal -- device self-check behind the activation path.
 * For bf16 activations, sq_quantize_act / sq_w8a8_linear form x / s as
 * fma(fma(-q0, s, x), y, q0) with q0 = x * y and y the correctly rounded
 * 1/s, obtained from the hardware reciprocal and one Newton step. This call
 * counts, over every binary32 s in [2^-100, 2^100), the values for which
 * that y differs from the IEEE quotient 1/s, and adds the count to
 * *mismatches (a device uint64 the caller zeroes). 0 on the running device
 * is the precondition of the fast path's exactness.
 */
sq_status sq_selfcheck_reciprocal(unsigned long long* mismatches, void* stream);

/*
 * sq_selfcheck_division -- device self-check behind every binary32 quotient
 * of the quantisation kernels. They divide a by b as q0 = RN(a * y),
 * q1 = fma(fma(-q0, b, a), y, q0) with y = RN(1/b). For the divisor
 * significands m in [b_begin, b_end) (b = 1 + m * 2^-23, m < 2^23) and
 * every numerator significand a in [1, 2), this call adds to *mismatches
 * the count of pairs where q1 differs from the IEEE quotient a / b (the
 * whole range, 2^46 pairs, takes some tens of seconds). Powers of two scale
 * every step exactly, so 0 over the whole range makes the scheme exact for
 * all operands whose steps stay in the normal range.
 */
sq_status sq_selfcheck_division(unsigned b_begin, unsigned b_end, unsigned long long* mismatches,
                                void* stream);

/*
 * sq_weight_col_max -- the weight side's per-input-channel maximum, stored
 * so that a new alpha needs no second pass over W: max_w of
 * calibrate_smoothquant (page "w8a8_smoothquant.py"),
 *   w_max_abs[j] = max(max_o |w[o][j]|, 1e-8)
 *   w          [n][k] in wt (F32 or BF16), 16-byte aligned, n >= 1
 *   w_max_abs  [k] fp32 out, 16-byte aligned
 */
sq_status sq_weight_col_max(const void* w, sq_dtype wt, int64_t n, int64_t k, float* w_max_abs,
                            void* stream);

/*
 * sq_recompute_smooth_scale -- SmoothQuantW8A8.recompute_smooth_scale (page
 * "w8a8_smoothquant.py"): s and the int8 weights for a new alpha from the
 * stored activation and weight maxima, with one pass over W (the column
 * max is not recomputed). The results are bit-identical to
 * sq_prepare_weight(w, ..., x_max_abs, alpha, ...) when w_max_abs comes from
 * sq_weight_col_max of the same w.
 *   x_max_abs  [k] fp32 from sq_calibrate, or NULL: never calibrated, s = 1
 *              and the call returns SQ_WARN_UNCALIBRATED
 *   w_max_abs  [k] fp32 from sq_weight_col_max (required with x_max_abs;
 *              every entry a finite binary32 >= 0), 16-byte aligned
 *   the other arguments and outputs as sq_prepare_weight
 */
sq_status sq_recompute_smooth_scale(const void* w, sq_dtype wt, int64_t n, int64_t k,
                                    const float* x_max_abs, const float* w_max_abs, float alpha,
                                    float* smooth, int8_t* w_q, float* w_scale, void* stream);

/*
 * Tiled int8 layout. The int8 codes of a [rows][k] matrix can also be kept
 * in 16 x 64 tiles: rows in groups of 16, K in 64-byte chunks, rows padded
 * to a multiple of 16 and k to K64 = k rounded up to a multiple of 64; tile
 * (g, c) (row group g, chunk c) is 1 KiB at byte offset (g * K64/64 + c) *
 * 1024, row-major inside (row r of the group at r * 64). Element (i, j) is at
 *   ((i / 16) * (K64 / 64) + j / 64) * 1024 + (i % 16) * 64 + j % 64.
 * The codes are the same as in the row-major layout; the padding columns
 * of every row hold zeros, the padding rows are never read into a stored
 * output. The products read each tile as one contiguous 1 KiB load (a
 * row-major 16-row x 64-byte block is 16 separate 64-byte pieces): at
 * M = N = K = 4096 the int8 product measures 57.0 us against 63.5 us
 * row-major (paired runs), and on the decode shape (16 x 4096 -> 11008)
 * 10.7 us against 13.1 us.
 * sq_tiled_bytes(rows, k) is the size of such an array (0 for rows <= 0 or
 * k <= 0).
 */
size_t sq_tiled_bytes(int64_t rows, int64_t k);

/*
 * sq_prepare_weight_tiled -- sq_prepare_weight with w_q in the tiled layout
 * (sq_tiled_bytes(n, k) bytes, 16-byte aligned; also scratch during the
 * call); smooth and w_scale as sq_prepare_weight, bit-identical codes.
 */
sq_status sq_prepare_weight_tiled(const void* w, sq_dtype wt, int64_t n, int64_t k,
                                  const float* x_max_abs, float alpha, float* smooth,
                                  int8_t* w_q, float* w_scale, void* stream);

/*
 * sq_quantize_act_tiled -- sq_quantize_act with x_q in the tiled layout
 * (sq_tiled_bytes(m, k) bytes, 16-byte aligned); x_scale as
 * sq_quantize_act, bit-identical codes.
 */
sq_status sq_quantize_act_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k,
                                const float* smooth, int8_t* x_q, float* x_scale, void* stream);

/*
 * sq_w8a8_gemm_tiled -- sq_w8a8_gemm with both x_q and w_q in the tiled
 * layout (from sq_quantize_act_tiled and sq_prepare_weight_tiled); the other
 * arguments, the arithmetic and the output as sq_w8a8_gemm (yt SQ_I32 gives
 * the raw int32 products), bit-identical to it. Up to 64 tokens the product
 * streams the weights (one pass over w_q per 64 tokens), beyond that it
 * runs on MFMA tiles.
 */
sq_status sq_w8a8_gemm_tiled(const int8_t* x_q, const float* x_scale, int64_t m,
                             const int8_t* w_q, const float* w_scale, int64_t n, int64_t k,
                             const void* bias, sq_dtype bias_t, void* y, sq_dtype yt, void* stream);

/*
 * sq_smoothing_factor -- step a3 alone (calibrate_smoothquant, page
 * "w8a8_smoothquant.py"): s from the stored maxima, exactly as
 * sq_prepare_weight computes it,
 *   s_j = max(f32(P(max(x_max_abs[j], 1e-8), alpha)) /
 *             f32(P(max(w_max_abs[j], 1e-8), 1 - alpha)), 1e-8)
 *   x_max_abs  [k] fp32 from sq_calibrate, or NULL: never calibrated, s = 1
 *              and the call returns SQ_WARN_UNCALIBRATED
 *   w_max_abs  [k] fp32 from sq_weight_col_max (every entry a finite
 *              binary32 >= 0), 16-byte aligned
 *   alpha      in [0, 1];  smooth [k] fp32 out, 16-byte aligned
 * With sq_weight_col_max and sq_quantize_weight it splits sq_prepare_weight
 * into separate calls (the column max does not need the activations'
 * maxima; s can be recomputed for a new alpha without touching W).
 */
sq_status sq_smoothing_factor(const float* x_max_abs, const float* w_max_abs, float alpha, int64_t k,
                              float* smooth, void* stream);

/*
 * sq_quantize_weight -- steps a4-a5 alone (freeze_quantization, page
 * "w8a8_smoothquant.py"): w~ = f32(w * s), one scale per output row,
 * int8 codes, exactly as sq_prepare_weight writes them.
 *   w       [n][k] in wt (F32 or BF16), 16-byte aligned, n >= 1
 *   smooth  [k] fp32 (every s_j > 0), 16-byte aligned
 *   w_q     [n][k] int8 out, 16-byte aligned;  w_scale [n] fp32 out
 */
sq_status sq_quantize_weight(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* smooth,
                             int8_t* w_q, float* w_scale, void* stream);

/*
 * sq_reference_linear -- the full-precision output quantization_error
 * compares against (page "w8a8_smoothquant.py",
 * SmoothQuantW8A8.quantization_error: the plain linear layer on the
 * unquantised input and weights):
 *   y[t][o] = f32(sum_j x[t][j] * w[o][j]) + bias[o]   -> yt
 * every product exact in fp32 (bf16 operands) or rounded once (fp32
 * operands), the sum accumulated in fp32 by the matrix units (order
 * unspecified).
 *   x     [m][k] in xt (F32 or BF16), 16-byte aligned
 *   w     [n][k] in xt (the same type as x), 16-byte aligned
 *   bias  [n] in bias_t (F32 or BF16), or NULL
 *   y     [m][n] in yt (SQ_F32 or SQ_BF16), 16-byte aligned
 * m = 0 is a no-op.
 */
sq_status sq_reference_linear(const void* x, sq_dtype xt, int64_t m, int64_t k, const void* w,
                              int64_t n, const void* bias, sq_dtype bias_t, void* y, sq_dtype yt,
                              void* stream);

/*
 * sq_relative_error -- quantization_error's measure (page
 * "w8a8_smoothquant.py", SmoothQuantW8A8.quantization_error):
 *   result[0] = ||y_fp - y_q||_F,  result[1] = ||y_fp||_F,
 *   result[2] = result[0] / max(result[1], 1e-12)
 * with the sums of squares in binary64, in a fixed order (the same count
 * gives the same bits).
 *   y_fp, y_q  [count] fp32 each (e.g. sq_reference_linear and
 *              sq_w8a8_gemm outputs), 16-byte aligned, count >= 1
 *   workspace  device memory of sq_relative_error_workspace_bytes(count)
 *              bytes, 8-byte aligned (partial sums; overwritten)
 *   result     [3] binary64 out, device memory, 8-byte aligned
 */
sq_status sq_relative_error(const float* y_fp, const float* y_q, int64_t count, void* workspace,
                            size_t workspace_bytes, double* result, void* stream);
size_t sq_relative_error_workspace_bytes(int64_t count);

/*
 * The learnable alpha (page "w8a8_smoothquant.py", the module docstring's
 * notes on it and SmoothQuantW8A8.__init__ / alpha): alpha = sigmoid(eta)
 * with eta the trained parameter, initialised to log(a / max(1e-6, 1 - a))
 * for an initial alpha a. Both computed in binary64 and rounded once to
 * binary32. Host functions (no device work).
 */
float sq_alpha_from_eta(float eta);
float sq_eta_from_alpha(double alpha);

/*
 * sq_ste_backward -- the straight-through backward of the quantized forward
 * and the gradient of the learnable alpha. Follows STEQuantize / ste_quantize
 * and SmoothQuantW8A8.forward (page "w8a8_smoothquant.py"): the forward
 * recomputes s from alpha, quantises X~ = X / s per token and W~ = W * s per
 * output channel, and multiplies the dequantised operands; the estimator
 * passes the gradient of each dequantised operand to X~ and W~ unchanged
 * (no gradient reaches the quantisers' scales). For the upstream gradient
 * dy of Y = Xd Wd^T + bias, Xd = x_q * x_scale, Wd = w_q * w_scale:
 *   gX[t][j] = sum_o dy[t][o] w_q[o][j] w_scale[o]
 *   gW[o][j] = sum_t dy[t][o] x_q[t][j] x_scale[t]
 *   dx[t][j] = gX[t][j] / s_j          dw[o][j] = gW[o][j] * s_j
 *   dbias[o] = sum_t dy[t][o]
 *   dsmooth_j = sum_o gW[o][j] w[o][j] - sum_t gX[t][j] x[t][j] / s_j^2
 *   dalpha = sum_j [s_raw_j >= 1e-8] dsmooth_j s_raw_j (ln mx_j + ln mw_j)
 *   deta = dalpha alpha (1 - alpha)
 * where s_raw_j is the smoothing factor before its floor (the floor is a
 * clamp, which passes no gradient below it), mx_j = max(x_max_abs[j],
 * 1e-8) and mw_j = w_max_abs[j]; neither maximum is differentiated (the
 * page keeps the activation maximum as a buffer and takes the weight
 * maximum of detached weights).
 * Arithmetic: the gradient products run on bf16 MFMA with every product
 * exact (the fp32 factor RN32(dy * scale) split into three bf16 planes, the
 * int8 codes exact in bf16) and fp32 sums; dx divides with IEEE binary32
 * division; the sums behind dsmooth, dalpha and dbias are binary64 in a
 * fixed order (the same inputs give the same bits).
 *   dy        [m][n] in dyt (F32 or BF16), aligned to its element
 *   x         [m][k] in xt, w [n][k] in wt (the forward's inputs), 16-byte aligned
 *   smooth    [k] the forward's s;  x_q [m][k], x_scale [m], w_q [n][k],
 *             w_scale [n] the forward's codes and scales (row-major,
 *             16-byte aligned)
 *   x_max_abs [k] the stored activation maxima, or NULL: never calibrated,
 *             s = 1 does not depend on alpha, dalpha = deta = 0 and the call
 *             returns SQ_WARN_UNCALIBRATED
 *   w_max_abs [k] from sq_weight_col_max (required with x_max_abs)
 *   alpha     the forward's alpha, in [0, 1]
 *   dx [m][k], dw [n][k] fp32 out, 16-byte aligned; dbias [n] fp32 out or
 *   NULL; dsmooth [k] fp32 out or NULL; dalpha_deta [2] binary64 out
 *   workspace sq_ste_backward_workspace_bytes(m, n, k) bytes, 256-byte
 *             aligned (overwritten)
 * m and n from 1 to SQ_STE_MAX_ROWS.
 */
#define SQ_STE_MAX_ROWS (1LL << 24)
size_t sq_ste_backward_workspace_bytes(int64_t m, int64_t n, int64_t k);
sq_status sq_ste_backward(const void* dy, sq_dtype dyt, int64_t m, int64_t n, int64_t k,
                          const void* x, sq_dtype xt, const void* w, sq_dtype wt,
                          const float* smooth, const int8_t* x_q, const float* x_scale,
                          const int8_t* w_q, const float* w_scale, const float* x_max_abs,
                          const float* w_max_abs, float alpha, float* dx, float* dw,
                          float* dbias, float* dsmooth, double* dalpha_deta,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sq_aux_loss_grad -- the auxiliary loss of the module docstring (page
 * "w8a8_smoothquant.py"), the relative squared error of the quantized
 * output, and its gradient at y_q (the part that reaches eta):
 *   loss = ||y_fp - y_q||_F^2 / max(||y_fp||_F^2, 1e-24)        (binary64)
 *   dy_q = 2 (y_q - y_fp) / max(||y_fp||_F^2, 1e-24)            (fp32)
 *   y_fp, y_q [count] fp32, 16-byte aligned;  dy_q [count] fp32 out
 *   loss      [1] binary64 out, device memory
 *   workspace sq_aux_loss_grad_workspace_bytes(count) bytes, 256-byte aligned
 */
size_t sq_aux_loss_grad_workspace_bytes(int64_t count);
sq_status sq_aux_loss_grad(const float* y_fp, const float* y_q, int64_t count, float* dy_q,
                           double* loss, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sq_w8a8_linear_tiled -- one frozen forward on weights in the tiled layout
 * (SmoothQuantW8A8.forward, quantized branch, page "w8a8_smoothquant.py"):
 * sq_quantize_act_tiled then sq_w8a8_gemm_tiled (the same codes, scales and
 * output bits), the codes in the caller's workspace.
 *   x         [m][k] in xt; smooth [k]; w_q in 16 x 64 tiles (from
 *             sq_prepare_weight_tiled), w_scale [n]
 *   bias      [n] in bias_t (F32 or BF16), or NULL; y [m][n] in yt
 *   workspace sq_w8a8_linear_tiled_workspace_bytes(m, k) bytes, 256-byte
 *             aligned: the tiled x_q at byte 0, then x_scale [m] at the
 *             next 256-byte boundary
 */
size_t sq_w8a8_linear_tiled_workspace_bytes(int64_t m, int64_t k);
sq_status sq_w8a8_linear_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k,
                               const float* smooth, const int8_t* w_q, const float* w_scale,
                               int64_t n, const void* bias, sq_dtype bias_t, void* y,
                               sq_dtype yt, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * sq_w8a8_linear_tiled_fused -- sq_w8a8_linear_tiled for up to 64 tokens as
 * ONE kernel, the activation quantisation fused into the weight-streaming
 * product's prologue: workgroup b quantises tokens b, b + grid, ... and
 * publishes each (a flag per token); every workgroup waits, bounded, for
 * the tokens, and one whose wait runs out quantises the missing tokens
 * itself (the same bytes). The same codes, scales and output bits as
 * sq_w8a8_linear_tiled. Measured slower on the decode shape (16 x 4096 ->
 * 11008: 22.5 us against 14.5 us for the two launches): the publication
 * puts several dependent memory round trips ahead of the first multiply.
 *   m         1 to 64 (SQ_ERR_SHAPE beyond)
 *   workspace sq_w8a8_linear_tiled_fused_workspace_bytes(m, k) bytes,
 *             256-byte aligned, ZERO-FILLED BEFORE ITS FIRST USE: its first
 *             1 KiB holds synchronisation words that every call leaves
 *             consistent for the next; then the tiled x_q (byte 1024) and
 *             x_scale [m]. Calls that share a workspace must not overlap.
 * The other arguments as sq_w8a8_linear_tiled.
 */
size_t sq_w8a8_linear_tiled_fused_workspace_bytes(int64_t m, int64_t k);
sq_status sq_w8a8_linear_tiled_fused(const void* x, sq_dtype xt, int64_t m, int64_t k,
                                     const float* smooth, const int8_t* w_q, const float* w_scale,
                                     int64_t n, const void* bias, sq_dtype bias_t, void* y,
                                     sq_dtype yt, void* workspace, size_t workspace_bytes,
                                     void* stream);
/* Test hook of sq_w8a8_linear_tiled_fused: the polls (about 60 ns each) a
 * workgroup waits for the other workgroups' tokens before it quantises them
 * itself (default 4096; 0 makes every workgroup quantise every token
 * itself). Process-wide; not for concurrent use with calls. */
void sq_set_fused_wait_polls(int polls);

/* Workspace bytes sq_w8a8_linear needs for m tokens of k channels. */
size_t sq_w8a8_linear_workspace_bytes(int64_t m, int64_t k);

/*
 * sq_w8a8_linear_noalloc -- sq_w8a8_linear for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same launches, arithmetic and
 * outputs (bit for bit), with the activation codes and scales kept in a
 * fixed device array of the library instead of a caller workspace. The
 * call allocates and frees nothing.
 *   - Limits: m <= SQ_NOALLOC_MAX_TOKENS and m * k <= SQ_NOALLOC_MAX_CODES
 *     (16 MiB of codes: e.g. 4096 tokens of 4096 channels); larger calls
 *     return SQ_ERR_WORKSPACE before launching anything.
 *   - The array: one copy per GPU, held from the library's load until the
 *     process ends (SQ_NOALLOC_MAX_CODES + 4 * SQ_NOALLOC_MAX_TOKENS bytes);
 *     its address is looked up on the first call on each device, which must
 *     be the current device (and the stream's).
 *   - Every call on one GPU shares that array: calls that overlap on one
 *     GPU (different streams, or different host threads) race and may read
 *     each other's codes. The codes and scales are not readable through the
 *     ABI.
 * The other arguments, checks and statuses are sq_w8a8_linear's.
 */
#define SQ_NOALLOC_MAX_CODES (1LL << 24)
#define SQ_NOALLOC_MAX_TOKENS (1LL << 14)
sq_status sq_w8a8_linear_noalloc(const void* x, sq_dtype xt, int64_t m, int64_t k,
                                 const float* smooth, const int8_t* w_q,
                                 const float* w_scale, int64_t n, const void* bias,
                                 void* y, sq_dtype yt, void* stream);

/* A static, human-readable name for a status code. */
const char* sq_status_string(sq_status status);

/* ABI version of this header (bumped on any incompatible change). */
#define SQ_ABI_VERSION 1
int sq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
