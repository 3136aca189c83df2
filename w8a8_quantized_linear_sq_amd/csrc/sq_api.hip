// sq_api.hip -- the C ABI of libsq.so (declared in include/sq.h): argument
// checks, then the kernel launches on the caller's stream. Nothing here
// allocates, frees or synchronises.
#include "../../include/sq.h"
#include "sq_device.h"

#include <atomic>
#include <mutex>

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool fp_in(sq_dtype t) { return t == SQ_F32 || t == SQ_BF16; }

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// m, n, rows: the kernels index rows, tiles and row groups in int32, adding
// at most a tile (256) or a row group to a row count, so every count stays
// at or below 2^30
constexpr int64_t kMaxRows = SQ_MAX_ROWS;
// output tiles of the MFMA-tile product (counted at its smallest tile,
// 128 x 128): one workgroup of up to 512 threads each, and a launch's grid
// times its block size must stay below 2^32
constexpr int64_t kMaxTiles = SQ_MAX_TILES;

bool tiles_fit(int64_t m, int64_t n) {
    return ((m + 127) / 128) * ((n + 127) / 128) <= kMaxTiles;
}

sq_status launched(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

// shared checks on k and a [.][k] pointer
sq_status check_k(int64_t k) {
    if (k <= 0 || k > SQ_MAX_K) return SQ_ERR_SHAPE;
    if (k % 16) return SQ_ERR_ALIGN;
    return SQ_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

int sq_abi_version(void) { return SQ_ABI_VERSION; }

const char* sq_status_string(sq_status s) {
    switch (s) {
        case SQ_OK: return "SQ_OK";
        case SQ_WARN_UNCALIBRATED: return "SQ_WARN_UNCALIBRATED: no calibration data, s = 1";
        case SQ_ERR_ARG: return "SQ_ERR_ARG: null pointer, alpha outside [0, 1] or bad enum";
        case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: size out of range";
        case SQ_ERR_DTYPE: return "SQ_ERR_DTYPE: unsupported type";
        case SQ_ERR_ALIGN: return "SQ_ERR_ALIGN: k not a multiple of 16 or pointer not 16-byte aligned";
        case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
        case SQ_ERR_HIP: return "SQ_ERR_HIP: a kernel launch failed";
    }
    return "unknown sq_status";
}

sq_status sq_calibrate(const void* x, sq_dtype xt, int64_t rows, int64_t k, float* running_max_abs,
                       void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (rows == 0) return SQ_OK;
    if (!x || !running_max_abs) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(running_max_abs)) return SQ_ERR_ALIGN;
    return launched(sq_launch_colmax(x, xt == SQ_BF16, rows, k, running_max_abs, as_stream(stream)));
}

sq_status sq_calibrate_first(const void* x, sq_dtype xt, int64_t rows, int64_t k, float* running_max_abs,
                             void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (rows < 0 || rows > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!running_max_abs || (rows > 0 && !x)) return SQ_ERR_ARG;
    if ((rows > 0 && !aligned16(x)) || !aligned16(running_max_abs)) return SQ_ERR_ALIGN;
    return launched(sq_launch_colmax_first(x, xt == SQ_BF16, rows, k, running_max_abs, as_stream(stream)));
}

sq_status sq_calibrate_batches(const void* const* x, const int64_t* rows, int nbatch, sq_dtype xt, int64_t k,
                               float* running_max_abs, int first, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (nbatch < 1 || nbatch > SQ_MAX_CALIB_BATCHES) return SQ_ERR_SHAPE;
    if (!x || !rows || !running_max_abs) return SQ_ERR_ARG;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    int64_t total = 0;
    for (int b = 0; b < nbatch; ++b) {
        if (rows[b] < 0 || rows[b] > kMaxRows) return SQ_ERR_SHAPE;
        total += rows[b];
        if (total > kMaxRows) return SQ_ERR_SHAPE;
        if (rows[b] > 0 && !x[b]) return SQ_ERR_ARG;
        if (rows[b] > 0 && !aligned16(x[b])) return SQ_ERR_ALIGN;
    }
    if (!aligned16(running_max_abs)) return SQ_ERR_ALIGN;
    if (total == 0 && !first) return SQ_OK;
    return launched(sq_launch_colmax_batches(x, rows, nbatch, xt == SQ_BF16, k, running_max_abs, first,
                                             as_stream(stream)));
}

sq_status sq_prepare_weight(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* x_max_abs,
                            float alpha, float* smooth, int8_t* w_q, float* w_scale, void* stream) {
    if (!fp_in(wt)) return SQ_ERR_DTYPE;
    if (n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;  // also rejects NaN
    if (!w || !smooth || !w_q || !w_scale) return SQ_ERR_ARG;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    if (x_max_abs && !aligned16(x_max_abs)) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    const int bf16 = wt == SQ_BF16;
    hipError_t e;
    if (!x_max_abs) {
        e = sq_launch_fill(smooth, 1.0f, k, s);
    } else {
        // column max of |W| per row group into a buffer the call overwrites
        // later anyway (w_q, or smooth itself for a single group), then s
        const int64_t groups = sq_colmax_partial_groups(n, k, bf16, n * k);
        unsigned* partial = groups == 1 ? (unsigned*)smooth : (unsigned*)w_q;
        e = sq_launch_colmax_partial(w, bf16, n, k, groups, partial, s);
        if (e == hipSuccess) {
            const double a_x = (double)alpha;
            const double a_w = 1.0 - (double)alpha;
            e = sq_launch_smooth_factor(x_max_abs, partial, groups, a_x, a_w, k, smooth, s);
        }
    }
    if (e == hipSuccess) e = sq_launch_quantize_weight(w, bf16, smooth, n, k, w_q, w_scale, s);
    if (e != hipSuccess) return SQ_ERR_HIP;
    return x_max_abs ? SQ_OK : SQ_WARN_UNCALIBRATED;
}

sq_status sq_quantize_act(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                          int8_t* x_q, float* x_scale, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x || !smooth || !x_q || !x_scale) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(smooth) || !aligned16(x_q)) return SQ_ERR_ALIGN;
    return launched(sq_launch_quantize_act(x, xt == SQ_BF16, smooth, m, k, x_q, x_scale, as_stream(stream)));
}

static sq_status check_gemm(const int8_t* x_q, const float* x_scale, int64_t m, const int8_t* w_q,
                            const float* w_scale, int64_t n, int64_t k, const void* bias,
                            sq_dtype bias_t, const void* y, sq_dtype yt) {
    if (!(yt == SQ_F32 || yt == SQ_BF16 || yt == SQ_I32)) return SQ_ERR_DTYPE;
    if (bias && !fp_in(bias_t)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows || n <= 0 || n > kMaxRows || !tiles_fit(m, n)) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x_q || !w_q || !y) return SQ_ERR_ARG;
    if (yt != SQ_I32 && (!x_scale || !w_scale)) return SQ_ERR_ARG;
    if (!aligned16(x_q) || !aligned16(w_q) || !aligned16(y)) return SQ_ERR_ALIGN;
    return SQ_OK;
}

static int out_kind(sq_dtype yt) { return yt == SQ_F32 ? 0 : yt == SQ_BF16 ? 1 : 2; }
static int bias_kind(const void* bias, sq_dtype bt) { return !bias ? 0 : bt == SQ_F32 ? 1 : 2; }

sq_status sq_w8a8_gemm(const int8_t* x_q, const float* x_scale, int64_t m, const int8_t* w_q,
                       const float* w_scale, int64_t n, int64_t k, const void* bias, sq_dtype bias_t,
                       void* y, sq_dtype yt, void* stream) {
    sq_status st = check_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_t, y, yt);
    if (st != SQ_OK || m == 0) return st;
    return launched(sq_launch_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_kind(bias, bias_t), y,
                                   out_kind(yt), 0, as_stream(stream)));
}

sq_status sq_quantize_tensor(const void* x, sq_dtype xt, int64_t count, int8_t* q, float* scale, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (count <= 0 || count > ((int64_t)1 << 40)) return SQ_ERR_SHAPE;
    if (count % 16) return SQ_ERR_ALIGN;
    if (!x || !q || !scale) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(q) || ((uintptr_t)scale & 3u) != 0) return SQ_ERR_ALIGN;
    return launched(sq_launch_quantize_tensor(x, xt == SQ_BF16, count, q, scale, as_stream(stream)));
}

sq_status sq_w8a8_gemm_per_tensor(const int8_t* x_q, const float* x_scale, int64_t m, const int8_t* w_q,
                                  const float* w_scale, int64_t n, int64_t k, const void* bias, sq_dtype bias_t,
                                  void* y, sq_dtype yt, void* stream) {
    sq_status st = check_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_t, y, yt);
    if (st != SQ_OK || m == 0) return st;
    return launched(sq_launch_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_kind(bias, bias_t), y,
                                   out_kind(yt), 1, as_stream(stream)));
}

sq_status sq_quantize_tensor_tiled(const void* x, sq_dtype xt, int64_t rows, int64_t k, int8_t* q, float* scale,
                                   void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (rows <= 0 || rows > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!x || !q || !scale) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(q) || ((uintptr_t)scale & 3u) != 0) return SQ_ERR_ALIGN;
    return launched(sq_launch_quantize_tensor_tiled(x, xt == SQ_BF16, rows, k, q, scale, as_stream(stream)));
}

sq_status sq_w8a8_gemm_per_tensor_tiled(const int8_t* x_q, const float* x_scale, int64_t m, const int8_t* w_q,
                                        const float* w_scale, int64_t n, int64_t k, const void* bias,
                                        sq_dtype bias_t, void* y, sq_dtype yt, void* stream) {
    sq_status st = check_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_t, y, yt);
    if (st != SQ_OK || m == 0) return st;
    return launched(sq_launch_gemm_tiled(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_kind(bias, bias_t), y,
                                         out_kind(yt), 1, as_stream(stream)));
}

sq_status sq_wo_linear(const void* x, sq_dtype xt, int64_t m, int64_t k, const int8_t* w_q, const float* w_scale,
                       int64_t n, const void* bias, sq_dtype bias_t, void* y, sq_dtype yt, void* stream) {
    if (xt != SQ_BF16) return SQ_ERR_DTYPE;
    if (!(yt == SQ_F32 || yt == SQ_BF16)) return SQ_ERR_DTYPE;
    if (bias && !fp_in(bias_t)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows || n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x || !w_q || !w_scale || !y) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(w_q) || ((uintptr_t)y & 3u) != 0) return SQ_ERR_ALIGN;
    return launched(sq_launch_wo_linear(x, m, k, w_q, w_scale, n, bias, bias_kind(bias, bias_t), y,
                                        yt == SQ_F32 ? 0 : 1, as_stream(stream)));
}

sq_status sq_wo_linear_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k, const int8_t* w_q,
                             const float* w_scale, int64_t n, const void* bias, sq_dtype bias_t, void* y, sq_dtype yt,
                             void* stream) {
    if (xt != SQ_BF16) return SQ_ERR_DTYPE;
    if (!(yt == SQ_F32 || yt == SQ_BF16)) return SQ_ERR_DTYPE;
    if (bias && !fp_in(bias_t)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows || n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x || !w_q || !w_scale || !y) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(w_q) || ((uintptr_t)y & 3u) != 0) return SQ_ERR_ALIGN;
    return launched(sq_launch_wo_linear_tiled(x, m, k, w_q, w_scale, n, bias, bias_kind(bias, bias_t), y,
                                              yt == SQ_F32 ? 0 : 1, as_stream(stream)));
}

sq_status sq_weight_col_max(const void* w, sq_dtype wt, int64_t n, int64_t k, float* w_max_abs, void* stream) {
    if (!fp_in(wt)) return SQ_ERR_DTYPE;
    if (n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!w || !w_max_abs) return SQ_ERR_ARG;
    if (!aligned16(w) || !aligned16(w_max_abs)) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    // the running max starts at the floor, so the result is the floored max
    hipError_t e = sq_launch_fill(w_max_abs, sq::kFloor, k, s);
    if (e == hipSuccess) e = sq_launch_colmax(w, wt == SQ_BF16, n, k, w_max_abs, s);
    return launched(e);
}

sq_status sq_recompute_smooth_scale(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* x_max_abs,
                                    const float* w_max_abs, float alpha, float* smooth, int8_t* w_q,
                                    float* w_scale, void* stream) {
    if (!fp_in(wt)) return SQ_ERR_DTYPE;
    if (n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;  // also rejects NaN
    if (!w || !smooth || !w_q || !w_scale) return SQ_ERR_ARG;
    if (x_max_abs && !w_max_abs) return SQ_ERR_ARG;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    if (x_max_abs && (!aligned16(x_max_abs) || !aligned16(w_max_abs))) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    hipError_t e;
    if (!x_max_abs) {
        e = sq_launch_fill(smooth, 1.0f, k, s);
    } else {
        // the stored column max stands for the single row group of the
        // smoothing-factor kernel (non-negative binary32: its bit pattern
        // orders as the value)
        e = sq_launch_smooth_factor(x_max_abs, (const unsigned*)w_max_abs, 1, (double)alpha, 1.0 - (double)alpha,
                                    k, smooth, s);
    }
    if (e == hipSuccess) e = sq_launch_quantize_weight(w, wt == SQ_BF16, smooth, n, k, w_q, w_scale, s);
    if (e != hipSuccess) return SQ_ERR_HIP;
    return x_max_abs ? SQ_OK : SQ_WARN_UNCALIBRATED;
}

size_t sq_tiled_bytes(int64_t rows, int64_t k) {
    if (rows <= 0 || k <= 0) return 0;
    return (size_t)((rows + 15) / 16 * 16) * (size_t)((k + 63) / 64 * 64);
}

sq_status sq_prepare_weight_tiled(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* x_max_abs,
                                  float alpha, float* smooth, int8_t* w_q, float* w_scale, void* stream) {
    if (!fp_in(wt)) return SQ_ERR_DTYPE;
    if (n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;  // also rejects NaN
    if (!w || !smooth || !w_q || !w_scale) return SQ_ERR_ARG;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    if (x_max_abs && !aligned16(x_max_abs)) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    const int bf16 = wt == SQ_BF16;
    hipError_t e;
    if (!x_max_abs) {
        e = sq_launch_fill(smooth, 1.0f, k, s);
    } else {
        // the row-group column maxima live in w_q (at least n * k bytes)
        // until the codes overwrite them, or in smooth for a single group
        const int64_t groups = sq_colmax_partial_groups(n, k, bf16, n * k);
        unsigned* partial = groups == 1 ? (unsigned*)smooth : (unsigned*)w_q;
        e = sq_launch_colmax_partial(w, bf16, n, k, groups, partial, s);
        if (e == hipSuccess)
            e = sq_launch_smooth_factor(x_max_abs, partial, groups, (double)alpha, 1.0 - (double)alpha, k, smooth, s);
    }
    if (e == hipSuccess) e = sq_launch_quantize_weight_tiled(w, bf16, smooth, n, k, w_q, w_scale, s);
    if (e != hipSuccess) return SQ_ERR_HIP;
    return x_max_abs ? SQ_OK : SQ_WARN_UNCALIBRATED;
}

sq_status sq_quantize_act_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                                int8_t* x_q, float* x_scale, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x || !smooth || !x_q || !x_scale) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(smooth) || !aligned16(x_q)) return SQ_ERR_ALIGN;
    return launched(sq_launch_quantize_act_tiled(x, xt == SQ_BF16, smooth, m, k, x_q, x_scale, as_stream(stream)));
}

sq_status sq_w8a8_gemm_tiled(const int8_t* x_q, const float* x_scale, int64_t m, const int8_t* w_q,
                             const float* w_scale, int64_t n, int64_t k, const void* bias, sq_dtype bias_t, void* y,
                             sq_dtype yt, void* stream) {
    sq_status st = check_gemm(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_t, y, yt);
    if (st != SQ_OK || m == 0) return st;
    return launched(sq_launch_gemm_tiled(x_q, x_scale, m, w_q, w_scale, n, k, bias, bias_kind(bias, bias_t), y,
                                         out_kind(yt), 0, as_stream(stream)));
}

sq_status sq_smoothing_factor(const float* x_max_abs, const float* w_max_abs, float alpha, int64_t k,
                              float* smooth, void* stream) {
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;  // also rejects NaN
    if (!w_max_abs || !smooth) return SQ_ERR_ARG;
    if (!aligned16(w_max_abs) || !aligned16(smooth) || (x_max_abs && !aligned16(x_max_abs))) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    if (!x_max_abs) return launched(sq_launch_fill(smooth, 1.0f, k, s)) == SQ_OK ? SQ_WARN_UNCALIBRATED : SQ_ERR_HIP;
    return launched(sq_launch_smooth_factor(x_max_abs, (const unsigned*)w_max_abs, 1, (double)alpha,
                                            1.0 - (double)alpha, k, smooth, s));
}

sq_status sq_quantize_weight(const void* w, sq_dtype wt, int64_t n, int64_t k, const float* smooth, int8_t* w_q,
                             float* w_scale, void* stream) {
    if (!fp_in(wt)) return SQ_ERR_DTYPE;
    if (n <= 0 || n > kMaxRows) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (!w || !smooth || !w_q || !w_scale) return SQ_ERR_ARG;
    if (!aligned16(w) || !aligned16(smooth) || !aligned16(w_q)) return SQ_ERR_ALIGN;
    return launched(sq_launch_quantize_weight(w, wt == SQ_BF16, smooth, n, k, w_q, w_scale, as_stream(stream)));
}

sq_status sq_reference_linear(const void* x, sq_dtype xt, int64_t m, int64_t k, const void* w, int64_t n,
                              const void* bias, sq_dtype bias_t, void* y, sq_dtype yt, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    if (!(yt == SQ_F32 || yt == SQ_BF16)) return SQ_ERR_DTYPE;
    if (bias && !fp_in(bias_t)) return SQ_ERR_DTYPE;
    if (m < 0 || m > kMaxRows || n <= 0 || n > kMaxRows || !tiles_fit(m, n)) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    if (m == 0) return SQ_OK;
    if (!x || !w || !y) return SQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return SQ_ERR_ALIGN;
    return launched(sq_launch_reference_gemm(x, w, xt == SQ_BF16, m, n, k, bias, bias_kind(bias, bias_t), y,
                                             out_kind(yt), as_stream(stream)));
}

size_t sq_relative_error_workspace_bytes(int64_t count) {
    return count <= 0 ? 0 : (size_t)16 * (size_t)sq_relative_error_blocks(count);
}

sq_status sq_relative_error(const float* y_fp, const float* y_q, int64_t count, void* workspace,
                            size_t workspace_bytes, double* result, void* stream) {
    if (count <= 0) return SQ_ERR_SHAPE;
    if (!y_fp || !y_q || !result) return SQ_ERR_ARG;
    if (!workspace || workspace_bytes < sq_relative_error_workspace_bytes(count)) return SQ_ERR_WORKSPACE;
    if (!aligned16(y_fp) || !aligned16(y_q) || ((uintptr_t)workspace & 7u) != 0 || ((uintptr_t)result & 7u) != 0)
        return SQ_ERR_ALIGN;
    return launched(sq_launch_relative_error(y_fp, y_q, count, (double*)workspace, result, as_stream(stream)));
}

sq_status sq_selfcheck_reciprocal(unsigned long long* mismatches, void* stream) {
    if (!mismatches) return SQ_ERR_ARG;
    if (((uintptr_t)mismatches & 7u) != 0) return SQ_ERR_ALIGN;
    return launched(sq_launch_selfcheck_reciprocal(mismatches, as_stream(stream)));
}

sq_status sq_selfcheck_division(unsigned b_begin, unsigned b_end, unsigned long long* mismatches,
                                void* stream) {
    if (!mismatches) return SQ_ERR_ARG;
    if (((uintptr_t)mismatches & 7u) != 0) return SQ_ERR_ALIGN;
    if (b_begin > b_end || b_end > (1u << 23)) return SQ_ERR_SHAPE;
    return launched(sq_launch_selfcheck_division(b_begin, b_end, mismatches, as_stream(stream)));
}

// sq_w8a8_linear_tiled's workspace: the tiled codes, then the scales.
// sq_w8a8_linear_tiled_fused's: its synchronisation words first (a fixed
// place, whatever m), then the same.
namespace {
constexpr size_t kFusedSyncBytes = 1024;  // at least sq_stream_fused_sync_bytes()
std::atomic<int> g_fused_wait_polls{4096};

sq_status check_linear_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                             const int8_t* w_q, const float* w_scale, int64_t n, const void* bias, sq_dtype bias_t,
                             const void* y, sq_dtype yt, const void* workspace, size_t workspace_bytes, size_t need) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    sq_status st = check_gemm(w_q, w_scale, m, w_q, w_scale, n, k, bias, bias_t, y, yt);
    if (st != SQ_OK || m == 0) return st;
    if (!x || !smooth) return SQ_ERR_ARG;
    if (!workspace || workspace_bytes < need) return SQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return SQ_ERR_ALIGN;
    if (!aligned16(x) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    return SQ_OK;
}
}  // namespace

size_t sq_w8a8_linear_tiled_workspace_bytes(int64_t m, int64_t k) {
    if (m <= 0 || k <= 0) return 0;
    return round_up(sq_tiled_bytes(m, k), 256) + 4 * (size_t)m;
}

sq_status sq_w8a8_linear_tiled(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                               const int8_t* w_q, const float* w_scale, int64_t n, const void* bias, sq_dtype bias_t,
                               void* y, sq_dtype yt, void* workspace, size_t workspace_bytes, void* stream) {
    sq_status st = check_linear_tiled(x, xt, m, k, smooth, w_q, w_scale, n, bias, bias_t, y, yt, workspace,
                                      workspace_bytes, sq_w8a8_linear_tiled_workspace_bytes(m, k));
    if (st != SQ_OK || m == 0) return st;
    int8_t* xq = (int8_t*)workspace;
    float* xs = (float*)((char*)workspace + round_up(sq_tiled_bytes(m, k), 256));
    hipStream_t s = as_stream(stream);
    hipError_t e = sq_launch_quantize_act_tiled(x, xt == SQ_BF16, smooth, m, k, xq, xs, s);
    if (e == hipSuccess)
        e = sq_launch_gemm_tiled(xq, xs, m, w_q, w_scale, n, k, bias, bias_kind(bias, bias_t), y, out_kind(yt), 0, s);
    return launched(e);
}

size_t sq_w8a8_linear_tiled_fused_workspace_bytes(int64_t m, int64_t k) {
    if (m <= 0 || k <= 0) return 0;
    return kFusedSyncBytes + sq_w8a8_linear_tiled_workspace_bytes(m, k);
}

void sq_set_fused_wait_polls(int polls) { g_fused_wait_polls.store(polls < 0 ? 0 : polls, std::memory_order_relaxed); }

sq_status sq_w8a8_linear_tiled_fused(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                                     const int8_t* w_q, const float* w_scale, int64_t n, const void* bias,
                                     sq_dtype bias_t, void* y, sq_dtype yt, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    if (m > kStreamMaxM) return SQ_ERR_SHAPE;
    sq_status st = check_linear_tiled(x, xt, m, k, smooth, w_q, w_scale, n, bias, bias_t, y, yt, workspace,
                                      workspace_bytes, sq_w8a8_linear_tiled_fused_workspace_bytes(m, k));
    if (st != SQ_OK || m == 0) return st;
    static_assert(kFusedSyncBytes % 256 == 0, "the codes stay 256-byte aligned");
    if (sq_stream_fused_sync_bytes() > kFusedSyncBytes) return SQ_ERR_HIP;
    char* base = (char*)workspace;
    int8_t* xq = (int8_t*)(base + kFusedSyncBytes);
    float* xs = (float*)(base + kFusedSyncBytes + round_up(sq_tiled_bytes(m, k), 256));
    return launched(sq_launch_linear_stream_fused(x, xt == SQ_BF16, smooth, m, k, xq, xs, w_q, w_scale, n, bias,
                                                  bias_kind(bias, bias_t), y, out_kind(yt), base,
                                                  g_fused_wait_polls.load(std::memory_order_relaxed),
                                                  as_stream(stream)));
}

size_t sq_w8a8_linear_workspace_bytes(int64_t m, int64_t k) {
    if (m <= 0 || k <= 0) return 0;
    return round_up((size_t)m * (size_t)k, 256) + 4 * (size_t)m;
}

sq_status sq_w8a8_linear(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                         const int8_t* w_q, const float* w_scale, int64_t n, const void* bias, void* y,
                         sq_dtype yt, void* workspace, size_t workspace_bytes, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    // the workspace holds the codes, so check it as the gemm's x_q
    int8_t* xq = (int8_t*)workspace;
    float* xs = workspace ? (float*)((char*)workspace + round_up((size_t)(m > 0 ? m : 0) * (size_t)(k > 0 ? k : 0), 256))
                          : nullptr;
    sq_status st = check_gemm(xq ? xq : (const int8_t*)w_q, w_scale, m, w_q, w_scale, n, k, bias, xt, y, yt);
    if (st != SQ_OK || m == 0) return st;
    if (!x || !smooth) return SQ_ERR_ARG;
    if (!workspace || workspace_bytes < sq_w8a8_linear_workspace_bytes(m, k)) return SQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return SQ_ERR_ALIGN;
    if (!aligned16(x) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    hipError_t e = sq_launch_quantize_act(x, xt == SQ_BF16, smooth, m, k, xq, xs, s);
    if (e == hipSuccess)
        e = sq_launch_gemm(xq, xs, m, w_q, w_scale, n, k, bias, bias_kind(bias, xt), y, out_kind(yt), 0, s);
    return launched(e);
}

// ---------------------------------------------------------------------------
// The learnable alpha and the straight-through backward
// ---------------------------------------------------------------------------
float sq_alpha_from_eta(float eta) { return (float)(1.0 / (1.0 + exp(-(double)eta))); }

float sq_eta_from_alpha(double alpha) {
    const double d = 1.0 - alpha;
    return (float)log(alpha / (d > 1e-6 ? d : 1e-6));
}

size_t sq_ste_backward_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m <= 0 || n <= 0 || k <= 0 || m > SQ_STE_MAX_ROWS || n > SQ_STE_MAX_ROWS || k > SQ_MAX_K) return 0;
    return sq_ste_layout(m, n, k).bytes;
}

sq_status sq_ste_backward(const void* dy, sq_dtype dyt, int64_t m, int64_t n, int64_t k, const void* x, sq_dtype xt,
                          const void* w, sq_dtype wt, const float* smooth, const int8_t* x_q, const float* x_scale,
                          const int8_t* w_q, const float* w_scale, const float* x_max_abs, const float* w_max_abs,
                          float alpha, float* dx, float* dw, float* dbias, float* dsmooth, double* dalpha_deta,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (!fp_in(dyt) || !fp_in(xt) || !fp_in(wt)) return SQ_ERR_DTYPE;
    if (m <= 0 || n <= 0 || m > SQ_STE_MAX_ROWS || n > SQ_STE_MAX_ROWS) return SQ_ERR_SHAPE;
    sq_status st = check_k(k);
    if (st != SQ_OK) return st;
    // the products' tile grids and the transposes' grids (64 x 64 tiles)
    if (!tiles_fit(m, k) || !tiles_fit(n, k)) return SQ_ERR_SHAPE;
    if (((m + 63) / 64) * ((n + 63) / 64) > kMaxTiles || ((m + 63) / 64 + (n + 63) / 64) * ((k + 63) / 64) > kMaxTiles)
        return SQ_ERR_SHAPE;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ARG;
    if (!dy || !x || !w || !smooth || !x_q || !x_scale || !w_q || !w_scale || !dx || !dw || !dalpha_deta)
        return SQ_ERR_ARG;
    if (x_max_abs && !w_max_abs) return SQ_ERR_ARG;
    if (!workspace || workspace_bytes < sq_ste_backward_workspace_bytes(m, n, k)) return SQ_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(x_q) || !aligned16(w_q) || !aligned16(dx) || !aligned16(dw))
        return SQ_ERR_ALIGN;
    if (((uintptr_t)dy & (dyt == SQ_BF16 ? 1u : 3u)) != 0 || ((uintptr_t)workspace & 255u) != 0 ||
        ((uintptr_t)dalpha_deta & 7u) != 0)
        return SQ_ERR_ALIGN;
    hipError_t e = sq_launch_ste_backward(dy, dyt == SQ_BF16, m, n, k, x, xt == SQ_BF16, w, wt == SQ_BF16, smooth,
                                          x_q, x_scale, w_q, w_scale, x_max_abs, w_max_abs, (double)alpha, dx, dw,
                                          dbias, dsmooth, dalpha_deta, workspace, as_stream(stream));
    if (e != hipSuccess) return SQ_ERR_HIP;
    return x_max_abs ? SQ_OK : SQ_WARN_UNCALIBRATED;
}

size_t sq_aux_loss_grad_workspace_bytes(int64_t count) {
    return count <= 0 ? 0 : sq_relative_error_workspace_bytes(count) + 256;
}

sq_status sq_aux_loss_grad(const float* y_fp, const float* y_q, int64_t count, float* dy_q, double* loss,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (count <= 0) return SQ_ERR_SHAPE;
    if (!y_fp || !y_q || !dy_q || !loss) return SQ_ERR_ARG;
    if (!workspace || workspace_bytes < sq_aux_loss_grad_workspace_bytes(count)) return SQ_ERR_WORKSPACE;
    if (!aligned16(y_fp) || !aligned16(y_q) || ((uintptr_t)dy_q & 3u) != 0 || ((uintptr_t)workspace & 255u) != 0 ||
        ((uintptr_t)loss & 7u) != 0)
        return SQ_ERR_ALIGN;
    double* norms = (double*)workspace;  // [3], then the partial sums
    double* partial = (double*)((char*)workspace + 256);
    return launched(sq_launch_aux_loss_grad(y_fp, y_q, count, partial, norms, dy_q, loss, as_stream(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// sq_w8a8_linear_noalloc: sq_w8a8_linear with its workspace (the activation
// codes and scales) in a fixed device array of this library instead of
// caller memory. Every GPU the library runs on holds its own copy of the
// array from the library's load until the process ends; every call on one
// GPU shares it (the codes and scales of the last call stay there), so calls
// that overlap on one GPU race. Nothing in it needs clearing: each call
// writes every code and scale it reads.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchCodes = SQ_NOALLOC_MAX_CODES;        // x_q bytes
constexpr size_t kScratchScales = 4 * SQ_NOALLOC_MAX_TOKENS;  // x_scale bytes

static __device__ __align__(256) unsigned char scratch[kScratchCodes + kScratchScales];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The device address of this GPU's copy of `scratch` (the array's name in
// host code is only a host-side stand-in), looked up once per device with
// that device current. nullptr on failure.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" sq_status sq_w8a8_linear_noalloc(const void* x, sq_dtype xt, int64_t m, int64_t k, const float* smooth,
                                            const int8_t* w_q, const float* w_scale, int64_t n, const void* bias,
                                            void* y, sq_dtype yt, void* stream) {
    if (!fp_in(xt)) return SQ_ERR_DTYPE;
    sq_status st = check_gemm(w_q, w_scale, m, w_q, w_scale, n, k, bias, xt, y, yt);
    if (st != SQ_OK || m == 0) return st;
    if (!x || !smooth) return SQ_ERR_ARG;
    if (m > SQ_NOALLOC_MAX_TOKENS || (uint64_t)m * (uint64_t)k > (uint64_t)SQ_NOALLOC_MAX_CODES)
        return SQ_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(smooth)) return SQ_ERR_ALIGN;
    char* base = (char*)scratch_on_current_device();
    if (!base) return SQ_ERR_HIP;
    int8_t* xq = (int8_t*)base;
    float* xs = (float*)(base + kScratchCodes);
    hipStream_t s = as_stream(stream);
    hipError_t e = sq_launch_quantize_act(x, xt == SQ_BF16, smooth, m, k, xq, xs, s);
    if (e == hipSuccess)
        e = sq_launch_gemm(xq, xs, m, w_q, w_scale, n, k, bias, bias_kind(bias, xt), y, out_kind(yt), 0, s);
    return launched(e);
}
