// sq_quant.hip -- the HBM-bound steps of the SmoothQuant W8A8 linear
// (page "w8a8_smoothquant.py", BiGRU_T_version):
//   * column max-abs reduction (SmoothQuantW8A8.calibrate's running max, and
//     calibrate_smoothquant's max over output rows of |W|);
//   * the smoothing factor s (calibrate_smoothquant), fused into the last
//     stage of the weight column max;
//   * smoothing + symmetric int8 of rows: weights W * s with one scale per
//     output channel (freeze_quantization -> quantize_per_channel_symmetric)
//     and activations X / s with one scale per token (forward ->
//     quantize_per_token_symmetric).
#include "../../include/sq.h"
#include "sq_device.h"

using namespace sq;

// max of the two 16-bit halves of a and b, independently (magnitudes of
// bf16 pairs: integer order is value order)
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    const uint32_t lo = max(a & 0xffffu, b & 0xffffu);
    const uint32_t hi = max(a >> 16, b >> 16);
    return lo | (hi << 16);
}

// ---------------------------------------------------------------------------
// fill
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, float v, int64_t count) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = v;
}

hipError_t sq_launch_fill(float* p, float v, int64_t count, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    unsigned blocks = (unsigned)((count + 255) / 256);
    hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, st, p, v, count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The rows of a column max's input, handed out as runs of consecutive rows
// of one buffer: runs(r0, r1, f) calls f(p, count) for each run within rows
// [r0, r1), p pointing at the run's first row (kvec u32x4 chunks per row).
// One matrix is a single run; several calibration batches are taken as one
// sequence of rows, a run per batch that the row range meets.
// ---------------------------------------------------------------------------
struct OneMatrix {
    const u32x4* x;
    int64_t kvec;
    template <class F>
    __device__ __forceinline__ void runs(int64_t r0, int64_t r1, F&& f) const {
        f(x + r0 * kvec, r1 - r0);
    }
};

struct BatchRows {
    const u32x4* x[SQ_MAX_CALIB_BATCHES];
    // one past batch b's last row in the sequence; entries past the last
    // batch hold the total, so they make no run
    int64_t end[SQ_MAX_CALIB_BATCHES];
    int64_t kvec;
    // the bounds are the same for the whole block (scalar registers), and
    // the loop is unrolled so that the table is never indexed at run time
    template <class F>
    __device__ __forceinline__ void runs(int64_t r0, int64_t r1, F&& f) const {
        int64_t start = 0;
#pragma unroll
        for (int b = 0; b < SQ_MAX_CALIB_BATCHES; ++b) {
            const int64_t lo = max(r0, start), hi = min(r1, end[b]);
            if (lo < hi) f(x[b] + (lo - start) * kvec, hi - lo);
            start = end[b];
        }
    }
};

// ---------------------------------------------------------------------------
// Column max of |x| over a group of rows.
// Block = 4 wavefronts over one strip of 64 / L 16-byte column chunks; a
// load instruction of a wavefront covers L rows of the strip (64 / L lanes
// per row), and wavefront w takes row steps w, w+4, ... of each run of the
// group's rows with 8 loads in flight (L > 1 spreads a short batch over more blocks); the
// partial maxima meet in LDS. |x| >= 0, so the order of the binary32 bit
// patterns as unsigned integers is the order of the values: every max is an
// exact integer max, independent of order.
//   FOLD:    out[j] = max(out[j], max) -- one row group: the owning thread
//            updates in place (or, with `overwrite`, writes the max without
//            reading out: a first calibration batch); several: integer
//            atomicMax (the running max of calibration keeps its value
//            across calls);
//   PARTIAL: out[g * k + j] = max over row group g (plain stores).
// ---------------------------------------------------------------------------
template <bool BF16, bool FOLD, int L, class Src>
__global__ __launch_bounds__(256) void colmax_kernel(Src src, int64_t rows, int64_t kvec,
                                                     int64_t rows_per_group, int64_t k,
                                                     unsigned* __restrict__ out, int overwrite) {
    constexpr int U = 8;
    constexpr int W = 64 / L;  // chunks per strip
    __shared__ u32x4 red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * W + lane % W;
    const int sub = lane / W;  // row within the instruction's L rows
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_group;
    const int64_t r1 = min(r0 + rows_per_group, rows);
    constexpr uint32_t kMask = BF16 ? 0x7fff7fffu : 0x7fffffffu;
    u32x4 m = {0, 0, 0, 0};
    auto merge = [&](u32x4& acc, u32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) acc[i] = max_u16x2(acc[i], v[i]);
            else acc[i] = max(acc[i], v[i]);
        }
    };
    auto fold = [&](u32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] &= kMask;
        merge(m, v);
    };
    if (c < kvec) {
        constexpr int STEP = 4 * L;  // rows per round of the 4 wavefronts
        src.runs(r0, r1, [&](const u32x4* p, int64_t count) {
            int64_t r = wave * L + sub;
            for (; r + STEP * (U - 1) < count; r += STEP * U) {
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = p[(r + STEP * u) * kvec + c];
#pragma unroll
                for (int u = 0; u < U; ++u) fold(v[u]);
            }
            for (; r < count; r += STEP) fold(p[r * kvec + c]);
        });
    }
    red[wave][lane] = m;
    __syncthreads();
    if (wave != 0 || lane >= W || c >= kvec) return;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int j = 0; j < L; ++j)
            if (w | j) merge(m, red[w][lane + j * W]);
    // the chunk's columns as binary32 bit patterns
    constexpr int NC = BF16 ? 8 : 4;
    uint32_t val[NC];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
            val[2 * i] = m[i] << 16;
            val[2 * i + 1] = m[i] & 0xffff0000u;
        } else {
            val[i] = m[i];
        }
    }
    const int64_t col0 = c * NC;
    if constexpr (FOLD) {
        if (gridDim.y == 1) {
#pragma unroll
            for (int i = 0; i < NC; ++i) out[col0 + i] = overwrite ? val[i] : max(out[col0 + i], val[i]);
        } else {
#pragma unroll
            for (int i = 0; i < NC; ++i) atomicMax(out + col0 + i, val[i]);
        }
    } else {
        unsigned* o = out + (int64_t)blockIdx.y * k + col0;
#pragma unroll
        for (int i = 0; i < NC; i += 4) *(u32x4*)(o + i) = u32x4{val[i], val[i + 1], val[i + 2], val[i + 3]};
    }
}

// Row groups for a column max over `rows` rows: enough blocks to keep HBM
// busy (about 1024) but at least 128 rows per group, so that a column gets
// few partial maxima (atomics when folding, partials when reducing).
// rows per load instruction: 4 for a batch of up to 2048 rows (four times
// the blocks, a short batch in flight at once), and for the partial maxima
// (the weights) of rows of at most 512 chunks, which L = 1 splits into only
// 8 strips (256 blocks of 4096 rows, one per CU; paired runs of the whole
// tiled weight preparation, same outputs: 4096 x 4096 29.8 -> 27.9 us,
// 12288 x 4096 91.5 -> 89.2 us, 11008 x 4096 76.5 -> 74.3 us, while longer
// rows measured slower with it); 1 otherwise (measured best)
static int colmax_l(int64_t rows, int64_t kvec, bool partial) {
    return rows <= 2048 || (partial && kvec <= 512) ? 4 : 1;
}

static void colmax_grid(int64_t rows, int64_t kvec, int64_t& gx, int64_t& groups, int64_t& rpg,
                        bool partial = false) {
    const int L = colmax_l(rows, kvec, partial);
    gx = (kvec + 64 / L - 1) / (64 / L);
    int64_t want = 1024 / gx;
    if (want < 1) want = 1;
    groups = (rows + 127) / 128;
    if (groups > want) groups = want;
    if (groups < 1) groups = 1;
    rpg = (rows + groups - 1) / groups;
    groups = (rows + rpg - 1) / rpg;
}

template <bool FOLD, int L>
static void launch_colmax_l(const void* x, int bf16, int64_t rows, int64_t kvec, int64_t k, unsigned* out,
                            int64_t groups, int64_t rpg, int overwrite, hipStream_t st) {
    dim3 grid((unsigned)((kvec + 64 / L - 1) / (64 / L)), (unsigned)groups);
    const OneMatrix src{(const u32x4*)x, kvec};
    if (bf16)
        hipLaunchKernelGGL((colmax_kernel<true, FOLD, L, OneMatrix>), grid, dim3(256), 0, st, src, rows, kvec, rpg,
                           k, out, overwrite);
    else
        hipLaunchKernelGGL((colmax_kernel<false, FOLD, L, OneMatrix>), grid, dim3(256), 0, st, src, rows, kvec, rpg,
                           k, out, overwrite);
}

template <bool FOLD>
static hipError_t launch_colmax(const void* x, int bf16, int64_t rows, int64_t k, unsigned* out, int64_t groups,
                                int64_t rpg, hipStream_t st, int overwrite = 0) {
    const int64_t kvec = bf16 ? k / 8 : k / 4;
    switch (colmax_l(rows, kvec, !FOLD)) {
        case 1: launch_colmax_l<FOLD, 1>(x, bf16, rows, kvec, k, out, groups, rpg, overwrite, st); break;
        default: launch_colmax_l<FOLD, 4>(x, bf16, rows, kvec, k, out, groups, rpg, overwrite, st); break;
    }
    return hipGetLastError();
}

hipError_t sq_launch_colmax(const void* x, int bf16, int64_t rows, int64_t k, float* running_max,
                            hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    int64_t gx, groups, rpg;
    colmax_grid(rows, bf16 ? k / 8 : k / 4, gx, groups, rpg);
    return launch_colmax<true>(x, bf16, rows, k, (unsigned*)running_max, groups, rpg, st);
}

hipError_t sq_launch_colmax_first(const void* x, int bf16, int64_t rows, int64_t k, float* running_max,
                                  hipStream_t st) {
    if (rows <= 0) return sq_launch_fill(running_max, 0.0f, k, st);
    int64_t gx, groups, rpg;
    colmax_grid(rows, bf16 ? k / 8 : k / 4, gx, groups, rpg);
    if (groups == 1)  // one row group: its owners write the max directly
        return launch_colmax<true>(x, bf16, rows, k, (unsigned*)running_max, 1, rpg, st, 1);
    // several row groups fold with atomics into a zeroed buffer
    hipError_t e = sq_launch_fill(running_max, 0.0f, k, st);
    if (e != hipSuccess) return e;
    return launch_colmax<true>(x, bf16, rows, k, (unsigned*)running_max, groups, rpg, st);
}

// Several calibration batches in one launch, read as one run of rows with
// the row groups of one matrix of that many rows (a group may span
// batches). When the run starts the max and has several row groups, a zero
// fill comes first and the groups fold with atomics. (One row group of
// narrow strips, or wider blocks over all rows, would need no fill; both
// measured slower on four batches of 128 tokens.)
template <int L>
static void launch_colmax_batches_l(const BatchRows& src, int bf16, int64_t total, int64_t kvec, int64_t rpg,
                                    int64_t groups, int64_t k, unsigned* out, int overwrite, hipStream_t st) {
    dim3 grid((unsigned)((kvec + 64 / L - 1) / (64 / L)), (unsigned)groups);
    if (bf16)
        hipLaunchKernelGGL((colmax_kernel<true, true, L, BatchRows>), grid, dim3(256), 0, st, src, total, kvec, rpg,
                           k, out, overwrite);
    else
        hipLaunchKernelGGL((colmax_kernel<false, true, L, BatchRows>), grid, dim3(256), 0, st, src, total, kvec,
                           rpg, k, out, overwrite);
}

hipError_t sq_launch_colmax_batches(const void* const* x, const int64_t* rows, int nbatch, int bf16, int64_t k,
                                    float* running_max, int first, hipStream_t st) {
    const int64_t kvec = bf16 ? k / 8 : k / 4;
    BatchRows src{};
    src.kvec = kvec;
    int64_t total = 0;
    for (int b = 0; b < SQ_MAX_CALIB_BATCHES; ++b) {
        if (b < nbatch) {
            src.x[b] = (const u32x4*)x[b];
            total += rows[b];
        }
        src.end[b] = total;
    }
    if (total == 0) return first ? sq_launch_fill(running_max, 0.0f, k, st) : hipSuccess;
    // a single batch with rows: the one-matrix kernel (a smaller argument
    // block, the same grid)
    for (int b = 0; b < nbatch; ++b) {
        if (rows[b] == total)
            return first ? sq_launch_colmax_first(x[b], bf16, total, k, running_max, st)
                         : sq_launch_colmax(x[b], bf16, total, k, running_max, st);
    }
    int64_t gx, groups, rpg;
    colmax_grid(total, kvec, gx, groups, rpg);
    int overwrite = 0;
    if (first) {
        if (groups == 1) {
            overwrite = 1;  // its owners write each column's max directly
        } else {
            hipError_t e = sq_launch_fill(running_max, 0.0f, k, st);
            if (e != hipSuccess) return e;
        }
    }
    unsigned* out = (unsigned*)running_max;
    if (colmax_l(total, kvec, false) == 4)
        launch_colmax_batches_l<4>(src, bf16, total, kvec, rpg, groups, k, out, overwrite, st);
    else
        launch_colmax_batches_l<1>(src, bf16, total, kvec, rpg, groups, k, out, overwrite, st);
    return hipGetLastError();
}

int64_t sq_colmax_partial_groups(int64_t rows, int64_t k, int bf16, int64_t scratch_bytes) {
    int64_t gx, groups, rpg;
    colmax_grid(rows, bf16 ? k / 8 : k / 4, gx, groups, rpg, true);
    const int64_t fit = scratch_bytes / (4 * k);
    if (groups > fit) groups = fit < 1 ? 1 : fit;
    return groups;
}

hipError_t sq_launch_colmax_partial(const void* x, int bf16, int64_t rows, int64_t k, int64_t groups,
                                    unsigned* partial, hipStream_t st) {
    // exactly `groups` row groups are written (a trailing group past the
    // last row writes zeros, neutral for the max of non-negative values)
    const int64_t rpg = (rows + groups - 1) / groups;
    return launch_colmax<false>(x, bf16, rows, k, partial, groups, rpg, st);
}

// ---------------------------------------------------------------------------
// Smoothing factor, per input channel j (calibrate_smoothquant), from the
// per-row-group column maxima of |W|:
//   mw_j = max(max_g partial[g][j], floor),  mx_j = max(x_max[j], floor)
//   s_j  = max(f32(P(mx_j, a_x)) / f32(P(mw_j, a_w)), floor)
// P(x, a) = x^a through binary64: exact forms built from correctly rounded
// sqrt for a in {0, 1/4, 1/2, 3/4, 1}, pow otherwise.
// A block owns 64 channels; its 4 wavefronts split the row groups (8 loads
// in flight each) and meet in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void smooth_factor_kernel(const float* __restrict__ x_max,
                                                            const unsigned* partial, int64_t groups, double a_x,
                                                            double a_w, int64_t k, float* s) {
    __shared__ unsigned red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + lane;
    unsigned mwb = 0;
    if (j < k) {
        int64_t g = wave;
        for (; g + 28 < groups; g += 32) {
            unsigned v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = partial[(g + 4 * u) * k + j];
#pragma unroll
            for (int u = 0; u < 8; ++u) mwb = max(mwb, v[u]);
        }
        for (; g < groups; g += 4) mwb = max(mwb, partial[g * k + j]);
    }
    red[wave][lane] = mwb;
    __syncthreads();  // every partial is read before s (which may alias it) is written
    if (wave != 0 || j >= k) return;
    mwb = max(max(red[0][lane], red[1][lane]), max(red[2][lane], red[3][lane]));
    const float mw = fmaxf(__uint_as_float(mwb), kFloor);
    const float mx = fmaxf(x_max[j], kFloor);
    const float num = (float)pow64((double)mx, a_x);
    const float den = (float)pow64((double)mw, a_w);
    s[j] = fmaxf(num / den, kFloor);
}

hipError_t sq_launch_smooth_factor(const float* x_max, const unsigned* partial, int64_t groups, double a_x,
                                   double a_w, int64_t k, float* s, hipStream_t st) {
    unsigned blocks = (unsigned)((k + 63) / 64);
    hipLaunchKernelGGL(smooth_factor_kernel, dim3(blocks), dim3(256), 0, st, x_max, partial, groups, a_x, a_w, k,
                       s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rows -> int8 codes with one scale per row, for both sides of the product:
//   weights (DIV = false):     v[j] = f32(w[j] * s_j)
//   activations (DIV = true):  v[j] = f32(x[j] / s_j)
//   scale = max(max_j |v[j]|, floor) / 127
//   q[j]  = round_half_even(v[j] / scale)
//
// Division. For a binary32 quotient a / b the kernels use y = RN(1/b),
// q0 = RN(a y), q1 = fma(fma(-q0, b, a), y, q0): Markstein's correction
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev. 34(1), 1990). With y the
// correctly rounded reciprocal and q0 within an ulp of a / b, the residual
// a - q0 b is exact in one fma and q0 + residual * y rounds to the correctly
// rounded quotient. Here that is not taken on trust: on gfx950 q1 equals the
// IEEE quotient RN(a/b) for every pair of binary32 significands (2^46
// pairs, checked on the device by sq_selfcheck_division); as every step is
// one correctly rounded operation, powers of two scale it exactly, so it
// holds for all operands as long as no step under- or overflows.
//   * x / s_j: y_j = RN(1/s_j) comes from recip_rn (also checked against
//     IEEE 1/s on the device, sq_selfcheck_reciprocal) for s_j in
//     [2^-40, 2^40), else NaN. For 2^-50 <= |q0| <= 2^120 (then
//     |x| >= 2^-90) or q0 = 0 no step leaves the normal range, so q1 is the
//     IEEE quotient. Where |q0| < 2^-50 a step may underflow and q1 may
//     differ from it, but both are below 2^-49 in magnitude, and such a
//     value changes no output: its code is 0 (the row scale is at least
//     floor / 127, about 2^-33.6), and it sets the row max only if every
//     quotient of the row is that small, when both maxima are below the
//     floor and the scale is floor / 127 either way. So the only guard is
//     on the other side, checked once per row and thread on the largest
//     |q0| (an infinite x gives q0 = inf): above 2^120, or where a y is
//     NaN, the thread's out-of-range quotients are recomputed with the IEEE
//     division. A NaN x gives NaN on both routes.
//   * scale = RN(max / 127) by the same correction with y = RN(1/127) (an
//     infinite max passes through), and rs = RN(1 / scale) by the refined
//     reciprocal below 2^100, the IEEE quotient above: both equal the IEEE
//     results, so the scale is the binary32 quotient the method defines.
//   * v / scale: scale is in [2^-34, 2^122] (floor / 127 up to max / 127)
//     and |v / scale| <= 127.00002, so no step overflows; a step can only
//     underflow when |v| < 2^-90, where the quotient is below 2^-50 and its
//     code is 0 either way. The code is then rint(quotient), computed by
//     adding 1.5 * 2^23 (round to nearest even into the low mantissa bits,
//     whose low byte is the two's complement code); |quotient| <= 127.00002
//     rounds into [-127, 127].
//
// Layout. A block of T threads owns a row at a time and walks a few rows
// with a grid stride. Thread t owns the 8-channel chunks t, t + T, ... (C
// of them) and keeps their s (and y) in registers; the row stays in
// registers between the max and the codes, so the input is read once; a
// further row's loads are issued before the current row is finished. One
// barrier per row (the block max goes through a double-buffered LDS slot);
// the wavefront max is taken by DPP and lane reads, not through LDS. The
// per-row work is done by every thread: done with the IEEE divisions and an
// LDS shuffle it made the activation quantiser 9% slower at 4096 x 4096.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void selfcheck_reciprocal_kernel(unsigned long long* mismatches) {
    const unsigned long long idx = (unsigned long long)blockIdx.x * 256 + threadIdx.x;
    const unsigned e = (unsigned)(idx >> 23), mant = (unsigned)(idx & 0x7fffffu);
    if (e >= 200) return;
    const float s = __uint_as_float(((e + 27u) << 23) | mant);  // 2^-100 .. 2^100
    const float r = __builtin_amdgcn_rcpf(s);
    const float y = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    if (__float_as_uint(y) != __float_as_uint(1.0f / s)) atomicAdd(mismatches, 1ull);
}

hipError_t sq_launch_selfcheck_reciprocal(unsigned long long* mismatches, hipStream_t st) {
    const unsigned long long total = 200ull << 23;
    hipLaunchKernelGGL(selfcheck_reciprocal_kernel, dim3((unsigned)(total / 256)), dim3(256), 0, st, mismatches);
    return hipGetLastError();
}

// divisor significands [b_begin, b_end) against every numerator significand
__global__ __launch_bounds__(256) void selfcheck_division_kernel(unsigned b_begin, unsigned b_end,
                                                                 unsigned long long* mismatches) {
    const unsigned bm = b_begin + blockIdx.x * 256 + threadIdx.x;
    if (bm >= b_end) return;
    const float b = __uint_as_float(0x3f800000u | bm);
    const float y = 1.0f / b;
    unsigned long long bad = 0;
    for (unsigned am = 0; am < (1u << 23); ++am) {
        const float a = __uint_as_float(0x3f800000u | am);
        if (__float_as_uint(div_rn(a, b, y)) != __float_as_uint(a / b)) ++bad;
    }
    if (bad) atomicAdd(mismatches, bad);
}

hipError_t sq_launch_selfcheck_division(unsigned b_begin, unsigned b_end, unsigned long long* mismatches,
                                        hipStream_t st) {
    if (b_end <= b_begin) return hipSuccess;
    hipLaunchKernelGGL(selfcheck_division_kernel, dim3((b_end - b_begin + 255) / 256), dim3(256), 0, st, b_begin,
                       b_end, mismatches);
    return hipGetLastError();
}


// TILED: the codes go to 16 x 64 tiles (rows in groups of 16, K in 64-byte
// chunks, tile (g, c) at (g * K64 / 64 + c) * 1 KiB, each tile row-major;
// K64 = k rounded up to 64), the padding columns of every row written as
// zero codes.
template <bool BF16, bool DIV, int T, int C, bool TILED>
__global__ __launch_bounds__(T) void quantize_rows_kernel(const void* __restrict__ x, const float* __restrict__ s,
                                                          int64_t m, int64_t k, int8_t* __restrict__ q,
                                                          float* __restrict__ scale_out) {
    static_assert(T % 64 == 0, "whole wavefronts: the block max goes through one LDS slot per wavefront");
    constexpr int NW = T / 64;
    constexpr int kV = BF16 ? 1 : 2;  // 16-byte loads per 8 channels
    __shared__ float red[2][NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t k8 = k >> 3;

    float sv[C][8], yv[DIV ? C : 1][8];
    bool y_bad = false;  // a factor outside the fast reciprocal's range
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t j8 = (int64_t)c * T + tid;
        if (j8 < k8) {
            const u32x4 a = *(const u32x4*)(s + j8 * 8);
            const u32x4 b = *(const u32x4*)(s + j8 * 8 + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sv[c][i] = __uint_as_float(a[i]);
                sv[c][4 + i] = __uint_as_float(b[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) sv[c][i] = 1.0f;
        }
        if constexpr (DIV) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                yv[c][i] = recip_rn(sv[c][i]);
                y_bad |= __builtin_isnan(yv[c][i]);
            }
        }
    }

    u32x4 raw[C][kV];
    auto load_row = [&](int64_t row) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j8 = (int64_t)c * T + tid;
            if (row < m && j8 < k8) {
                const u32x4* p = BF16 ? (const u32x4*)((const uint16_t*)x + row * k + j8 * 8)
                                      : (const u32x4*)((const float*)x + row * k + j8 * 8);
#pragma unroll
                for (int v = 0; v < kV; ++v) raw[c][v] = p[v];
            } else {
#pragma unroll
                for (int v = 0; v < kV; ++v) raw[c][v] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto unpack = [&](int c, float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) {
                v[2 * i] = bf16_lo(raw[c][0][i]);
                v[2 * i + 1] = bf16_hi(raw[c][0][i]);
            } else {
                v[i] = __uint_as_float(raw[c][0][i]);
                v[4 + i] = __uint_as_float(raw[c][1][i]);
            }
        }
    };
    // the fast quotient's proven range (q0 = 0 is exact as well)
    auto in_range = [](float q0) {
        const float a0 = __builtin_fabsf(q0);
        return a0 >= 0x1p-50f && a0 <= 0x1p120f;
    };

    int64_t row = blockIdx.x;
    load_row(row);
    for (int parity = 0; row < m; row += gridDim.x, parity ^= 1) {
        float xs[C][8];
        float qmax = 0.0f;  // largest |q0| of the thread's quotients (NaN ignored)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float v[8];
            unpack(c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (DIV) {
                    xs[c][i] = div_rn(v[i], sv[c][i], yv[c][i]);
                    qmax = fmaxf(qmax, __builtin_fabsf(v[i] * yv[c][i]));
                } else {
                    xs[c][i] = v[i] * sv[c][i];
                }
            }
        }
        if constexpr (DIV) {
            // one branch per row, never taken for sane inputs
            if (y_bad || !(qmax <= 0x1p120f)) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    float v[8];
                    unpack(c, v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float q0 = v[i] * yv[c][i];
                        if (!in_range(q0) && q0 != 0.0f) xs[c][i] = v[i] / sv[c][i];
                    }
                }
            }
        }
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, __builtin_fabsf(xs[c][i]));
        // the next row's loads are in flight while this row finishes
        load_row(row + gridDim.x);
        mx = wave_max_nonneg(mx);
        if (lane == 0) red[parity][wave] = mx;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[parity][w]);
        const float scale = row_scale(fmaxf(mx, kFloor));
        const float rs = row_scale_recip(scale);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j8 = (int64_t)c * T + tid;
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = __float_as_uint(div_rn(xs[c][i], scale, rs) + kMagic);
            const u32x2 codes = u32x2{pack_low_bytes(b[0], b[1], b[2], b[3]), pack_low_bytes(b[4], b[5], b[6], b[7])};
            if constexpr (TILED) {
                // streaming stores: the codes are not read again here (the
                // weight preparation measured 0.5 us faster at 4096 x 4096)
                const int64_t k64 = (k + 63) & ~(int64_t)63;
                if (j8 < (k64 >> 3))
                    __builtin_nontemporal_store(
                        j8 < k8 ? codes : u32x2{0u, 0u},
                        (u32x2*)(q + ((row >> 4) * (k64 >> 6) + (j8 >> 3)) * 1024 + (row & 15) * 64 + (j8 & 7) * 8));
            } else {
                if (j8 < k8) *(u32x2*)(q + row * k + j8 * 8) = codes;
            }
        }
        if (tid == 0) scale_out[row] = scale;
    }
}

template <bool BF16, bool DIV, bool TILED = false>
static hipError_t launch_rows(const void* x, const float* s, int64_t m, int64_t k, int8_t* q, float* scale,
                              hipStream_t st) {
    // threads per row T and 8-channel chunks per thread C, with T * C * 8 >= k
    const int64_t k8 = k / 8;
    int T, C;
    if (k8 <= 512) {
        T = 256; C = k8 <= 256 ? 1 : 2;
        // few rows (one block each, latency-bound): one chunk per thread
        // shortens each row's chain (16 x 4096: 3.3 -> 3.0 us in paired runs)
        if (m < 256 && C == 2) { T = 512; C = 1; }
    }
    else if (k8 <= 1024) { T = 512; C = 2; }
    else if (k8 <= 1408) {
        // many rows: 8 wavefronts with 3 chunks each beat 6 with 4 and 11
        // with 2 (paired runs over rotated sets, 11008 channels, tiled
        // activation codes: 4096 rows 28.0 -> 25.9 us, 1024 rows 15.8 ->
        // 13.9 us; weights level or better); few rows: the wider block's
        // shorter chain per row wins (256 rows: 6.2 against 6.3 and 7.5 us)
        if (m >= 1024) { T = 512; C = 3; }
        else { T = 704; C = 2; }
    }
    else if (k8 <= 1536) { T = 512; C = 3; }
    else if (k8 <= 2048) { T = 1024; C = 2; }
    else return hipErrorInvalidValue;
    // several rows per block (walked with a grid stride): the next row's
    // loads overlap the current row's arithmetic, and the smoothing factors
    // are loaded once per block. Rows up to 4096 channels: 2 per block (1 for
    // fewer than 1024 rows, which are latency-bound; 4 from 8192 rows on:
    // paired runs of the tiled weight preparation on two boxes, same
    // outputs, 12288 x 4096 87.0 -> 81.5 and 88.1 -> 81.6 us, 11008 x 4096
    // 72.4 -> 71.3 and 72.8 -> 70.1 us, while 4096 rows keep 2); longer rows: up to 16 (the factors' load stays well below the
    // rows' own bytes), but no fewer blocks than CUs. Measured best on MI355X.
    int64_t rows_per_block = m >= 8192 ? 4 : (m >= 1024 ? 2 : 1);  // few rows: one block each
    if (k8 > 512) rows_per_block = m >= 16 * 256 ? 16 : (m >= 256 ? m / 256 : 1);
    int64_t blocks = (m + rows_per_block - 1) / rows_per_block;
    if (blocks > 16384) blocks = 16384;
    dim3 grid((unsigned)blocks), block(T);
#define SQ_ROWS_CASE(TT, CC)                                                                                  \
    if (T == TT && C == CC) {                                                                                 \
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, DIV, TT, CC, TILED>), grid, block, 0, st, x, s, m, k, q, scale); \
        return hipGetLastError();                                                                             \
    }
    SQ_ROWS_CASE(256, 1) SQ_ROWS_CASE(256, 2) SQ_ROWS_CASE(512, 1) SQ_ROWS_CASE(512, 2) SQ_ROWS_CASE(384, 4) SQ_ROWS_CASE(704, 2) SQ_ROWS_CASE(512, 3) SQ_ROWS_CASE(1024, 2)
#undef SQ_ROWS_CASE
    return hipErrorInvalidValue;
}

hipError_t sq_launch_quantize_act(const void* x, int bf16, const float* s, int64_t m, int64_t k, int8_t* xq,
                                  float* x_scale, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    return bf16 ? launch_rows<true, true>(x, s, m, k, xq, x_scale, st)
                : launch_rows<false, true>(x, s, m, k, xq, x_scale, st);
}

hipError_t sq_launch_quantize_weight(const void* w, int bf16, const float* s, int64_t n, int64_t k, int8_t* wq,
                                     float* w_scale, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    return bf16 ? launch_rows<true, false>(w, s, n, k, wq, w_scale, st)
                : launch_rows<false, false>(w, s, n, k, wq, w_scale, st);
}

// the same codes in 16 x 64 tiles (the buffers hold the padded size)
hipError_t sq_launch_quantize_act_tiled(const void* x, int bf16, const float* s, int64_t m, int64_t k, int8_t* xq,
                                        float* x_scale, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    return bf16 ? launch_rows<true, true, true>(x, s, m, k, xq, x_scale, st)
                : launch_rows<false, true, true>(x, s, m, k, xq, x_scale, st);
}

hipError_t sq_launch_quantize_weight_tiled(const void* w, int bf16, const float* s, int64_t n, int64_t k, int8_t* wq,
                                           float* w_scale, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    return bf16 ? launch_rows<true, false, true>(w, s, n, k, wq, w_scale, st)
                : launch_rows<false, false, true>(w, s, n, k, wq, w_scale, st);
}

// ---------------------------------------------------------------------------
// Per-tensor variant (page "quantized_linear.py", quantize_tensor, 8 bits):
//   scale = max_i |x_i| / 127, replaced by 1 when below 1e-8
//   q_i   = clamp(round_half_even(x_i / scale), -128, 127)
// Three launches and no scratch: the block maxima of |x| (bit patterns) go
// to the first bytes of the code buffer, one block folds them into the
// scale, then every element's code (the same exact quotient and rounding as
// the row quantiser above; the scale is >= 1e-8 or exactly 1).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void tensor_max_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                         unsigned* __restrict__ partial) {
    constexpr int U = 4;
    constexpr uint32_t kMask = BF16 ? 0x7fff7fffu : 0x7fffffffu;
    __shared__ float red[4];
    u32x4 m = {0, 0, 0, 0};
    auto fold = [&](u32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = v[i] & kMask;
            if constexpr (BF16) m[i] = max_u16x2(m[i], a);
            else m[i] = max(m[i], a);
        }
    };
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + stride * (U - 1) < nvec; i += stride * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = x[i + stride * u];
#pragma unroll
        for (int u = 0; u < U; ++u) fold(v[u]);
    }
    for (; i < nvec; i += stride) fold(x[i]);
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (BF16) mx = fmaxf(mx, fmaxf(bf16_lo(m[j]), bf16_hi(m[j])));
        else mx = fmaxf(mx, __uint_as_float(m[j]));
    }
    mx = wave_max(mx);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.x] = __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

__global__ __launch_bounds__(256) void tensor_scale_kernel(const unsigned* __restrict__ partial, int blocks,
                                                           float* __restrict__ scale) {
    __shared__ float red[4];
    unsigned m = 0;
    // at most 4 rounds (1024 block maxima), their loads issued together
#pragma unroll 4
    for (int i = threadIdx.x; i < blocks; i += 256) m = max(m, partial[i]);
    float mx = wave_max(__uint_as_float(m));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        float sc = mx / kQmax;
        if (sc < kFloor) sc = 1.0f;  // the page's replacement (not a floor)
        *scale = sc;
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void tensor_codes_kernel(const u32x4* __restrict__ x, int64_t groups,
                                                           const float* __restrict__ scale, int8_t* __restrict__ q) {
    constexpr int kV = BF16 ? 1 : 2;  // 16-byte loads per 8 elements
    const float sc = *scale;
    const float rs = 1.0f / sc;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += (int64_t)gridDim.x * 256) {
        float v[8];
        if constexpr (BF16) {
            const u32x4 a = x[g];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_lo(a[i]);
                v[2 * i + 1] = bf16_hi(a[i]);
            }
        } else {
            const u32x4 a = x[g * kV], b = x[g * kV + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = __uint_as_float(a[i]);
                v[4 + i] = __uint_as_float(b[i]);
            }
        }
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = __float_as_uint(div_rn(v[i], sc, rs) + kMagic);
        *(u32x2*)(q + g * 8) = u32x2{pack_low_bytes(c[0], c[1], c[2], c[3]), pack_low_bytes(c[4], c[5], c[6], c[7])};
    }
}

// The codes into 16 x 64 tiles, the padding columns of every row written as
// zero codes: the row-major walk of the flat kernel above over rows x K64 / 8
// groups of 8 elements (reads contiguous; each thread's 8 bytes go to their
// tile). Staging 16-row slabs through LDS to store whole tiles, or walking
// in the tiles' order, measured slower.
template <bool BF16>
__global__ __launch_bounds__(256) void tensor_codes_tiled_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                                 int64_t k, const float* __restrict__ scale,
                                                                 int8_t* __restrict__ q) {
    constexpr int kV = BF16 ? 1 : 2;  // 16-byte loads per 8 elements
    const float sc = *scale;
    const float rs = 1.0f / sc;
    const int64_t k8 = k >> 3, k64 = (k + 63) & ~(int64_t)63, p8 = k64 >> 3;
    const int64_t groups = rows * p8;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += (int64_t)gridDim.x * 256) {
        const int64_t row = g / p8, j8 = g - row * p8;
        u32x2 codes = {0u, 0u};
        if (j8 < k8) {
            const int64_t src = row * k8 + j8;
            float v[8];
            if constexpr (BF16) {
                const u32x4 a = x[src];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_lo(a[i]);
                    v[2 * i + 1] = bf16_hi(a[i]);
                }
            } else {
                const u32x4 a = x[src * kV], b = x[src * kV + 1];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = __uint_as_float(a[i]);
                    v[4 + i] = __uint_as_float(b[i]);
                }
            }
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = __float_as_uint(div_rn(v[i], sc, rs) + kMagic);
            codes = u32x2{pack_low_bytes(c[0], c[1], c[2], c[3]), pack_low_bytes(c[4], c[5], c[6], c[7])};
        }
        *(u32x2*)(q + ((row >> 4) * (k64 >> 6) + (j8 >> 3)) * 1024 + (row & 15) * 64 + (j8 & 7) * 8) = codes;
    }
}

int64_t sq_tensor_max_blocks(int64_t count) {
    int64_t b = count / 8192;  // about 8 KiB of input per block
    if (b < 1) b = 1;
    if (b > 1024) b = 1024;
    return b;  // the partials (4 bytes each) fit in the count-byte code buffer
}

// rows > 0: the codes into 16 x 64 tiles of a [rows][count / rows] matrix
static hipError_t quantize_tensor(const void* x, int bf16, int64_t count, int64_t rows, int8_t* q, float* scale,
                                  hipStream_t st) {
    const int64_t nvec = bf16 ? count / 8 : count / 4;
    const int64_t blocks = sq_tensor_max_blocks(count);
    unsigned* partial = (unsigned*)q;
    if (bf16)
        hipLaunchKernelGGL(tensor_max_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)x, nvec,
                           partial);
    else
        hipLaunchKernelGGL(tensor_max_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)x, nvec,
                           partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, st, (const unsigned*)partial, (int)blocks, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (rows > 0) {
        const int64_t k = count / rows;
        const int64_t groups = rows * ((k + 63) / 64 * 8);
        int64_t cb = (groups + 255) / 256;
        if (cb > 4096) cb = 4096;
        const dim3 grid((unsigned)cb);
        if (bf16)
            hipLaunchKernelGGL(tensor_codes_tiled_kernel<true>, grid, dim3(256), 0, st, (const u32x4*)x, rows, k,
                               (const float*)scale, q);
        else
            hipLaunchKernelGGL(tensor_codes_tiled_kernel<false>, grid, dim3(256), 0, st, (const u32x4*)x, rows, k,
                               (const float*)scale, q);
        return hipGetLastError();
    }
    const int64_t groups = count / 8;
    int64_t cb = (groups + 255) / 256;
    if (cb > 4096) cb = 4096;
    if (bf16)
        hipLaunchKernelGGL(tensor_codes_kernel<true>, dim3((unsigned)cb), dim3(256), 0, st, (const u32x4*)x, groups,
                           (const float*)scale, q);
    else
        hipLaunchKernelGGL(tensor_codes_kernel<false>, dim3((unsigned)cb), dim3(256), 0, st, (const u32x4*)x, groups,
                           (const float*)scale, q);
    return hipGetLastError();
}

hipError_t sq_launch_quantize_tensor(const void* x, int bf16, int64_t count, int8_t* q, float* scale,
                                     hipStream_t st) {
    return quantize_tensor(x, bf16, count, 0, q, scale, st);
}

hipError_t sq_launch_quantize_tensor_tiled(const void* x, int bf16, int64_t rows, int64_t k, int8_t* q,
                                           float* scale, hipStream_t st) {
    return quantize_tensor(x, bf16, rows * k, rows, q, scale, st);
}
