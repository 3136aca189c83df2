// sq_quant.hip -- the HBM-bound steps of the SmoothQuant W8A8 linear
// (page "w8a8_smoothquant.py", BiGRU_T_version):
//   * column max-abs reduction (SmoothQuantW8A8.calibrate's running max, and
//     calibrate_smoothquant's max over output rows of |W|);
//   * the smoothing factor s (calibrate_smoothquant);
//   * smoothing + per-output-channel int8 of the weights
//     (freeze_quantization -> quantize_per_channel_symmetric);
//   * smoothing + per-token int8 of the activations
//     (forward -> X / s -> quantize_per_token_symmetric).
#include "sq_device.h"

using namespace sq;

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
// Column max of |x| over rows, folded into out[] with an integer atomic max.
// |x| is non-negative, so the order of the binary32 bit patterns as unsigned
// integers is the order of the values: the fold is exact and independent of
// the order in which blocks run.
// Each thread owns one 16-byte column chunk (8 bf16 or 4 fp32 columns) and
// walks `rows_per_block` rows; a block is 256 chunks wide.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void colmax_kernel(const u32x4* __restrict__ x, int64_t rows,
                                                     int64_t kvec, int rows_per_block,
                                                     unsigned* __restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= kvec) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    int64_t r1 = r0 + rows_per_block;
    if (r1 > rows) r1 = rows;
    constexpr uint32_t kMask = BF16 ? 0x7fff7fffu : 0x7fffffffu;
    u32x4 m0 = {0, 0, 0, 0}, m1 = {0, 0, 0, 0};
    int64_t r = r0;
    // four rows in flight per thread
    for (; r + 4 <= r1; r += 4) {
        u32x4 v0 = x[(r + 0) * kvec + c];
        u32x4 v1 = x[(r + 1) * kvec + c];
        u32x4 v2 = x[(r + 2) * kvec + c];
        u32x4 v3 = x[(r + 3) * kvec + c];
        if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t a0 = v0[i] & kMask, a1 = v1[i] & kMask, a2 = v2[i] & kMask, a3 = v3[i] & kMask;
                uint32_t lo = max(max(a0 & 0xffffu, a1 & 0xffffu), max(a2 & 0xffffu, a3 & 0xffffu));
                uint32_t hi = max(max(a0 >> 16, a1 >> 16), max(a2 >> 16, a3 >> 16));
                m0[i] = max(m0[i], lo);
                m1[i] = max(m1[i], hi);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m0[i] = max(m0[i], max(max(v0[i] & kMask, v1[i] & kMask), max(v2[i] & kMask, v3[i] & kMask)));
        }
    }
    for (; r < r1; ++r) {
        u32x4 v0 = x[r * kvec + c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t a0 = v0[i] & kMask;
            if constexpr (BF16) {
                m0[i] = max(m0[i], a0 & 0xffffu);
                m1[i] = max(m1[i], a0 >> 16);
            } else {
                m0[i] = max(m0[i], a0);
            }
        }
    }
    if constexpr (BF16) {
        unsigned* o = out + c * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            atomicMax(o + 2 * i, m0[i] << 16);
            atomicMax(o + 2 * i + 1, m1[i] << 16);
        }
    } else {
        unsigned* o = out + c * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) atomicMax(o + i, m0[i]);
    }
}

hipError_t sq_launch_colmax(const void* x, int bf16, int64_t rows, int64_t k, float* out_max,
                            hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int64_t kvec = bf16 ? k / 8 : k / 4;
    const int64_t gx = (kvec + 255) / 256;
    // about 1024 blocks in all, at least 4 rows each
    int64_t gy = 1024 / gx;
    if (gy < 1) gy = 1;
    int64_t rpb = (rows + gy - 1) / gy;
    if (rpb < 4) rpb = 4;
    gy = (rows + rpb - 1) / rpb;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (bf16)
        hipLaunchKernelGGL(colmax_kernel<true>, grid, dim3(256), 0, st, (const u32x4*)x, rows, kvec,
                           (int)rpb, (unsigned*)out_max);
    else
        hipLaunchKernelGGL(colmax_kernel<false>, grid, dim3(256), 0, st, (const u32x4*)x, rows, kvec,
                           (int)rpb, (unsigned*)out_max);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Smoothing factor, per input channel j (calibrate_smoothquant):
//   s_j = max(f32(P(max(mx_j, floor), a_x)) / f32(P(max(mw_j, floor), a_w)), floor)
// P(x, a) = x^a through binary64: exact forms built from correctly rounded
// sqrt for a in {0, 1/4, 1/2, 3/4, 1}, pow otherwise. `io` holds the raw
// column max of |W| on entry and s on exit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double pow64(double x, double a) {
    if (a == 0.0) return 1.0;
    if (a == 1.0) return x;
    if (a == 0.5) return __builtin_sqrt(x);
    if (a == 0.25) return __builtin_sqrt(__builtin_sqrt(x));
    if (a == 0.75) return __builtin_sqrt(x) * __builtin_sqrt(__builtin_sqrt(x));
    return pow(x, a);
}

__global__ __launch_bounds__(256) void smooth_factor_kernel(const float* __restrict__ x_max,
                                                            float* __restrict__ io, double a_x,
                                                            double a_w, int64_t k) {
    int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= k) return;
    float mx = fmaxf(x_max[j], kFloor);
    float mw = fmaxf(io[j], kFloor);
    float num = (float)pow64((double)mx, a_x);
    float den = (float)pow64((double)mw, a_w);
    io[j] = fmaxf(num / den, kFloor);
}

hipError_t sq_launch_smooth_factor(const float* x_max, float* io, double a_x, double a_w,
                                   int64_t k, hipStream_t st) {
    unsigned blocks = (unsigned)((k + 255) / 256);
    hipLaunchKernelGGL(smooth_factor_kernel, dim3(blocks), dim3(256), 0, st, x_max, io, a_x, a_w, k);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loads of 8 consecutive elements as fp32 (bf16: one 16-byte load; fp32: two).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t elem, float (&v)[8]) {
    if constexpr (BF16) {
        u32x4 u = *(const u32x4*)((const uint16_t*)base + elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(u[i]);
            v[2 * i + 1] = bf16_hi(u[i]);
        }
    } else {
        const float* f = (const float*)base + elem;
        u32x4 a = *(const u32x4*)f;
        u32x4 b = *(const u32x4*)(f + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    }
}

__device__ __forceinline__ void load8_f32(const float* __restrict__ p, float (&v)[8]) {
    u32x4 a = *(const u32x4*)p;
    u32x4 b = *(const u32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(a[i]);
        v[4 + i] = __uint_as_float(b[i]);
    }
}

// ---------------------------------------------------------------------------
// Weights: one wavefront per output row o.
//   pass 1: m = max_j |f32(w[o][j] * s_j)|
//   scale  = max(m, floor) / 127
//   pass 2: codes of f32(w[o][j] * s_j) (the row is re-read from L2)
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const void* __restrict__ w,
                                                              const float* __restrict__ s, int64_t n,
                                                              int64_t k, int8_t* __restrict__ wq,
                                                              float* __restrict__ w_scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const int64_t k8 = k >> 3;
    const int64_t base = row * k;
    float m = 0.0f;
    for (int64_t j8 = lane; j8 < k8; j8 += 64) {
        float v[8], sv[8];
        load8<BF16>(w, base + j8 * 8, v);
        load8_f32(s + j8 * 8, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i] * sv[i]));
    }
    m = wave_max(m);
    const float scale = fmaxf(m, kFloor) / kQmax;
    const float rs = 1.0f / scale;
    for (int64_t j8 = lane; j8 < k8; j8 += 64) {
        float v[8], sv[8];
        load8<BF16>(w, base + j8 * 8, v);
        load8_f32(s + j8 * 8, sv);
        float c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = code_of(v[i] * sv[i], scale, rs);
        u32x2 packed = {pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])};
        *(u32x2*)(wq + base + j8 * 8) = packed;
    }
    if (lane == 0) w_scale[row] = scale;
}

hipError_t sq_launch_quantize_weight(const void* w, int bf16, const float* s, int64_t n, int64_t k,
                                     int8_t* wq, float* w_scale, hipStream_t st) {
    unsigned blocks = (unsigned)((n + 3) / 4);
    if (bf16)
        hipLaunchKernelGGL(quantize_weight_kernel<true>, dim3(blocks), dim3(256), 0, st, w, s, n, k, wq,
                           w_scale);
    else
        hipLaunchKernelGGL(quantize_weight_kernel<false>, dim3(blocks), dim3(256), 0, st, w, s, n, k, wq,
                           w_scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Activations: a team of W wavefronts per token row; each lane holds C steps
// of 8 consecutive channels of x~ = f32(x / s) in registers, so the row is
// read once and x / s is formed once.
//   m = max_j |x~_j| (lane -> wave -> team), scale = max(m, floor) / 127,
//   codes of x~_j.
// Teams walk rows with a grid stride; the block's loop count is uniform so
// the team barrier is reached by every thread.
// ---------------------------------------------------------------------------
template <bool BF16, int W, int C>
__global__ __launch_bounds__(256) void quantize_act_kernel(const void* __restrict__ x,
                                                           const float* __restrict__ s, int64_t m,
                                                           int64_t k, int8_t* __restrict__ xq,
                                                           float* __restrict__ x_scale) {
    constexpr int kTeams = 4 / W;
    __shared__ float red[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = wave / W;
    const int wit = wave % W;  // wave index inside its team
    const int64_t k8 = k >> 3;
    for (int64_t rbase = (int64_t)blockIdx.x * kTeams; rbase < m; rbase += (int64_t)gridDim.x * kTeams) {
        const int64_t row = rbase + team;
        const bool active = row < m;
        // issue every load of the row first, then compute
        constexpr int kV = BF16 ? 1 : 2;
        u32x4 raw[C][kV];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j8 = (int64_t)(c * W + wit) * 64 + lane;
            if (active && j8 < k8) {
                const u32x4* p = BF16 ? (const u32x4*)((const uint16_t*)x + row * k + j8 * 8)
                                      : (const u32x4*)((const float*)x + row * k + j8 * 8);
#pragma unroll
                for (int v = 0; v < kV; ++v) raw[c][v] = p[v];
            } else {
#pragma unroll
                for (int v = 0; v < kV; ++v) raw[c][v] = u32x4{0, 0, 0, 0};
            }
        }
        float xs[C][8];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t j8 = (int64_t)(c * W + wit) * 64 + lane;
            float v[8], sv[8];
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_lo(raw[c][0][i]);
                    v[2 * i + 1] = bf16_hi(raw[c][0][i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = __uint_as_float(raw[c][0][i]);
                    v[4 + i] = __uint_as_float(raw[c][1][i]);
                }
            }
            if (j8 < k8) {
                load8_f32(s + j8 * 8, sv);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) sv[i] = 1.0f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xs[c][i] = v[i] / sv[i];
                mx = fmaxf(mx, fabsf(xs[c][i]));
            }
        }
        mx = wave_max(mx);
        if constexpr (W > 1) {
            if (lane == 0) red[wave] = mx;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < W; ++i) mx = fmaxf(mx, red[team * W + i]);
            __syncthreads();
        }
        const float scale = fmaxf(mx, kFloor) / kQmax;
        const float rs = 1.0f / scale;
        if (active) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int64_t j8 = (int64_t)(c * W + wit) * 64 + lane;
                if (j8 < k8) {
                    float q[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = code_of(xs[c][i], scale, rs);
                    u32x2 packed = {pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7])};
                    *(u32x2*)(xq + row * k + j8 * 8) = packed;
                }
            }
            if (wit == 0 && lane == 0) x_scale[row] = scale;
        }
    }
}

template <bool BF16>
static hipError_t launch_act(const void* x, const float* s, int64_t m, int64_t k, int8_t* xq,
                             float* x_scale, hipStream_t st) {
    // team width W and steps per lane C such that 512 * W * C >= k
    int W, C;
    const int64_t steps = (k + 511) / 512;  // 8-channel steps per lane for one wave
    if (steps <= 8) {
        W = 1;
        C = (int)steps;
    } else if (steps <= 16) {
        W = 2;
        C = (int)((steps + 1) / 2);
    } else {
        W = 4;
        C = (int)((steps + 3) / 4);
    }
    // round C up to an instantiated value
    C = C <= 1 ? 1 : C <= 2 ? 2 : C <= 4 ? 4 : C <= 6 ? 6 : 8;
    const int teams = 4 / W;
    int64_t blocks = (m + teams - 1) / teams;
    if (blocks > 8192) blocks = 8192;
    dim3 grid((unsigned)blocks), block(256);
#define SQ_ACT_CASE(WW, CC)                                                                      \
    if (W == WW && C == CC) {                                                                    \
        hipLaunchKernelGGL((quantize_act_kernel<BF16, WW, CC>), grid, block, 0, st, x, s, m, k, xq, \
                           x_scale);                                                             \
        return hipGetLastError();                                                                \
    }
    SQ_ACT_CASE(1, 1) SQ_ACT_CASE(1, 2) SQ_ACT_CASE(1, 4) SQ_ACT_CASE(1, 6) SQ_ACT_CASE(1, 8)
    SQ_ACT_CASE(2, 6) SQ_ACT_CASE(2, 8) SQ_ACT_CASE(4, 6) SQ_ACT_CASE(4, 8)
#undef SQ_ACT_CASE
    return hipErrorInvalidValue;
}

hipError_t sq_launch_quantize_act(const void* x, int bf16, const float* s, int64_t m, int64_t k,
                                  int8_t* xq, float* x_scale, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    return bf16 ? launch_act<true>(x, s, m, k, xq, x_scale, st)
                : launch_act<false>(x, s, m, k, xq, x_scale, st);
}
