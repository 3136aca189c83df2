// sq_skinny.hip -- the INT8 x INT8 -> INT32 product and its dequantisation
// for few tokens (m <= 64), the decode shape: every weight byte is used by
// at most 64 tokens, so the product is bound by streaming w_q from HBM, not
// by the matrix units.
//
// Same arithmetic as the tiled kernel (page "w8a8_smoothquant.py",
// SmoothQuantW8A8.forward, integer route):
//   acc[t][o] = sum_j xq[t][j] * wq[o][j]                  (exact int32)
//   y[t][o]   = f32(acc) * sx[t] * sw[o] (+ bias[o])       (fp32 -> out type)
//
// Design (gfx950):
//   * one workgroup of 4 wavefronts per 32 or 64 weight rows; the grid
//     covers n (344 workgroups for 11008 rows at 32), so every CU streams;
//   * the wavefronts split K into 64-byte blocks dealt round-robin (wave w
//     takes blocks w, w + 4, ...), so together they read each weight row in
//     256-byte runs; each lane loads its 16-byte operand pieces straight
//     into registers (no LDS staging: a weight byte is used by one
//     wavefront only), 8 blocks per round in flight;
//   * v_mfma_i32_16x16x64_i8 with the tokens as the 16-row operand: each
//     of the TM token fragments meets each of the NG weight fragments of a
//     block; rows past m or n are clamped for loading and never stored;
//   * the four int32 partial sums meet in LDS (integer addition: exact and
//     independent of order) and wavefront 0 applies the scales and bias.
#include "sq_device.h"

using namespace sq;

namespace {

constexpr int kWaves = 4;
constexpr int kBlk = 64;    // bytes of K per MFMA

// v_mfma_i32_16x16x64_i8 operands: lane l holds 16 k-consecutive bytes of
// row (l % 16) at k offset 16 * (l / 16); result lane l, register r ->
// row 4 * (l / 16) + r, column l % 16.
template <int TM, int NG, int OUT>
__global__ __launch_bounds__(64 * kWaves) void skinny_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int m, int n, int k,
    const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
    int bias_kind, void* __restrict__ Y) {
    constexpr int U = TM + NG <= 3 ? 8 : 4;  // blocks per round in flight
    constexpr int kRows = 16 * NG;            // weight rows per workgroup
    __shared__ i32x4 red[kWaves - 1][TM][NG][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * kRows;
    const int r16 = lane & 15, grp = lane >> 4;

    const int8_t* brow[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) brow[g] = B + (int64_t)min(n0 + g * 16 + r16, n - 1) * k + grp * 16;
    const int8_t* arow[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) arow[t] = A + (int64_t)min(t * 16 + r16, m - 1) * k + grp * 16;

    i32x4 acc[TM][NG];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[t][g] = i32x4{0, 0, 0, 0};

    const int KB = k / kBlk;  // whole blocks
    // rounds of U blocks per wavefront, double-buffered in registers: the
    // loads of round r + 1 are issued before the MFMAs of round r
    constexpr int STRIDE = kWaves * U;
    i32x4 b0[U][NG], a0[U][TM], b1[U][NG], a1[U][TM];
    auto load_round = [&](int kb0, i32x4 (&b)[U][NG], i32x4 (&a)[U][TM]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int off = (kb0 + kWaves * u) * kBlk;
#pragma unroll
            for (int g = 0; g < NG; ++g) b[u][g] = *(const i32x4*)(brow[g] + off);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                a[u][t] = *(const i32x4*)(arow[t] + off);
            }
        }
    };
    auto mma_round = [&](const i32x4 (&b)[U][NG], const i32x4 (&a)[U][TM]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    acc[t][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][t], b[u][g], acc[t][g], 0, 0, 0);
    };
    constexpr int kLoads = U * (NG + TM);
    int kb = wave;
    const int rounds = KB > wave ? (KB - wave) / STRIDE : 0;  // whole rounds
    if (rounds > 0) {
        load_round(kb, b0, a0);
        int r = 0;
        for (; r + 2 <= rounds - 1; r += 2) {
            load_round(kb + STRIDE, b1, a1);
            mma_round(b0, a0);
            __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, U * TM * NG, 0);
            load_round(kb + 2 * STRIDE, b0, a0);
            mma_round(b1, a1);
            __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, U * TM * NG, 0);
            kb += 2 * STRIDE;
        }
        if (r + 1 <= rounds - 1) {
            load_round(kb + STRIDE, b1, a1);
            mma_round(b0, a0);
            __builtin_amdgcn_sched_group_barrier(0x020, kLoads, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, U * TM * NG, 0);
            mma_round(b1, a1);
            kb += 2 * STRIDE;
        } else {
            mma_round(b0, a0);
            kb += STRIDE;
        }
    }
    for (; kb < KB; kb += kWaves) {
        const int off = kb * kBlk;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const i32x4 a = *(const i32x4*)(arow[t] + off);
#pragma unroll
            for (int g = 0; g < NG; ++g)
                acc[t][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, *(const i32x4*)(brow[g] + off), acc[t][g], 0, 0, 0);
        }
    }
    if ((k % kBlk) && wave == KB % kWaves) {
        // a last partial block (k is a multiple of 16): pieces past k are 0
        const int off = KB * kBlk;
        const bool in = off + grp * 16 < k;
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const i32x4 a = in ? *(const i32x4*)(arow[t] + off) : zero;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const i32x4 b = in ? *(const i32x4*)(brow[g] + off) : zero;
                acc[t][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t][g], 0, 0, 0);
            }
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) red[wave - 1][t][g][lane] = acc[t][g];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[t][g] += red[w][t][g][lane];

#pragma unroll
    for (int g = 0; g < NG; ++g) {
    const int o = n0 + g * 16 + r16;
    if (o >= n) continue;
    float swo = 0.0f, bo = 0.0f;
    if constexpr (OUT != 2) {
        swo = sb[o];
        if (bias_kind == 1) bo = ((const float*)bias)[o];
        else if (bias_kind == 2) bo = __uint_as_float((uint32_t)((const uint16_t*)bias)[o] << 16);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = t * 16 + grp * 4 + r;
            if (row >= m) continue;
            const int64_t off = (int64_t)row * n + o;
            if constexpr (OUT == 2) {
                ((int*)Y)[off] = acc[t][g][r];
            } else {
                float y = (float)acc[t][g][r] * sa[row] * swo;
                if (bias_kind) y = y + bo;
                if constexpr (OUT == 0) ((float*)Y)[off] = y;
                else ((__bf16*)Y)[off] = (__bf16)y;
            }
        }
    }
    }
}

template <int TM, int NG>
hipError_t launch_tm(const int8_t* xq, const float* sx, int m, const int8_t* wq, const float* sw, int n, int k,
                     const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st) {
    const dim3 grid((n + 16 * NG - 1) / (16 * NG)), block(64 * kWaves);
    switch (out_kind) {
        case 0:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, 0>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y);
            break;
        case 1:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, 1>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y);
            break;
        default:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, 2>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y);
            break;
    }
    return hipGetLastError();
}

}  // namespace

// Weight rows per workgroup grow with the token groups: every workgroup
// reads all m token rows once, so more weight rows per workgroup cut that
// traffic (measured best: 32 rows up to 32 tokens, 64 beyond).
hipError_t sq_launch_gemm_skinny(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                 int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                 hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch ((mi + 15) / 16) {
        case 1: return launch_tm<1, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        case 2: return launch_tm<2, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        case 3: return launch_tm<3, 4>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        case 4: return launch_tm<4, 4>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        default: return hipErrorInvalidValue;
    }
}
