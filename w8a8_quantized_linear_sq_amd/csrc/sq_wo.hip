// sq_wo.hip -- weight-only int8 linear: bf16 activations times int8 weights
// with one scale per output channel, for few tokens (the decode shape).
//
// Follows the torchao page "quantization/subclass.py",
// Int8WeightOnlyQuantizedLinearWeight._quantized_op: the int8 weights are
// converted to the activations' type (bf16, exactly), multiplied with the
// activations, scaled per output channel, then the bias is added:
//   y[t][o] = f32(sum_j x[t][j] * wq[o][j]) * sw[o] (+ bias[o])   -> out type
// Every bf16 x int8 product is exact in fp32; the sum is accumulated in fp32
// by the matrix units.
//
// Design (gfx950): the weight-streaming structure of the W8A8 product for
// few tokens (sq_skinny.hip), with bf16 token fragments:
//   * one workgroup of 2 wavefronts per 32 weight rows; K is split over the
//     wavefronts in 256-element segments dealt alternately, each wavefront
//     staging its segments of the weight rows (256 bytes per row) and of
//     the token rows (512 bytes per row) through its own LDS ring with
//     direct global -> LDS loads (one load covers 4 weight rows x 256 bytes
//     or 2 token rows x 512 bytes, contiguous per row);
//   * 16-byte chunk c of row r sits at slot c ^ (r & 15) within its LDS row,
//     so the 16-row fragment reads spread over every bank;
//   * v_mfma_f32_16x16x32_bf16 with the tokens as the 16-row operand; the
//     weight fragment (8 int8 per lane) is widened to bf16 in registers
//     (every int8 is a bf16 exactly);
//   * the K tail past the last whole segment goes through registers in
//     32-element blocks, a last partial block zero-filled;
//   * the partial sums of the two wavefronts meet in LDS in a fixed order,
//     and wavefront 0 applies the scale and the bias.
#include "sq_device.h"

using namespace sq;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kSegK = 256;                  // K elements per staged segment
constexpr int kWTile = 16 * kSegK;          // 16 weight rows x 256 bytes
constexpr int kXTile = 16 * kSegK * 2;      // 16 token rows x 512 bytes
constexpr int kLgkm0 = 0xc07f;              // s_waitcnt lgkmcnt(0) only

constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int slot(int r, int c) { return c ^ (r & 15); }

// 8 int8 (two dwords) -> 8 bf16, exactly
__device__ __forceinline__ bf16x8 widen(u32x2 w) {
    bf16x8 out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t word = i < 4 ? w[0] : w[1];
        const int v = (int)(int8_t)(word >> (8 * (i & 3)));
        out[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint((float)v) >> 16));
    }
    return out;
}

// v_mfma_f32_16x16x32_bf16 operands: lane l holds 8 k-consecutive bf16 of
// row (l % 16) at k offset 8 * (l / 16); result lane l, register r -> row
// 4 * (l / 16) + r, column l % 16.
template <int TM, int NG, int D, int W, int OUT>
__global__ __launch_bounds__(64 * W) void wo_kernel(const uint16_t* __restrict__ X, const int8_t* __restrict__ Bw,
                                                    int m, int n, int k, const float* __restrict__ sb,
                                                    const void* __restrict__ bias, int bias_kind,
                                                    void* __restrict__ Y) {
    constexpr int STAGE = NG * kWTile + TM * kXTile;
    constexpr int LOADS = NG * 4 + TM * 8;  // DMA loads per stage
    static_assert(W * D * STAGE >= (W - 1) * TM * NG * 64 * 16, "reduction must fit the staging area");
    __shared__ __attribute__((aligned(1024))) int8_t smem[W * D * STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16 * NG;
    const int r16 = lane & 15, grp = lane >> 4;
    int8_t* my = smem + wave * D * STAGE;

    // ---- DMA sources. Weight load q (0..3) of group g: rows 4q .. 4q+3,
    // lane i -> row 4q + i/16, slot i%16; token load q (0..7) of group t:
    // rows 2q, 2q+1, lane i -> row 2q + i/32, slot i%32.
    const int8_t* wsrc[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 4 * q + grp;
            wsrc[g][q] = Bw + (int64_t)min(n0 + g * 16 + r, n - 1) * k + slot(r, r16) * 16;
        }
    const int8_t* xsrc[TM][8];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 2 * q + (lane >> 5);
            xsrc[t][q] = (const int8_t*)(X + (int64_t)min(t * 16 + r, m - 1) * k) + slot(r, lane & 31) * 16;
        }
    auto issue = [&](int seg, int buf) {
        int8_t* st = my + buf * STAGE;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(wsrc[g][q] + seg * kSegK),
                                                 (lds_ptr_t)(st + g * kWTile + q * 1024), 16, 0, 0);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(xsrc[t][q] + seg * kSegK * 2),
                                                 (lds_ptr_t)(st + NG * kWTile + t * kXTile + q * 1024), 16, 0, 0);
    };

    f32x4 acc[TM][NG];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[t][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int KS = k / kSegK;
    const int nseg = KS > wave ? (KS - wave + W - 1) / W : 0;
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nseg) issue(wave + W * d, d);
    for (int i = 0; i < nseg; ++i) {
        const int buf = i % D;
        if (D >= 2 && i + 1 < nseg) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        const int8_t* st = my + buf * STAGE;
#pragma unroll
        for (int b = 0; b < kSegK / 32; ++b) {
            bf16x8 wf[NG], xf[TM];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int c = 2 * b + (grp >> 1);
                wf[g] = widen(*(const u32x2*)(st + g * kWTile + r16 * kSegK + slot(r16, c) * 16 + (grp & 1) * 8));
            }
#pragma unroll
            for (int t = 0; t < TM; ++t)
                xf[t] = *(const bf16x8*)(st + NG * kWTile + t * kXTile + r16 * 512 + slot(r16, 4 * b + grp) * 16);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[t], wf[g], acc[t][g], 0, 0, 0);
        }
        if (i + D < nseg) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            issue(wave + W * (i + D), buf);
        }
    }

    // ---- K past the segments: 32-element blocks through registers, then a
    // ---- last partial block (k is a multiple of 16), zero-filled
    const bf16x8 zero8 = {};
    for (int kb = KS * (kSegK / 32) + wave; kb * 32 < k; kb += W) {
        const int k0 = kb * 32 + grp * 8;
        const bool in = k0 < k;  // whole block, or the 16-element tail
        bf16x8 wf[NG], xf[TM];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int8_t* p = Bw + (int64_t)min(n0 + g * 16 + r16, n - 1) * k + k0;
            wf[g] = in ? widen(*(const u32x2*)p) : zero8;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint16_t* p = X + (int64_t)min(t * 16 + r16, m - 1) * k + k0;
            xf[t] = in ? *(const bf16x8*)p : zero8;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g)
                acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[t], wf[g], acc[t][g], 0, 0, 0);
    }

    // ---- the wavefronts' partial sums meet in LDS (the staging area, free
    // ---- once every wavefront is past its loop), in a fixed order
    __syncthreads();
    f32x4 (*red)[TM][NG][64] = (f32x4 (*)[TM][NG][64])smem;
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) red[wave - 1][t][g][lane] = acc[t][g];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[t][g] += red[w][t][g][lane];

#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int o = n0 + g * 16 + r16;
        if (o >= n) continue;
        const float swo = sb[o];
        float bo = 0.0f;
        if (bias_kind == 1) bo = ((const float*)bias)[o];
        else if (bias_kind == 2) bo = __uint_as_float((uint32_t)((const uint16_t*)bias)[o] << 16);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = t * 16 + grp * 4 + r;
                if (row >= m) continue;
                float y = acc[t][g][r] * swo;
                if (bias_kind) y = y + bo;
                const int64_t off = (int64_t)row * n + o;
                if constexpr (OUT == 0) ((float*)Y)[off] = y;
                else ((__bf16*)Y)[off] = (__bf16)y;
            }
        }
    }
}

template <int TM, int D>
hipError_t launch_wo(const uint16_t* x, int m, const int8_t* wq, const float* sw, int n, int k, const void* bias,
                     int bias_kind, void* y, int out_kind, hipStream_t st) {
    constexpr int NG = 2, W = 2;
    const dim3 grid((n + 16 * NG - 1) / (16 * NG)), block(64 * W);
    if (out_kind == 0)
        hipLaunchKernelGGL((wo_kernel<TM, NG, D, W, 0>), grid, block, 0, st, x, wq, m, n, k, sw, bias, bias_kind, y);
    else
        hipLaunchKernelGGL((wo_kernel<TM, NG, D, W, 1>), grid, block, 0, st, x, wq, m, n, k, sw, bias, bias_kind, y);
    return hipGetLastError();
}

}  // namespace

// Tokens are processed in chunks of up to 64 (each chunk streams the
// weights once): the kernel is built for the decode shape.
hipError_t sq_launch_wo_linear(const void* x, int64_t m, int64_t k, const int8_t* wq, const float* sw, int64_t n,
                               const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st) {
    const int ob = out_kind == 0 ? 4 : 2;
    for (int64_t r0 = 0; r0 < m; r0 += 64) {
        const int mc = (int)((m - r0 < 64) ? m - r0 : 64);
        const uint16_t* xc = (const uint16_t*)x + r0 * k;
        void* yc = (int8_t*)y + r0 * n * ob;
        hipError_t e;
        switch ((mc + 15) / 16) {
            case 1: e = launch_wo<1, 2>(xc, mc, wq, sw, (int)n, (int)k, bias, bias_kind, yc, out_kind, st); break;
            case 2: e = launch_wo<2, 1>(xc, mc, wq, sw, (int)n, (int)k, bias, bias_kind, yc, out_kind, st); break;
            case 3: e = launch_wo<3, 1>(xc, mc, wq, sw, (int)n, (int)k, bias, bias_kind, yc, out_kind, st); break;
            default: e = launch_wo<4, 1>(xc, mc, wq, sw, (int)n, (int)k, bias, bias_kind, yc, out_kind, st); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
