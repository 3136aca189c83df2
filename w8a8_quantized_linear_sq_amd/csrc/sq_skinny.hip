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
//   * one workgroup of 2 wavefronts per 32 (up to 32 tokens) or 64 weight
//     rows; the grid covers n (344 workgroups for 11008 rows), so every CU
//     streams;
//   * K is split over the 2 wavefronts in 256-byte segments dealt
//     alternately; each wavefront stages its segments, the workgroup's
//     weight rows and the token rows, through its own LDS ring (3 stages
//     for 16 tokens, fewer for more) with direct global -> LDS loads
//     (global_load_lds_dwordx4): one load covers 4 rows x 256 contiguous
//     bytes, so HBM sees whole lines and long runs. Reading the 16-row MFMA
//     fragments straight from memory (16 rows x 64 bytes per load) measured
//     about 30% slower, and token fragments loaded into registers forced
//     waits on every staged load (one counter), so both operands go
//     through LDS;
//   * inside a 256-byte LDS row, chunk c of row r sits at slot c ^ (r & 15),
//     so a fragment read (16 rows, the same chunk) touches every bank once;
//   * v_mfma_i32_16x16x64_i8 with the tokens as the 16-row operand: each
//     of the TM token fragments meets each of the NG weight fragments of a
//     block; rows past m or n are clamped for loading and never stored;
//   * K past the last whole segment goes through registers in 64-byte
//     blocks, a final partial block zero-filled;
//   * the two int32 partial sums meet in LDS (integer addition: exact and
//     independent of order) and wavefront 0 applies the scales and bias.
#include "sq_device.h"

using namespace sq;

namespace {

constexpr int kBlk = 64;    // bytes of K per MFMA

// v_mfma_i32_16x16x64_i8 operands: lane l holds 16 k-consecutive bytes of
// row (l % 16) at k offset 16 * (l / 16); result lane l, register r ->
// row 4 * (l / 16) + r, column l % 16.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kSeg = 256;             // bytes of K per staged segment (4 blocks)
constexpr int kTile = 16 * kSeg;      // one 16-row group x one segment in LDS

// s_waitcnt immediate (gfx9 encoding): at most n vector memory operations
// outstanding, no wait on the other counters
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0 = 0xc07f;  // lgkmcnt(0) only

// position of 16-byte chunk c of row r inside its 256-byte LDS row: the XOR
// spreads the 16 rows of a fragment read over all banks
__device__ __forceinline__ int seg_pos(int r, int c) { return c ^ (r & 15); }

template <int TM, int NG, int D, int kWaves, int OUT>
__global__ __launch_bounds__(64 * kWaves) void skinny_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int m, int n, int k,
    const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
    int bias_kind, void* __restrict__ Y, int scalar_scales) {
    constexpr int kRows = 16 * NG;            // weight rows per workgroup
    constexpr int TILES = NG + TM;            // weight groups, then token groups
    constexpr int STAGE = TILES * kTile;      // one wavefront's LDS stage
    constexpr int LOADS = TILES * 4;          // DMA loads per stage (4 rows x 256 B each)
    static_assert(kWaves * D * STAGE >= (kWaves - 1) * TM * NG * 64 * 16, "reduction must fit the staging area");
    __shared__ __attribute__((aligned(1024))) int8_t smem[kWaves * D * STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * kRows;
    const int r16 = lane & 15, grp = lane >> 4;
    int8_t* my = smem + wave * D * STAGE;

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

    // ---- whole 256-byte segments, staged through this wavefront's LDS ring.
    // DMA load q of row group g covers rows 4q .. 4q+3 of the group: lane i
    // writes LDS position i (row 4q + i/16, chunk slot i%16) and reads the
    // global chunk that slot holds, so each row is read as 256 contiguous
    // bytes. Wavefront w takes segments w, w + 4, ...
    const int KS = k / kSeg;
    const int8_t* dsrc[TILES][4];
#pragma unroll
    for (int g = 0; g < TILES; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 4 * q + grp;       // lane / 16
            const int c = seg_pos(r, r16);   // the chunk whose slot is lane % 16 (XOR is an involution)
            dsrc[g][q] = g < NG ? B + (int64_t)min(n0 + g * 16 + r, n - 1) * k + c * 16
                                : A + (int64_t)min((g - NG) * 16 + r, m - 1) * k + c * 16;
        }
    auto issue = [&](int seg, int buf) {
#pragma unroll
        for (int g = 0; g < TILES; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(dsrc[g][q] + seg * kSeg),
                                                 (lds_ptr_t)(my + buf * STAGE + g * kTile + q * 1024), 16, 0, 0);
    };
    // fragment of k-block b (64 bytes) for this lane: row r16, chunk 4b + grp
    int foff[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) foff[b] = r16 * kSeg + seg_pos(r16, 4 * b + grp) * 16;

    const int nseg = KS > wave ? (KS - wave + kWaves - 1) / kWaves : 0;
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nseg) issue(wave + kWaves * d, d);
    for (int i = 0; i < nseg; ++i) {
        const int buf = i % D;
        // stage i has landed once only the later stages' DMA remains
        if (D >= 2 && i + 1 < nseg) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        const int8_t* st = my + buf * STAGE;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            i32x4 bf[NG], af[TM];
#pragma unroll
            for (int g = 0; g < NG; ++g) bf[g] = *(const i32x4*)(st + g * kTile + foff[b]);
#pragma unroll
            for (int t = 0; t < TM; ++t) af[t] = *(const i32x4*)(st + (NG + t) * kTile + foff[b]);
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    acc[t][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[t], bf[g], acc[t][g], 0, 0, 0);
        }
        if (i + D < nseg) {
            // refill this buffer once its fragments are in registers
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            issue(wave + kWaves * (i + D), buf);
        }
    }

    // ---- whole 64-byte blocks past the segments, then a partial block
    const int KB = k / kBlk;
    for (int kb = KS * 4 + wave; kb < KB; kb += kWaves) {
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

    // the partial sums meet in LDS (the staging area, free once every
    // wavefront is past its loop)
    __syncthreads();
    i32x4 (*red)[TM][NG][64] = (i32x4 (*)[TM][NG][64])smem;
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
        swo = sb[scalar_scales ? 0 : o];
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
                float y = (float)acc[t][g][r] * sa[scalar_scales ? 0 : row] * swo;
                if (bias_kind) y = y + bo;
                if constexpr (OUT == 0) ((float*)Y)[off] = y;
                else ((__bf16*)Y)[off] = (__bf16)y;
            }
        }
    }
    }
}

template <int TM, int NG, int D, int W>
hipError_t launch_tm(const int8_t* xq, const float* sx, int m, const int8_t* wq, const float* sw, int n, int k,
                     const void* bias, int bias_kind, void* y, int out_kind, int scalar_scales,
                     hipStream_t st) {
    const dim3 grid((n + 16 * NG - 1) / (16 * NG)), block(64 * W);
    switch (out_kind) {
        case 0:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, D, W, 0>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y, scalar_scales);
            break;
        case 1:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, D, W, 1>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y, scalar_scales);
            break;
        default:
            hipLaunchKernelGGL((skinny_kernel<TM, NG, D, W, 2>), grid, block, 0, st, xq, wq, m, n, k, sx, sw, bias,
                               bias_kind, y, scalar_scales);
            break;
    }
    return hipGetLastError();
}

}  // namespace

// Per token-group count TM: weight rows per workgroup 16 * NG, LDS stages
// per wavefront D, wavefronts per workgroup W (measured best on MI355X for
// 16 tokens: 2 wavefronts x 3 stages x 32 rows, 72 KiB of LDS, two
// workgroups per CU). More token groups take more LDS per stage, so fewer
// stages; every workgroup reads all m token rows once, so more weight rows
// per workgroup keep that traffic down for 33-64 tokens.
hipError_t sq_launch_gemm_skinny(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                 int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                 int scalar_scales, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch ((mi + 15) / 16) {
        case 1: return launch_tm<1, 2, 3, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st);
        case 2: return launch_tm<2, 2, 2, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st);
        case 3: return launch_tm<3, 4, 1, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st);
        case 4: return launch_tm<4, 4, 1, 2>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st);
        default: return hipErrorInvalidValue;
    }
}
