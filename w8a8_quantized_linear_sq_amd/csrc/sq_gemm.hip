// sq_gemm.hip -- INT8 x INT8 -> INT32 product with the dequantisation fused
// into its epilogue, for gfx950 (CDNA4) int8 MFMA.
//
// Page "w8a8_smoothquant.py" (BiGRU_T_version), SmoothQuantW8A8.forward:
// the page multiplies the dequantised operands in fp32 and notes that real
// hardware does INT8 x INT8 -> INT32 -> fp32. Here
//   acc[t][o] = sum_j xq[t][j] * wq[o][j]                  (exact int32)
//   y[t][o]   = f32(acc) * sx[t] * sw[o] (+ bias[o])       (fp32 -> out type)
//
// Design (gfx950):
//   * one 256-thread workgroup (4 wavefronts in a 2 x 2 grid) per BM x BN
//     output tile; each wavefront owns a (BM/2) x (BN/2) block held in
//     accumulation registers as 32 x 32 tiles of v_mfma_i32_32x32x32_i8;
//   * K is walked in BK = 64-byte steps. A and B tiles go global -> registers
//     -> LDS, double-buffered: the loads of step k+1 are in flight while the
//     MFMAs of step k run, and one barrier per step separates the buffers;
//   * LDS rows are padded to 80 bytes so that the 16-byte operand reads of
//     a wavefront hit distinct banks;
//   * rows past m or n are clamped for loading (their results are never
//     stored); K-chunks past k are zero-filled;
//   * the 1-D grid is remapped so that the tiles dispatched to one XCD (the
//     hardware deals workgroups round-robin over the 8 XCDs) form a compact
//     block sharing A rows and B columns in that XCD's L2.
#include "sq_device.h"

using namespace sq;

namespace {

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 16;  // padded LDS row, bytes
constexpr int kXcds = 8;

// MFMA 32x32x32 i8 operand: lane l holds 16 k-consecutive bytes of row
// (l % 32) at k offset 16 * (l / 32) of a 32-wide k slice; A and B use the
// same mapping, so the hardware's pairing of bytes is the same for both.
// Result: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l % 32.

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int m, int n, int k,
    const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
    int bias_kind, void* __restrict__ Y, int grid_m, int grid_n) {
    constexpr int WM = BM / 2, WN = BN / 2;  // per-wavefront block
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_CHUNKS = BM * (kBK / 16) / 256;  // 16-byte chunks per thread
    constexpr int B_CHUNKS = BN * (kBK / 16) / 256;
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * kLdsRow];
    int8_t* As = smem;                              // [2][BM][kLdsRow]
    int8_t* Bs = smem + 2 * BM * kLdsRow;           // [2][BN][kLdsRow]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- tile order: XCD-compact, then grouped along m --------------------
    const int total = grid_m * grid_n;
    int pid = blockIdx.x;
    if (total % kXcds == 0) pid = (pid % kXcds) * (total / kXcds) + pid / kXcds;
    constexpr int GROUP = 4;
    const int group_size = GROUP * grid_n;
    const int first_m = (pid / group_size) * GROUP;
    const int gm = min(grid_m - first_m, GROUP);
    const int tile_m = first_m + (pid % group_size) % gm;
    const int tile_n = (pid % group_size) / gm;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // ---- global -> register mapping: chunk c of row r ---------------------
    const int ld_c = tid & 3;   // 16-byte chunk inside the 64-byte k step
    const int ld_r = tid >> 2;  // first row; rows step by 64
    const int8_t* a_ptr[A_CHUNKS];
    const int8_t* b_ptr[B_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        int r = min(m0 + ld_r + 64 * i, m - 1);
        a_ptr[i] = A + (int64_t)r * k + ld_c * 16;
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        int r = min(n0 + ld_r + 64 * i, n - 1);
        b_ptr[i] = B + (int64_t)r * k + ld_c * 16;
    }
    i32x4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load_tile = [&](int kt) {
        const int kb = kt * kBK;
        const bool ok = kb + ld_c * 16 < k;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i)
            ra[i] = ok ? *(const i32x4*)(a_ptr[i] + kb) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i)
            rb[i] = ok ? *(const i32x4*)(b_ptr[i] + kb) : i32x4{0, 0, 0, 0};
    };
    auto store_tile = [&](int buf) {
        int8_t* as = As + buf * BM * kLdsRow;
        int8_t* bs = Bs + buf * BN * kLdsRow;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i)
            *(i32x4*)(as + (ld_r + 64 * i) * kLdsRow + ld_c * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i)
            *(i32x4*)(bs + (ld_r + 64 * i) * kLdsRow + ld_c * 16) = rb[i];
    };

    i32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = i32x16{};

    const int KT = (k + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int fr = lane & 31;          // operand row inside a 32-row slice
    const int fk = (lane >> 5) * 16;   // operand k offset inside a 32-wide slice
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
        const int8_t* as = As + cur * BM * kLdsRow + (wm * WM + fr) * kLdsRow + fk;
        const int8_t* bs = Bs + cur * BN * kLdsRow + (wn * WN + fr) * kLdsRow + fk;
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 32) {
            i32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = *(const i32x4*)(as + i * 32 * kLdsRow + ks);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = *(const i32x4*)(bs + j * 32 * kLdsRow + ks);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    const int ecol = lane & 31;
    const int erow = (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WN + j * 32 + ecol;
        if (col >= n) continue;
        float swc = 0.0f, bc = 0.0f;
        if constexpr (OUT != 2) {
            swc = sb[col];
            if (bias_kind == 1) bc = ((const float*)bias)[col];
            else if (bias_kind == 2) bc = __uint_as_float((uint32_t)((const uint16_t*)bias)[col] << 16);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + erow + (r & 3);
                if (row >= m) continue;
                const int64_t off = (int64_t)row * n + col;
                const int a = acc[i][j][r];
                if constexpr (OUT == 2) {
                    ((int*)Y)[off] = a;
                } else {
                    float y = (float)a * sa[row] * swc;
                    if (bias_kind) y = y + bc;
                    if constexpr (OUT == 0) ((float*)Y)[off] = y;
                    else ((__bf16*)Y)[off] = (__bf16)y;
                }
            }
        }
    }
}

template <int BM, int BN>
hipError_t launch_tile(const int8_t* xq, const float* sx, int m, const int8_t* wq, const float* sw,
                       int n, int k, const void* bias, int bias_kind, void* y, int out_kind,
                       hipStream_t st) {
    const int gm = (m + BM - 1) / BM, gn = (n + BN - 1) / BN;
    dim3 grid(gm * gn), block(256);
    switch (out_kind) {
        case 0:
            hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, 0>), grid, block, 0, st, xq, wq, m, n, k, sx, sw,
                               bias, bias_kind, y, gm, gn);
            break;
        case 1:
            hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, 1>), grid, block, 0, st, xq, wq, m, n, k, sx, sw,
                               bias, bias_kind, y, gm, gn);
            break;
        default:
            hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, 2>), grid, block, 0, st, xq, wq, m, n, k, sx, sw,
                               bias, bias_kind, y, gm, gn);
            break;
    }
    return hipGetLastError();
}

}  // namespace

// Tile choice: the configuration whose tiles cover m x n with the fewest
// idle MFMA slots over whole waves of 256 workgroups (one per CU), larger
// tiles first on ties.
hipError_t sq_launch_gemm(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                          const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                          void* y, int out_kind, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    struct Cfg { int bm, bn; };
    const Cfg cfgs[] = {{256, 256}, {128, 256}, {128, 128}};
    int best = 0;
    double best_eff = -1.0;
    for (int i = 0; i < 3; ++i) {
        const int64_t tiles = ((m + cfgs[i].bm - 1) / cfgs[i].bm) * ((n + cfgs[i].bn - 1) / cfgs[i].bn);
        const int64_t waves = (tiles + 255) / 256;
        const double eff = (double)(m * n) / ((double)waves * 256.0 * cfgs[i].bm * cfgs[i].bn);
        if (eff > best_eff * 1.05) {
            best_eff = eff;
            best = i;
        }
    }
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch (best) {
        case 0: return launch_tile<256, 256>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        case 1: return launch_tile<128, 256>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
        default: return launch_tile<128, 128>(xq, sx, mi, wq, sw, ni, ki, bias, bias_kind, y, out_kind, st);
    }
}
