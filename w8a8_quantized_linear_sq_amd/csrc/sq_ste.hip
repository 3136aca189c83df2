// sq_ste.hip -- the straight-through backward of the quantized forward and
// the gradient of the learnable alpha, for gfx950.
//
// Page "w8a8_smoothquant.py" (BiGRU_T_version): the module docstring's notes
// on the learnable alpha (alpha = sigmoid(eta), round and clamp passed
// through by a straight-through estimator, a relative squared error as an
// auxiliary loss), STEQuantize / ste_quantize (the gradient of the
// dequantised value goes to the quantiser's input unchanged, none to its
// scale) and SmoothQuantW8A8.forward (s recomputed from alpha, X~ = X / s,
// W~ = W * s, both quantised, Y = Xd Wd^T + bias). With Xd = xq * sx (per
// token) and Wd = wq * sw (per output channel):
//   gX[t][j] = sum_o dy[t][o] wq[o][j] sw[o]     dx = gX / s_j
//   gW[o][j] = sum_t dy[t][o] xq[t][j] sx[t]     dw = gW * s_j
//   db[o]    = sum_t dy[t][o]
//   ds_j     = sum_o gW[o][j] w[o][j] - sum_t gX[t][j] x[t][j] / s_j^2
//   dalpha   = sum_j [s_raw_j >= 1e-8] ds_j s_raw_j (ln mx_j + ln mw_j)
//   deta     = dalpha alpha (1 - alpha)
//
// Design:
//   * both products contract over the rows of their int8 operand, so the
//     operands are first rearranged so that the contraction is contiguous
//     (the form the MFMA tile kernel reads): the fp32 factor
//     v = RN32(dy * scale) is split exactly into three bf16 planes,
//     v = a1 + a2 + a3 (8 significant bits each), laid side by side along
//     the contraction; the int8 codes are transposed into bf16 (exact).
//     The tile kernel's periodic-B form then sums the three planes against
//     the same codes in one launch: every product is exact in fp32 and only
//     the fp32 accumulation rounds, as in the page's fp32 autograd;
//   * the two products write gX and gW into dx and dw; where gX's output
//     has few 256 x 256 tiles (the prefill shape), its contraction is split
//     over the output channels in two halves that run side by side in one
//     launch of 256 x 256 tiles, each half a matrix of its own, and the
//     column pass adds them (half 0 + half 1) before the fold;
//   * one column-sum pass per output folds the smoothing (dx = gX / s with
//     IEEE division, dw = gW * s) and accumulates sum gX x and sum gW w in
//     binary64 per row group (a fixed order: the same inputs give the same
//     bits);
//   * ds_j with its share of dalpha and the bias gradient share one launch
//     (independent blocks); the alpha sum follows; all fixed-order trees.
#include "sq_device.h"

using namespace sq;

namespace {

// bf16 round-to-nearest-even of a finite binary32 value (the bit pattern)
__device__ __forceinline__ uint32_t bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// v = a1 + a2 + a3 exactly, each a bf16: a1 = RN_bf16(v) leaves a remainder
// of at most 16 significant bits (exact in fp32), a2 = RN_bf16 of that
// leaves at most 8, which a3 holds exactly (as long as no piece falls below
// bf16's normal range, i.e. |v| >= 2^-110; below that the lost part is
// under 2^-133 in magnitude).
__device__ __forceinline__ void split3(float v, uint32_t& a1, uint32_t& a2, uint32_t& a3) {
    a1 = bf16_rne(v);
    const float r1 = v - bf16_val(a1);
    a2 = bf16_rne(r1);
    const float r2 = r1 - bf16_val(a2);
    a3 = bf16_rne(r2);
}

template <bool BF16>
__device__ __forceinline__ float load_val(const void* p, int64_t i) {
    if constexpr (BF16) return bf16_val(((const uint16_t*)p)[i]);
    else return ((const float*)p)[i];
}

// Plane p of RN32(dy[t][o] * sc[o]) for o < n, zero for n <= o < ld (ld a
// multiple of 64), with the columns in parts of nh (nh divides ld, a
// multiple of 32): part h = o / nh is a matrix [m][3 nh] of its own at
// h * m * 3 nh, row t holding the three planes of its nh columns side by
// side, a[h][t][p * nh + o % nh] (nh = ld: one part). Thread: 8
// consecutive o of every row it visits. VEC (dy and sc 16-byte aligned, n a
// multiple of 8): dy and sc read 16 bytes at a time; else, and past n,
// element by element. The planes are written 16 bytes at a time.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void ste_pack_rows_kernel(const void* __restrict__ dy, const float* __restrict__ sc,
                                                            int64_t m, int64_t n, int64_t ld, int64_t nh,
                                                            uint16_t* __restrict__ a) {
    const int64_t o0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (o0 >= ld) return;
    uint16_t* part = a + (o0 / nh) * m * 3 * nh + o0 % nh;
    const bool whole = VEC && o0 + 8 <= n;
    float f[8];
    if (whole) {
        load8<false>(sc, o0, f);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = o0 + e < n ? sc[o0 + e] : 0.0f;
    }
    for (int64_t t = blockIdx.y; t < m; t += gridDim.y) {
        float v[8];
        if (whole) {
            load8<BF16>(dy, t * n + o0, v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = o0 + e < n ? load_val<BF16>(dy, t * n + o0 + e) : 0.0f;
        }
        uint32_t h[3][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split3(v[e] * f[e], h[0][e], h[1][e], h[2][e]);
        uint16_t* row = part + t * 3 * nh;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            const u32x4 w = {h[p][0] | (h[p][1] << 16), h[p][2] | (h[p][3] << 16), h[p][4] | (h[p][5] << 16),
                             h[p][6] | (h[p][7] << 16)};
            *(u32x4*)(row + p * nh) = w;
        }
    }
}

// a[o][p * ld + t] = plane p of RN32(dy[t][o] * sc[t]) for t < m, zero for
// m <= t < ld; rows o < n. 64 x 64 tiles through LDS (tile (ti, oi) with
// ti = blockIdx.x % (ld / 64)).
constexpr int kTP = 72;  // LDS row pitch in bf16 (16-byte aligned rows)
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void ste_pack_cols_kernel(const void* __restrict__ dy, const float* __restrict__ sc,
                                                            int64_t m, int64_t n, int64_t ld, uint16_t* __restrict__ a) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[3][64][kTP];  // [plane][o][t]
    const int64_t tiles_t = ld / 64;
    const int64_t t0 = (blockIdx.x % tiles_t) * 64, o0 = (blockIdx.x / tiles_t) * 64;
    // thread: four consecutive o (tx) of four consecutive t (ty), so that
    // each plane's four t of one o go to LDS as one 8-byte store
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    uint32_t h[3][4][4];  // [plane][o][t]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tt = 4 * ty + r;
        const int64_t t = t0 + tt;
        const float f = t < m ? sc[t] : 0.0f;
        // four consecutive o of row t: one load when VEC (dy 16-byte aligned,
        // n a multiple of 4) and all four lie below n
        float d[4];
        if (VEC && t < m && o0 + tx * 4 + 4 <= n) {
            load4<BF16>(dy, t * n + o0 + tx * 4, d);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t o = o0 + tx * 4 + e;
                d[e] = (t < m && o < n) ? load_val<BF16>(dy, t * n + o) : 0.0f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t o = o0 + tx * 4 + e;
            const float v = (t < m && o < n) ? d[e] * f : 0.0f;
            split3(v, h[0][e][r], h[1][e][r], h[2][e][r]);
        }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *(u32x2*)&tile[p][tx * 4 + e][4 * ty] =
                u32x2{h[p][e][0] | (h[p][e][1] << 16), h[p][e][2] | (h[p][e][3] << 16)};
    __syncthreads();
    // 64 rows o x 3 planes x 8 pieces of 16 bytes (8 t each)
    for (int c = threadIdx.x; c < 64 * 3 * 8; c += 256) {
        const int oo = c / 24, p = (c / 8) % 3, piece = c % 8;
        const int64_t o = o0 + oo;
        if (o >= n) continue;
        const u32x4 v = *(const u32x4*)&tile[p][oo][piece * 8];
        *(u32x4*)(a + o * 3 * ld + p * ld + t0 + piece * 8) = v;
    }
}

// bf16(q[o][j]) (exact) for o < rows, zero for rows <= o < ld; j < k, with
// the o in parts of nh (nh divides ld, a multiple of 8): part h = o / nh is
// a matrix [k][nh] of its own at h * k * nh, b[h][j][o % nh] (nh = ld: one
// part, b[j][o]). q is [rows][k] int8 row-major; 64 x 64 tiles through LDS.
constexpr int kQP = 68;  // LDS row pitch in bytes
__global__ __launch_bounds__(256) void ste_transpose_codes_kernel(const int8_t* __restrict__ q, int64_t rows,
                                                                  int64_t k, int64_t ld, int64_t nh,
                                                                  uint16_t* __restrict__ b) {
    __shared__ __attribute__((aligned(16))) int8_t tile[64][kQP];  // [o][j]
    const int64_t tiles_o = ld / 64;
    const int64_t o0 = (blockIdx.x % tiles_o) * 64, j0 = (blockIdx.x / tiles_o) * 64;
    {
        const int oo = threadIdx.x >> 2, part = threadIdx.x & 3;
        const int64_t o = o0 + oo, j = j0 + part * 16;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (o < rows && j < k) v = *(const u32x4*)(q + o * k + j);  // k % 16 == 0: whole pieces
#pragma unroll
        for (int e = 0; e < 4; ++e) *(uint32_t*)&tile[oo][part * 16 + 4 * e] = v[e];
    }
    __syncthreads();
    // thread c < 128: 4 consecutive j (jq) x 8 consecutive o (piece), read
    // as one 4-byte word per o (the 4 j of that o), written as 4 rows of 8 o
    if (threadIdx.x < 128) {
        const int piece = threadIdx.x & 7, jq = threadIdx.x >> 3;
        uint32_t word[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) word[r] = *(const uint32_t*)&tile[piece * 8 + r][jq * 4];
        const int64_t o = o0 + piece * 8;  // 8 o in one part
        uint16_t* dst = b + (o / nh) * k * nh + o % nh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = j0 + jq * 4 + q;
            if (j >= k) break;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // |code| <= 128: exact in bf16
                const float lo = (float)(int8_t)(word[2 * e] >> (8 * q));
                const float hi = (float)(int8_t)(word[2 * e + 1] >> (8 * q));
                w[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
            }
            *(u32x4*)(dst + j * nh) = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// Column sums over row groups, with an optional elementwise factor and an
// optional fold of s:
//   part[g][c] = sum over rows r of group g of y[r][c] * z[r][c] (binary64,
//                rows in order; z = 1 when ZK == 0)
//   OP 1: out[r][c] = y[r][c] / s[c] (IEEE);  OP 2: out[r][c] = y[r][c] * s[c]
// with out = y (in place) unless TWO: then y holds two fp32 partial
// matrices, the second at y + rows * cols, and y[r][c] stands for their
// sum RN32(y0 + y1) (the halves of a split product), written to out.
// y is fp32 when OP != 0 (else YBF16 selects its type); z is fp32 (ZK 1)
// or bf16 (ZK 2). VEC: cols % 4 == 0 and y and z 16-byte aligned (8 for a
// bf16 y), 4 columns per thread as one vector; otherwise 4 scalar columns.
template <int ZK, int OP, bool YBF16, bool VEC, bool TWO = false>
__global__ __launch_bounds__(256) void ste_colsum_kernel(void* __restrict__ y, const void* __restrict__ z,
                                                         const float* __restrict__ s, int64_t rows, int64_t cols,
                                                         int64_t rpg, double* __restrict__ part,
                                                         float* __restrict__ out) {
    static_assert(!TWO || (OP != 0 && !YBF16), "two partials: fp32, folded into out");
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (c0 >= cols) return;
    const int64_t g = blockIdx.y;
    const int64_t r0 = g * rpg, r1 = min(rows, r0 + rpg);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (OP != 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = c0 + e < cols ? s[c0 + e] : 1.0f;
    }
    auto load_row = [&](int64_t r, float (&yv)[4], float (&zv)[4]) {
        const int64_t base = r * cols + c0;
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[e] = 1.0f;
        if constexpr (VEC && !YBF16) {
            const float4 v = *(const float4*)((const float*)y + base);
            yv[0] = v.x; yv[1] = v.y; yv[2] = v.z; yv[3] = v.w;
            if constexpr (TWO) {
                const float4 u = *(const float4*)((const float*)y + rows * cols + base);
                yv[0] += u.x; yv[1] += u.y; yv[2] += u.z; yv[3] += u.w;
            }
        } else if constexpr (VEC) {
            const u32x2 v = *(const u32x2*)((const uint16_t*)y + base);
            yv[0] = bf16_lo(v.x); yv[1] = bf16_hi(v.x); yv[2] = bf16_lo(v.y); yv[3] = bf16_hi(v.y);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yv[e] = c0 + e < cols ? load_val<YBF16>(y, base + e) : 0.0f;
                if constexpr (TWO) yv[e] += c0 + e < cols ? ((const float*)y)[rows * cols + base + e] : 0.0f;
            }
        }
        if constexpr (ZK == 1 && VEC) {
            const float4 v = *(const float4*)((const float*)z + base);
            zv[0] = v.x; zv[1] = v.y; zv[2] = v.z; zv[3] = v.w;
        } else if constexpr (ZK == 2 && VEC) {
            const u32x2 v = *(const u32x2*)((const uint16_t*)z + base);
            zv[0] = bf16_lo(v.x); zv[1] = bf16_hi(v.x); zv[2] = bf16_lo(v.y); zv[3] = bf16_hi(v.y);
        } else if constexpr (ZK != 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) zv[e] = c0 + e < cols ? load_val<ZK == 2>(z, base + e) : 0.0f;
        }
    };
    auto finish_row = [&](int64_t r, const float (&yv)[4], const float (&zv)[4]) {
        const int64_t base = r * cols + c0;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += (double)yv[e] * (double)zv[e];
        if constexpr (OP != 0) {
            float o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = OP == 1 ? yv[e] / sc[e] : yv[e] * sc[e];
            float* dst = TWO ? out : (float*)y;
            if constexpr (VEC) {
                *(float4*)(dst + base) = make_float4(o4[0], o4[1], o4[2], o4[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < cols) dst[base + e] = o4[e];
            }
        }
    };
    // rows in order (the binary64 sums' order), four rows' loads in flight
    constexpr int U = 4;
    int64_t r = r0;
    for (; r + U <= r1; r += U) {
        float yv[U][4], zv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) load_row(r + u, yv[u], zv[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) finish_row(r + u, yv[u], zv[u]);
    }
    for (; r < r1; ++r) {
        float yv[4], zv[4];
        load_row(r, yv, zv);
        finish_row(r, yv, zv);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (c0 + e < cols) part[g * cols + c0 + e] = acc[e];
}

// Sums of row-group partials for one column per lane: wavefront `wave` of
// kSumWaves takes the groups wave, wave + kSumWaves, ... in that order with
// eight loads in flight, and the callers add the wavefronts' sums in
// wavefront order through LDS, so every call sums in the same order.
constexpr int kSumWaves = 8;

__device__ __forceinline__ double sum_groups(const double* __restrict__ p, int64_t groups, int64_t stride,
                                             int64_t j, int wave) {
    double acc = 0.0;
    int64_t g = wave;
    for (; g + kSumWaves * 7 < groups; g += kSumWaves * 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(g + kSumWaves * u) * stride + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; g < groups; g += kSumWaves) acc += p[g * stride + j];
    return acc;
}

// ds[j] = sum_o gW[o][j] w[o][j] - sum_t gX[t][j] x[t][j] / s_j^2 from the
// column passes' partials, and the per-channel term of dalpha,
//   term[j] = [s_raw_j >= floor] ds_j s_raw_j (ln mx_j + ln mw_j)
// (0 without calibration). A block owns 64 channels.
__device__ __forceinline__ void ste_ds_block(int64_t blk, double (&red)[2][kSumWaves][64],
                                             const double* __restrict__ px, int64_t gx,
                                             const double* __restrict__ pw, int64_t gw, const float* __restrict__ s,
                                             const float* __restrict__ mx, const float* __restrict__ mw, double a_x,
                                             double a_w, int64_t k, float* __restrict__ ds_out,
                                             double* __restrict__ term) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j = blk * 64 + lane;
    double sw_ = 0.0, sx_ = 0.0;
    if (j < k) {
        sw_ = sum_groups(pw, gw, k, j, wave);
        sx_ = sum_groups(px, gx, k, j, wave);
    }
    red[0][wave][lane] = sw_;
    red[1][wave][lane] = sx_;
    __syncthreads();
    if (wave != 0 || j >= k) return;
    sw_ = 0.0;
    sx_ = 0.0;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) {
        sw_ += red[0][w][lane];
        sx_ += red[1][w][lane];
    }
    const double sj = (double)s[j];
    const double ds = sw_ - sx_ / (sj * sj);
    if (ds_out) ds_out[j] = (float)ds;
    double tj = 0.0;
    if (mx) {
        const float mxj = fmaxf(mx[j], kFloor);
        const float num = (float)pow64((double)mxj, a_x);
        const float den = (float)pow64((double)mw[j], a_w);
        const float raw = num / den;
        if (raw >= kFloor) tj = ds * (double)raw * (log((double)mxj) + log((double)mw[j]));
    }
    term[j] = tj;
}

// out[0] = dalpha = sum_j term[j], out[1] = deta = dalpha alpha (1 - alpha):
// one block, each thread a strided range in order, then a fixed tree.
__global__ __launch_bounds__(256) void ste_alpha_kernel(const double* __restrict__ term, int64_t k, double alpha,
                                                        double* __restrict__ out) {
    __shared__ double red[256];
    double acc = 0.0;
    // unrolled so that the loads are issued together; the adds keep their
    // order
#pragma unroll 8
    for (int64_t j = threadIdx.x; j < k; j += 256) acc += term[j];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = red[0];
        out[1] = red[0] * alpha * (1.0 - alpha);
    }
}

// db[o] = sum_g pb[g][o] (binary64 in the fixed order of sum_groups, then
// fp32); a block owns 64 outputs
__device__ __forceinline__ void ste_bias_block(int64_t blk, double (&red)[kSumWaves][64],
                                               const double* __restrict__ pb, int64_t groups, int64_t n,
                                               float* __restrict__ db) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t o = blk * 64 + lane;
    red[wave][lane] = o < n ? sum_groups(pb, groups, n, o, wave) : 0.0;
    __syncthreads();
    if (wave != 0 || o >= n) return;
    double acc = 0.0;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) acc += red[w][lane];
    db[o] = (float)acc;
}

// ds (blocks below kblocks, 64 channels each) and db (the blocks after
// them, 64 outputs each) in one launch: both only read the column passes'
// partials, so their blocks are independent.
__global__ __launch_bounds__(64 * kSumWaves) void ste_finish_kernel(
    const double* __restrict__ px, int64_t gx, const double* __restrict__ pw, int64_t gw,
    const float* __restrict__ s, const float* __restrict__ mx, const float* __restrict__ mw, double a_x, double a_w,
    int64_t k, float* __restrict__ ds_out, double* __restrict__ term, int64_t kblocks,
    const double* __restrict__ pb, int64_t gb, int64_t n, float* __restrict__ db) {
    __shared__ double red[2][kSumWaves][64];
    const int64_t blk = blockIdx.x;
    if (blk < kblocks)
        ste_ds_block(blk, red, px, gx, pw, gw, s, mx, mw, a_x, a_w, k, ds_out, term);
    else
        ste_bias_block(blk - kblocks, red[0], pb, gb, n, db);
}

// dy_q[i] = 2 (y_q[i] - y_fp[i]) / den and loss = ||y_fp - y_q||^2 / den with
// den = max(||y_fp||^2, 1e-24), from the two norms in norms[0], norms[1]
__global__ __launch_bounds__(256) void ste_aux_grad_kernel(const float* __restrict__ y_fp, const float* __restrict__ y_q,
                                                           int64_t count, const double* __restrict__ norms,
                                                           float* __restrict__ dy_q, double* __restrict__ loss) {
    const double f = norms[1], d = norms[0];
    const double den = fmax(f * f, 1e-24);
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride)
        dy_q[i] = (float)(2.0 * ((double)y_q[i] - (double)y_fp[i]) / den);
    if (blockIdx.x == 0 && threadIdx.x == 0) *loss = d * d / den;
}

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }
bool aligned16_ptr(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Row groups of a column-sum pass: about 2048 blocks in all, at least 8
// rows per group, and at most 128 groups, since every group writes a row
// of binary64 partials that the ds and bias kernels read back (at the
// prefill shape 128 against up to 512 measured 5 us faster per call; 64
// slower)
int64_t colsum_groups(int64_t rows, int64_t cols) {
    const int64_t gx = (cols + 1023) / 1024;
    int64_t g = 2048 / gx;
    g = std::max<int64_t>(1, std::min<int64_t>(g, (rows + 7) / 8));
    return std::min<int64_t>(g, 128);
}

template <int ZK, int OP, bool YBF16, bool TWO = false>
hipError_t launch_colsum(void* y, const void* z, const float* s, int64_t rows, int64_t cols, int64_t groups,
                         double* part, bool vec, hipStream_t st, float* out = nullptr) {
    const int64_t rpg = (rows + groups - 1) / groups;
    const dim3 grid((unsigned)((cols + 1023) / 1024), (unsigned)groups);
    if (vec)
        hipLaunchKernelGGL((ste_colsum_kernel<ZK, OP, YBF16, true, TWO>), grid, dim3(256), 0, st, y, z, s, rows, cols,
                           rpg, part, out);
    else
        hipLaunchKernelGGL((ste_colsum_kernel<ZK, OP, YBF16, false, TWO>), grid, dim3(256), 0, st, y, z, s, rows,
                           cols, rpg, part, out);
    return hipGetLastError();
}

// gX with its contraction (the n output channels, three planes each) split
// in two halves run side by side in one launch of 256 x 256 tiles, where
// gX [m][k] alone has at most half as many such tiles as the chip has
// compute units and m is large enough for the product to dominate; the
// halves' fp32 results are added in a fixed order by the column pass.
bool ste_split_gx(int64_t m, int64_t k) { return m >= 1024 && ((m + 255) / 256) * ((k + 255) / 256) <= 128; }

}  // namespace

// Workspace layout of the straight-through backward (each region 256-byte
// aligned): the two packed factors, the two transposed codes, the column
// partial sums of the three passes and the per-channel terms of dalpha.
SteLayout sq_ste_layout(int64_t m, int64_t n, int64_t k) {
    SteLayout L{};
    const int64_t m64 = pad64(m), n64 = pad64(n);
    L.m64 = m64;
    L.n64 = n64;
    L.gx = colsum_groups(m, k);
    L.gw = colsum_groups(n, k);
    L.gb = colsum_groups(m, n);
    size_t off = 0;
    L.split = ste_split_gx(m, k);
    L.nh = L.split ? n64 / 2 : n64;
    L.a1 = off; off = align256(off + (size_t)m * 3 * n64 * 2);
    L.bw = off; off = align256(off + (size_t)k * n64 * 2);
    L.a2 = off; off = align256(off + (size_t)n * 3 * m64 * 2);
    L.bx = off; off = align256(off + (size_t)k * m64 * 2);
    L.px = off; off = align256(off + (size_t)L.gx * k * 8);
    L.pw = off; off = align256(off + (size_t)L.gw * k * 8);
    L.pb = off; off = align256(off + (size_t)L.gb * n * 8);
    L.term = off; off = align256(off + (size_t)k * 8);
    L.gxh = off; off = align256(off + (L.split ? (size_t)2 * m * k * 4 : 0));
    L.bytes = off;
    return L;
}

hipError_t sq_launch_ste_backward(const void* dy, int dy_bf16, int64_t m, int64_t n, int64_t k, const void* x,
                                  int x_bf16, const void* w, int w_bf16, const float* s, const int8_t* xq,
                                  const float* sx, const int8_t* wq, const float* sw, const float* mx,
                                  const float* mw, double alpha, float* dx, float* dw, float* db, float* ds,
                                  double* dalpha_deta, void* workspace, hipStream_t st) {
    const SteLayout L = sq_ste_layout(m, n, k);
    char* base = (char*)workspace;
    uint16_t* a1 = (uint16_t*)(base + L.a1);
    uint16_t* bw = (uint16_t*)(base + L.bw);
    uint16_t* a2 = (uint16_t*)(base + L.a2);
    uint16_t* bx = (uint16_t*)(base + L.bx);
    double* px = (double*)(base + L.px);
    double* pw = (double*)(base + L.pw);
    double* pb = (double*)(base + L.pb);
    double* term = (double*)(base + L.term);
    float* gxh = (float*)(base + L.gxh);
    hipError_t e;
    // gX: a1 = RN32(dy * sw) in three planes [m][3 n64], bw = wq^T [k][n64];
    // split: each in two parts over the n (a1 [2][m][3 nh], bw [2][k][nh]),
    // the two halves of gX to gxh [2][m][k]
    {
        const dim3 grid((unsigned)((L.n64 + 2047) / 2048), (unsigned)std::min<int64_t>(m, 65535));
        const bool vec = aligned16_ptr(dy) && aligned16_ptr(sw) && n % 8 == 0;
        if (dy_bf16) {
            if (vec) hipLaunchKernelGGL((ste_pack_rows_kernel<true, true>), grid, dim3(256), 0, st, dy, sw, m, n, L.n64, L.nh, a1);
            else hipLaunchKernelGGL((ste_pack_rows_kernel<true, false>), grid, dim3(256), 0, st, dy, sw, m, n, L.n64, L.nh, a1);
        } else {
            if (vec) hipLaunchKernelGGL((ste_pack_rows_kernel<false, true>), grid, dim3(256), 0, st, dy, sw, m, n, L.n64, L.nh, a1);
            else hipLaunchKernelGGL((ste_pack_rows_kernel<false, false>), grid, dim3(256), 0, st, dy, sw, m, n, L.n64, L.nh, a1);
        }
        hipLaunchKernelGGL(ste_transpose_codes_kernel, dim3((unsigned)((L.n64 / 64) * ((k + 63) / 64))), dim3(256), 0,
                           st, wq, n, k, L.n64, L.nh, bw);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = L.split ? sq_launch_gemm_bf16_periodic_split2(a1, bw, m, k, 3 * L.nh * 2, L.nh * 2, gxh, st)
                    : sq_launch_gemm_bf16_periodic(a1, bw, m, k, 3 * L.n64 * 2, L.n64 * 2, dx, st);
        if (e != hipSuccess) return e;
    }
    // gW: a2 = RN32(dy^T * sx) in three planes [n][3 m64], bx = xq^T [k][m64]
    {
        const dim3 grid((unsigned)((L.m64 / 64) * ((n + 63) / 64)));
        const bool vec = aligned16_ptr(dy) && n % 4 == 0;
        if (dy_bf16) {
            if (vec) hipLaunchKernelGGL((ste_pack_cols_kernel<true, true>), grid, dim3(256), 0, st, dy, sx, m, n, L.m64, a2);
            else hipLaunchKernelGGL((ste_pack_cols_kernel<true, false>), grid, dim3(256), 0, st, dy, sx, m, n, L.m64, a2);
        } else {
            if (vec) hipLaunchKernelGGL((ste_pack_cols_kernel<false, true>), grid, dim3(256), 0, st, dy, sx, m, n, L.m64, a2);
            else hipLaunchKernelGGL((ste_pack_cols_kernel<false, false>), grid, dim3(256), 0, st, dy, sx, m, n, L.m64, a2);
        }
        hipLaunchKernelGGL(ste_transpose_codes_kernel, dim3((unsigned)((L.m64 / 64) * ((k + 63) / 64))), dim3(256), 0,
                           st, xq, m, k, L.m64, L.m64, bx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = sq_launch_gemm_bf16_periodic(a2, bx, n, k, 3 * L.m64 * 2, L.m64 * 2, dw, st);
        if (e != hipSuccess) return e;
    }
    // dx = gX / s with sum_t gX x;  dw = gW * s with sum_o gW w
    if (L.split)
        e = x_bf16 ? launch_colsum<2, 1, false, true>(gxh, x, s, m, k, L.gx, px, true, st, dx)
                   : launch_colsum<1, 1, false, true>(gxh, x, s, m, k, L.gx, px, true, st, dx);
    else
        e = x_bf16 ? launch_colsum<2, 1, false>(dx, x, s, m, k, L.gx, px, true, st)
                   : launch_colsum<1, 1, false>(dx, x, s, m, k, L.gx, px, true, st);
    if (e != hipSuccess) return e;
    e = w_bf16 ? launch_colsum<2, 2, false>(dw, w, s, n, k, L.gw, pw, true, st)
               : launch_colsum<1, 2, false>(dw, w, s, n, k, L.gw, pw, true, st);
    if (e != hipSuccess) return e;
    // db's column sums of dy
    if (db) {
        const bool vec = n % 4 == 0 && ((uintptr_t)dy & (dy_bf16 ? 7 : 15)) == 0;
        e = dy_bf16 ? launch_colsum<0, 0, true>((void*)dy, nullptr, nullptr, m, n, L.gb, pb, vec, st)
                    : launch_colsum<0, 0, false>((void*)dy, nullptr, nullptr, m, n, L.gb, pb, vec, st);
        if (e != hipSuccess) return e;
    }
    // ds and the per-channel terms of dalpha, and db, in one launch; then
    // dalpha, deta
    const int64_t kblocks = (k + 63) / 64, nblocks = db ? (n + 63) / 64 : 0;
    hipLaunchKernelGGL(ste_finish_kernel, dim3((unsigned)(kblocks + nblocks)), dim3(64 * kSumWaves), 0, st, px, L.gx,
                       pw, L.gw, s, mx, mw, alpha, 1.0 - alpha, k, ds, term, kblocks, pb, L.gb, n, db);
    hipLaunchKernelGGL(ste_alpha_kernel, dim3(1), dim3(256), 0, st, term, k, alpha, dalpha_deta);
    return hipGetLastError();
}

hipError_t sq_launch_aux_loss_grad(const float* y_fp, const float* y_q, int64_t count, double* partial,
                                   double* norms, float* dy_q, double* loss, hipStream_t st) {
    hipError_t e = sq_launch_relative_error(y_fp, y_q, count, partial, norms, st);
    if (e != hipSuccess) return e;
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, 4096);
    hipLaunchKernelGGL(ste_aux_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y_fp, y_q, count, norms, dy_q,
                       loss);
    return hipGetLastError();
}
