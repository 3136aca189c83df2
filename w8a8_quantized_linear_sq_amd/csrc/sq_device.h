// sq_device.h -- device helpers and kernel launch declarations shared by the
// HIP translation units of libsq.so (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace sq {

// The floor of the method, the binary32 value nearest to 1e-8 (0x322BCC77).
constexpr float kFloor = 1e-8f;
constexpr float kQmax = 127.0f;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 pair in one dword -> the two fp32 values (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Max over the 64 lanes of a wavefront (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Max over the 64 lanes of a wavefront for non-negative binary32 values (no
// NaN), taken on the bit patterns as unsigned integers (their order is the
// values' order): within each row of 16 lanes by DPP (swaps inside quads,
// then rotations of the row by 4 and 8), then across the four rows from one
// lane of each. Every lane must be active; the result is uniform.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, false));  // row_ror 4
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));  // row_ror 8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)u, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Eight consecutive elements at `off` of a bf16 or fp32 array as fp32
// (exact widening): one 16-byte load for bf16, two for fp32; the address
// must be 16-byte aligned.
template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t off, float (&v)[8]) {
    if constexpr (BF16) {
        const u32x4 r = *(const u32x4*)((const uint16_t*)x + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(r[i]);
            v[2 * i + 1] = bf16_hi(r[i]);
        }
    } else {
        const u32x4 a = *(const u32x4*)((const float*)x + off);
        const u32x4 b = *(const u32x4*)((const float*)x + off + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    }
}

// Four consecutive elements likewise: 8 bytes for bf16, 16 for fp32 (the
// address aligned to that size).
template <bool BF16>
__device__ __forceinline__ void load4(const void* x, int64_t off, float (&v)[4]) {
    if constexpr (BF16) {
        const u32x2 r = *(const u32x2*)((const uint16_t*)x + off);
        v[0] = bf16_lo(r[0]);
        v[1] = bf16_hi(r[0]);
        v[2] = bf16_lo(r[1]);
        v[3] = bf16_hi(r[1]);
    } else {
        const u32x4 r = *(const u32x4*)((const float*)x + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
    }
}

// The quantisers' exact division (Markstein's correction, see sq_quant.hip):
// y = RN(1/b), q0 = RN(a y), q1 = fma(fma(-q0, b, a), y, q0) = RN(a / b).
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: RN(q + kMagic)'s low byte is rint(q)

// RN(1/s) for s in [2^-40, 2^40): the hardware reciprocal refined by one
// Newton-Raphson step for 1/s in its fma form, r + r (1 - s r); on gfx950 it
// equals the IEEE quotient 1/s for every binary32 s in [2^-100, 2^100)
// (sq_selfcheck_reciprocal). Elsewhere NaN, which fails every guard.
__device__ __forceinline__ float recip_rn(float s) {
    const float r = __builtin_amdgcn_rcpf(s);
    const float y = __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    return (s >= 0x1p-40f && s < 0x1p40f) ? y : __builtin_nanf("");
}

__device__ __forceinline__ float div_rn(float a, float b, float y) {
    const float q0 = a * y;
    return __builtin_fmaf(__builtin_fmaf(-q0, b, a), y, q0);
}

// The per-row scale RN(a / 127) for a >= the floor (a may be +inf): the
// same correction with y = RN(1/127). The largest finite a keeps every step
// in the normal range, so it equals the IEEE quotient (the significand pairs
// are all checked by sq_selfcheck_division); +inf passes through.
__device__ __forceinline__ float row_scale(float a) {
    constexpr float y = 1.0f / kQmax;
    return __builtin_isinf(a) ? a : div_rn(a, kQmax, y);
}

// RN(1/s) for a row scale s >= floor / 127 (about 2^-33.6): the Newton-refined
// reciprocal of recip_rn where it is checked equal to the IEEE quotient
// (below 2^100), the IEEE division above (scales reach 2^121, and inf).
__device__ __forceinline__ float row_scale_recip(float s) {
    if (__builtin_expect(s < 0x1p100f, 1)) {
        const float r = __builtin_amdgcn_rcpf(s);
        return __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r);
    }
    return 1.0f / s;
}

// low bytes of four words -> one word
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // [a.b0, b.b0, 0, 0]
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);              // [a, b, c, d]
}

// P(x, a) = x^a through binary64 (the smoothing factor's powers): exact
// forms built from correctly rounded sqrt for a in {0, 1/4, 1/2, 3/4, 1},
// pow otherwise.
__device__ __forceinline__ double pow64(double x, double a) {
    if (a == 0.0) return 1.0;
    if (a == 1.0) return x;
    if (a == 0.5) return __builtin_sqrt(x);
    if (a == 0.25) return __builtin_sqrt(__builtin_sqrt(x));
    if (a == 0.75) return __builtin_sqrt(x) * __builtin_sqrt(__builtin_sqrt(x));
    return pow(x, a);
}

}  // namespace sq

// ---- launchers (host side), one per kernel family; each returns the
// ---- hipError_t of its launch.
hipError_t sq_launch_fill(float* p, float v, int64_t count, hipStream_t st);
// running column max of |x| folded into running_max (calibration)
hipError_t sq_launch_colmax(const void* x, int bf16, int64_t rows, int64_t k, float* running_max,
                            hipStream_t st);
// the same for a first batch: running_max = the batch's column max, whatever
// it held (one launch when the batch fits one row group)
hipError_t sq_launch_colmax_first(const void* x, int bf16, int64_t rows, int64_t k, float* running_max,
                                  hipStream_t st);
// several calibration batches (x[b], rows[b], b < nbatch <= 8) folded into
// running_max in one launch (after a zero fill when first and the rows make
// several row groups); first: running_max starts from these batches alone
hipError_t sq_launch_colmax_batches(const void* const* x, const int64_t* rows, int nbatch, int bf16, int64_t k,
                                    float* running_max, int first, hipStream_t st);
// row groups for a partial column max whose [groups][k] uint32 result must
// fit in scratch_bytes (at least 1)
int64_t sq_colmax_partial_groups(int64_t rows, int64_t k, int bf16, int64_t scratch_bytes);
// partial[g][j] = max over row group g of |x[.][j]| (binary32 bit patterns)
hipError_t sq_launch_colmax_partial(const void* x, int bf16, int64_t rows, int64_t k, int64_t groups,
                                    unsigned* partial, hipStream_t st);
// s[j] from x_max[j] and the max over groups of partial[.][j]; partial may
// alias s when groups == 1
hipError_t sq_launch_smooth_factor(const float* x_max, const unsigned* partial, int64_t groups, double a_x,
                                   double a_w, int64_t k, float* s, hipStream_t st);
hipError_t sq_launch_quantize_weight(const void* w, int bf16, const float* s, int64_t n,
                                     int64_t k, int8_t* wq, float* w_scale, hipStream_t st);
hipError_t sq_launch_quantize_act(const void* x, int bf16, const float* s, int64_t m, int64_t k,
                                  int8_t* xq, float* x_scale, hipStream_t st);
// per-tensor codes and scale of x[count] (count a multiple of 16; q 16-byte
// aligned, also holds the block maxima until the codes overwrite them)
hipError_t sq_launch_quantize_tensor(const void* x, int bf16, int64_t count, int8_t* q, float* scale,
                                     hipStream_t st);
// the same codes into 16 x 64 tiles of a [rows][k] matrix
hipError_t sq_launch_quantize_tensor_tiled(const void* x, int bf16, int64_t rows, int64_t k, int8_t* q,
                                           float* scale, hipStream_t st);
// counts s in [2^-100, 2^100) whose kernel reciprocal differs from IEEE 1/s
hipError_t sq_launch_selfcheck_reciprocal(unsigned long long* mismatches, hipStream_t st);
// counts significand pairs (divisors [b_begin, b_end)) where the kernels'
// quotient differs from IEEE a / b
hipError_t sq_launch_selfcheck_division(unsigned b_begin, unsigned b_end, unsigned long long* mismatches,
                                        hipStream_t st);
// out_kind: 0 fp32, 1 bf16, 2 int32; bias_kind: 0 none, 1 fp32, 2 bf16;
// scalar_scales: sx and sw are single values (per-tensor) instead of [m], [n]
hipError_t sq_launch_gemm(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                          const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                          void* y, int out_kind, int scalar_scales, hipStream_t st);
// 16 x 64 tiled int8 (rows in groups of 16, K in 64-byte chunks, tile (g, c)
// at (g * K64 / 64 + c) * 1 KiB, each tile row-major, K64 = k rounded up to
// 64, padding columns zero): the quantisers writing codes in that layout,
// and the product reading both operands in it
hipError_t sq_launch_quantize_act_tiled(const void* x, int bf16, const float* s, int64_t m, int64_t k, int8_t* xq,
                                        float* x_scale, hipStream_t st);
hipError_t sq_launch_quantize_weight_tiled(const void* w, int bf16, const float* s, int64_t n, int64_t k, int8_t* wq,
                                           float* w_scale, hipStream_t st);
hipError_t sq_launch_gemm_tiled(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                int scalar_scales, hipStream_t st);
// the reference linear of quantization_error: x [m][k] times w [n][k]
// (both bf16, or both fp32), fp32 sums, plus bias; out_kind 0 fp32, 1 bf16
hipError_t sq_launch_reference_gemm(const void* x, const void* w, int bf16, int64_t m, int64_t n, int64_t k,
                                    const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st);
// relative Frobenius error of y_q against y_fp ([count] fp32 each, 16-byte
// aligned): sq_relative_error_blocks(count) pairs of binary64 partial sums
// in partial, then out[0] = ||y_fp - y_q||, out[1] = ||y_fp||, out[2] the
// ratio (denominator floored at 1e-12)
int sq_relative_error_blocks(int64_t count);
hipError_t sq_launch_relative_error(const float* y_fp, const float* y_q, int64_t count, double* partial,
                                    double* out, hipStream_t st);
// tokens up to which the product streams the weights instead of running on
// MFMA tiles
constexpr int64_t kStreamMaxM = 64;
// weight-only int8 linear: bf16 x [m][k] times int8 wq [n][k] with fp32
// scales sw [n]; out_kind 0 fp32, 1 bf16; bias_kind as above
hipError_t sq_launch_wo_linear(const void* x, int64_t m, int64_t k, const int8_t* wq, const float* sw, int64_t n,
                               const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st);
// the same with w_q in 16 x 64 tiles
hipError_t sq_launch_wo_linear_tiled(const void* x, int64_t m, int64_t k, const int8_t* wq, const float* sw,
                                     int64_t n, const void* bias, int bias_kind, void* y, int out_kind,
                                     hipStream_t st);
// the W8A8 product for m <= kStreamMaxM on row-major operands through the
// weight-only kernel's stream
hipError_t sq_launch_gemm_stream(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                 int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                 int scalar_scales, hipStream_t st);
// the W8A8 product for m <= kStreamMaxM on operands in 16 x 64 tiles (the
// weight stream of the weight-only kernel, int8 activation codes)
hipError_t sq_launch_gemm_stream_tiled(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                                       const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                                       void* y, int out_kind, int scalar_scales, hipStream_t st);
// y [m][n] fp32 = a [m][kbytes/2] (bf16) times b [n][ldb/2] (bf16) summed
// over kbytes/2 terms with b's columns repeating every ldb/2 (kbytes and ldb
// multiples of 64 bytes, kbytes a multiple of ldb)
hipError_t sq_launch_gemm_bf16_periodic(const void* a, const void* b, int64_t m, int64_t n, int64_t kbytes,
                                        int64_t ldb, float* y, hipStream_t st);
// the same with the contraction split in two halves, one launch: y[h] =
// a[h] b[h], a[h] at h * m * kbytes bytes, b[h] at h * n * ldb bytes, y[h]
// at h * m * n floats
hipError_t sq_launch_gemm_bf16_periodic_split2(const void* a, const void* b, int64_t m, int64_t n, int64_t kbytes,
                                               int64_t ldb, float* y, hipStream_t st);

// The straight-through backward (learnable alpha): workspace regions (byte
// offsets, 256-aligned) for m tokens, n output channels, k input channels.
struct SteLayout {
    int64_t m64, n64;          // m, n rounded up to 64 (the packed contraction)
    int64_t gx, gw, gb;        // row groups of the three column-sum passes
    size_t a1, bw, a2, bx;     // packed factors and transposed codes (bf16)
    size_t px, pw, pb, term;   // binary64 partial sums and per-channel terms
    bool split;                // gX's contraction split in two halves (one launch)
    int64_t nh;                // n64 / 2 when split, else n64
    size_t gxh;                // the two halves of gX, fp32 [2][m][k] (split only)
    size_t bytes;              // total
};
SteLayout sq_ste_layout(int64_t m, int64_t n, int64_t k);
// dx [m][k], dw [n][k] (fp32; also the products' outputs), db [n] (or
// NULL), ds [k] (or NULL), dalpha_deta [2]; mx NULL: no alpha gradient
hipError_t sq_launch_ste_backward(const void* dy, int dy_bf16, int64_t m, int64_t n, int64_t k, const void* x,
                                  int x_bf16, const void* w, int w_bf16, const float* s, const int8_t* xq,
                                  const float* sx, const int8_t* wq, const float* sw, const float* mx,
                                  const float* mw, double alpha, float* dx, float* dw, float* db, float* ds,
                                  double* dalpha_deta, void* workspace, hipStream_t st);
// dy_q = 2 (y_q - y_fp) / max(||y_fp||^2, 1e-24) and the loss ||y_fp -
// y_q||^2 / that; partial: sq_relative_error_blocks(count) pairs, norms [3]
hipError_t sq_launch_aux_loss_grad(const float* y_fp, const float* y_q, int64_t count, double* partial,
                                   double* norms, float* dy_q, double* loss, hipStream_t st);
// the W8A8 linear for m <= kStreamMaxM in one launch: the weight stream
// quantises the activations itself (codes to xq in 16 x 64 tiles, scales
// to sx) before multiplying them; sync: sq_stream_fused_sync_bytes() bytes
// of the caller's workspace, zero before the first call; wait_polls bounds
// each workgroup's wait for the other workgroups' tokens
hipError_t sq_launch_linear_stream_fused(const void* x, int bf16, const float* s, int64_t m, int64_t k,
                                         int8_t* xq, float* sx, const int8_t* wq, const float* sw, int64_t n,
                                         const void* bias, int bias_kind, void* y, int out_kind, void* sync,
                                         int wait_polls, hipStream_t st);
size_t sq_stream_fused_sync_bytes();
