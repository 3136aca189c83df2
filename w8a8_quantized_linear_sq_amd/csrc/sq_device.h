// sq_device.h -- device helpers and kernel launch declarations shared by the
// HIP translation units of libsq.so (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace sq

// ---- launchers (host side), one per kernel family; each returns the
// ---- hipError_t of its launch.
hipError_t sq_launch_fill(float* p, float v, int64_t count, hipStream_t st);
// running column max of |x| folded into running_max (calibration)
hipError_t sq_launch_colmax(const void* x, int bf16, int64_t rows, int64_t k, float* running_max,
                            hipStream_t st);
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
