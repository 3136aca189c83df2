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

// round_half_even(v / scale) clamped to [-128, 127], where rs = RN(1/scale).
// RN(v * rs) is within 2^-15.9 of v / scale for |v / scale| <= 127.00002
// (two binary32 roundings of a quotient below 2^7). When that approximation
// lies more than 2^-14 away from every half-integer, the correctly rounded
// quotient lies on the same side of the same half-integers and rounds to
// the same integer; otherwise the exact IEEE quotient decides.
__device__ __forceinline__ float code_of(float v, float scale, float rs) {
    float q = v * rs;
    float c = __builtin_rintf(q);
    float d = q - c;  // exact (Sterbenz)
    if (__builtin_fabsf(d) >= 0.5f - 0x1p-14f) c = __builtin_rintf(v / scale);
    return __builtin_fminf(__builtin_fmaxf(c, -128.0f), 127.0f);
}

// Four codes (already integral floats in [-128, 127]) -> one packed dword.
__device__ __forceinline__ uint32_t pack4(float c0, float c1, float c2, float c3) {
    uint32_t b0 = (uint32_t)(int)c0 & 0xffu, b1 = (uint32_t)(int)c1 & 0xffu;
    uint32_t b2 = (uint32_t)(int)c2 & 0xffu, b3 = (uint32_t)(int)c3 & 0xffu;
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

}  // namespace sq

// ---- launchers (host side), one per kernel family; each returns the
// ---- hipError_t of its launch.
hipError_t sq_launch_fill(float* p, float v, int64_t count, hipStream_t st);
hipError_t sq_launch_colmax(const void* x, int bf16, int64_t rows, int64_t k,
                            float* out_max, hipStream_t st);
hipError_t sq_launch_smooth_factor(const float* x_max, float* io, double a_x, double a_w,
                                   int64_t k, hipStream_t st);
hipError_t sq_launch_quantize_weight(const void* w, int bf16, const float* s, int64_t n,
                                     int64_t k, int8_t* wq, float* w_scale, hipStream_t st);
hipError_t sq_launch_quantize_act(const void* x, int bf16, const float* s, int64_t m, int64_t k,
                                  int8_t* xq, float* x_scale, hipStream_t st);
// out_kind: 0 fp32, 1 bf16, 2 int32; bias_kind: 0 none, 1 fp32, 2 bf16
hipError_t sq_launch_gemm(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                          const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                          void* y, int out_kind, hipStream_t st);
