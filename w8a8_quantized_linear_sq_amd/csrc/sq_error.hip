// sq_error.hip -- quantization_error's measure on the GPU.
//
// Page "w8a8_smoothquant.py" (BiGRU_T_version),
// SmoothQuantW8A8.quantization_error: the Frobenius norm of the difference
// between the full-precision output and the quantized one, over the norm of
// the full-precision output (floored at 1e-12):
//   ratio = ||y_fp - y_q||_F / max(||y_fp||_F, 1e-12)
// The sums of squares are taken in binary64 (the fp32 differences are exact
// in binary64), in two passes with a fixed order, so that a given count
// always gives the same bits:
//   * pass 1: a grid of B blocks (B fixed by the count), each thread summing
//     a grid-stride range of 16-byte groups, then the block in a fixed tree;
//     one pair of partial sums per block in the workspace;
//   * pass 2: one block adds the B pairs in a fixed tree and writes the two
//     norms and the ratio.
// HBM-bound: 8 bytes read per element.
#include "sq_device.h"

using namespace sq;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 1024;
constexpr int kPerThread = 16;  // elements per thread, at least, before more blocks

// Sum of v over the block's threads in a fixed order: the wavefront in a
// fixed butterfly, then the 4 wavefront sums in index order. Every thread
// returns the block's sum.
__device__ double block_sum(double v, double* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double s = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) s += red[w];
    return s;
}

__global__ __launch_bounds__(kThreads) void sqerr_partial_kernel(const float* __restrict__ a,
                                                                 const float* __restrict__ b, int64_t count,
                                                                 double* __restrict__ partial) {
    __shared__ double red[kThreads / 64];
    double d2 = 0.0, f2 = 0.0;
    const int64_t groups = count / 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < groups; i += stride) {
        const float4 va = ((const float4*)a)[i];
        const float4 vb = ((const float4*)b)[i];
        const double e0 = (double)va.x - (double)vb.x, e1 = (double)va.y - (double)vb.y;
        const double e2 = (double)va.z - (double)vb.z, e3 = (double)va.w - (double)vb.w;
        d2 += e0 * e0;
        d2 += e1 * e1;
        d2 += e2 * e2;
        d2 += e3 * e3;
        f2 += (double)va.x * va.x;
        f2 += (double)va.y * va.y;
        f2 += (double)va.z * va.z;
        f2 += (double)va.w * va.w;
    }
    // the last count % 4 elements, one per thread of block 0
    if (blockIdx.x == 0 && threadIdx.x < count - groups * 4) {
        const int64_t i = groups * 4 + threadIdx.x;
        const double e = (double)a[i] - (double)b[i];
        d2 += e * e;
        f2 += (double)a[i] * a[i];
    }
    d2 = block_sum(d2, red);
    f2 = block_sum(f2, red);
    if (threadIdx.x == 0) {
        partial[2 * blockIdx.x] = d2;
        partial[2 * blockIdx.x + 1] = f2;
    }
}

__global__ __launch_bounds__(kThreads) void sqerr_final_kernel(const double* __restrict__ partial, int blocks,
                                                               double* __restrict__ out) {
    __shared__ double red[kThreads / 64];
    double d2 = 0.0, f2 = 0.0;
    // at most kMaxBlocks / kThreads = 4 rounds, unrolled so that their loads
    // are issued together (the adds keep their order)
#pragma unroll 4
    for (int i = threadIdx.x; i < blocks; i += kThreads) {
        d2 += partial[2 * i];
        f2 += partial[2 * i + 1];
    }
    d2 = block_sum(d2, red);
    f2 = block_sum(f2, red);
    if (threadIdx.x == 0) {
        const double num = sqrt(d2), den = sqrt(f2);
        out[0] = num;
        out[1] = den;
        out[2] = num / (den > 1e-12 ? den : 1e-12);
    }
}

}  // namespace

int sq_relative_error_blocks(int64_t count) {
    const int64_t per_block = (int64_t)kThreads * kPerThread;
    int64_t blocks = (count + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    return (int)blocks;
}

hipError_t sq_launch_relative_error(const float* y_fp, const float* y_q, int64_t count, double* partial,
                                    double* out, hipStream_t st) {
    const int blocks = sq_relative_error_blocks(count);
    hipLaunchKernelGGL(sqerr_partial_kernel, dim3(blocks), dim3(kThreads), 0, st, y_fp, y_q, count, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sqerr_final_kernel, dim3(1), dim3(kThreads), 0, st, partial, blocks, out);
    return hipGetLastError();
}
