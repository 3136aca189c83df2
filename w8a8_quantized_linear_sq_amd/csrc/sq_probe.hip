// sq_probe.hip -- measurement probe, not part of the library's ABI: the
// rate the int8 matrix units of this part sustain with no memory work at
// all, the ceiling any int8 product of the same size can reach here. Built
// into its own shared library (libsq_probe.so), loaded only by the
// benchmark's reference mode.
//
// The kernel issues exactly the matrix instructions of the int8 product's
// 256 x 256 tiles (gemm_kernel in sq_gemm.hip) for an m x n x k product:
// one workgroup of 8 wavefronts per output tile, wavefronts in a 2 x 4 grid
// of 128 x 64 blocks, per 64-byte K step 16 v_mfma_i32_32x32x32_i8 per
// wavefront (8 accumulator tiles x 2 k slices). Its operands are bytes of
// the tile's own int8 rows, loaded into registers once and reused every
// step (so their bit patterns, and the power they draw, are those of real
// codes); nothing else touches memory until the end. Each
// workgroup reads the shader clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around its loop (barrier to barrier), so
// the clock the chip held under this load follows from the two, and from
// the second when workgroups started and ended, within a launch and
// between two launches in a row.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;

// Both counters, read after every outstanding memory operation of the
// wavefront has completed (the asm's memory clobber also keeps the compiler
// from moving loads or stores across it); the block waits for its own
// counter reads before it ends.
__device__ __forceinline__ void read_clocks(uint64_t& cycles, uint64_t& ticks) {
    asm volatile(
        "s_waitcnt vmcnt(0) lgkmcnt(0)\n\t"
        "s_memtime %0\n\t"
        "s_memrealtime %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=s"(cycles), "=s"(ticks)
        :
        : "memory");
}

__global__ __launch_bounds__(512) void mfma_ceiling_kernel(const int8_t* __restrict__ xq,
                                                           const int8_t* __restrict__ wq, int64_t k,
                                                           int tiles_n, int steps, int* __restrict__ sink,
                                                           uint64_t* __restrict__ clocks) {
    uint64_t entry;  // 100 MHz counter as the wavefront starts
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(entry) : : "memory");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int wm = wave >> 2, wn = wave & 3;

    // fragments of k slices 0 and 1: 16 code bytes per lane, each
    // instruction one contiguous KiB of the tile's rows (the bytes of 16
    // rows' first 64 columns in row-major codes), so the few loads before
    // the loop cost little
    i32x4 a[2][4], b[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = tm * kTile + wm * 128 + i * 32 + 16 * s + (lane >> 2);
            a[s][i] = *(const i32x4*)(xq + (int64_t)row * k + 16 * (lane & 3));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = tn * kTile + wn * 64 + j * 32 + 16 * s + (lane >> 2);
            b[s][j] = *(const i32x4*)(wq + (int64_t)row * k + 16 * (lane & 3));
        }
    }
    i32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = i32x16{};
    // an empty asm that uses every fragment: the loads complete before it,
    // and the (volatile) clock read stays after it
#pragma unroll
    for (int s = 0; s < 2; ++s)
        asm volatile("" ::"v"(a[s][0]), "v"(a[s][1]), "v"(a[s][2]), "v"(a[s][3]), "v"(b[s][0]), "v"(b[s][1]));
    uint64_t c0, r0, c1, r1;
    __syncthreads();  // the workgroup's loop starts when its last wavefront has its operands
    read_clocks(c0, r0);
    for (int st = 0; st < steps; ++st) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
    }
    // the last results must be complete before the clocks are read
    int fold = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) fold ^= acc[i][j][e];
    sink[(int64_t)blockIdx.x * 512 + threadIdx.x] = fold;
    // the two wavefronts that share a SIMD need not progress evenly (one may
    // finish its whole loop first), so the loop ends when the last one does
    __syncthreads();
    read_clocks(c1, r1);
    if (threadIdx.x == 0) {
        clocks[5 * blockIdx.x] = c1 - c0;
        clocks[5 * blockIdx.x + 1] = r1 - r0;
        clocks[5 * blockIdx.x + 2] = entry;
        clocks[5 * blockIdx.x + 3] = r0;
        clocks[5 * blockIdx.x + 4] = r1;
    }
}

}  // namespace

// m x n x k int8 product's matrix instructions with no memory work (see
// above). xq: m x k and wq: n x k row-major int8 codes on the device (only
// their first 64 bytes of each row are read); m and n multiples of 256, k a
// multiple of 64, both at least 64. sink: (m / 256) (n / 256) 512 int32 on
// the device (the folded accumulators, kept so the work is not dropped).
// clocks: 5 (m / 256) (n / 256) uint64 on the device: per workgroup the
// shader cycles and the 100 MHz ticks of its loop, then the 100 MHz counter
// as its first wavefront starts, at the loop's start and at its end (its
// last store complete). stream: a hipStream_t or
// null. Returns 0, or -1 for a shape outside these limits, or the HIP error
// of the launch.
extern "C" int sqp_mfma_ceiling(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k, int* sink,
                                uint64_t* clocks, void* stream) {
    if (m < kTile || n < kTile || k < 64 || m % kTile || n % kTile || k % 64) return -1;
    const int64_t tiles = (m / kTile) * (n / kTile);
    if (tiles > (1 << 20) || k / 64 > (1 << 24)) return -1;
    const int tiles_n = (int)(n / kTile);
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)tiles), dim3(512), 0, (hipStream_t)stream, xq, wq, k,
                       tiles_n, (int)(k / 64), sink, clocks);
    return (int)hipGetLastError();
}
