// sq_probe.hip -- measurement probes, not part of the library's ABI: the
// rate the int8 matrix units of this part sustain with no memory work at
// all, the ceiling any int8 product of the same size can reach here
// (mfma_ceiling_kernel), and the product's operand stream alone and beside
// those instructions (stream_probe_kernel, below). Built into their own
// shared library (libsq_probe.so), loaded only by the benchmark.
//
// The ceiling kernel issues exactly the matrix instructions of the int8 product's
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

// The product's operand stream, with or without its matrix instructions:
// per 64-byte K step each workgroup brings its tile's 32 KiB of operand
// tiles (16 row groups of A and 16 of B, one 1 KiB tile each, tiled codes)
// into a 4-stage LDS ring with direct-to-LDS buffer loads, three steps
// ahead, 4 loads per wavefront per step, in the product's tile order
// (XCD-compact, groups of 4 along m). With MFMA, each wavefront also runs
// the ceiling kernel's 16 instructions per step on operands held in
// registers. Nothing reads the LDS and there is no barrier inside the loop:
// the two halves of the product's loop, alone and together.
constexpr int kStage = 32768;
constexpr int kXcds = 8;
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3: 32-bit data format, stride 0

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma_load16(const int8_t* base, int bytes, int voff, lds_ptr_t dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferFlags),
                                             dst, 16, voff, 0, 0, 0);
}

// s_waitcnt immediate: at most n vector memory operations outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

template <bool MFMA>
__global__ __launch_bounds__(512, 1) void stream_probe_kernel(const int8_t* __restrict__ A,
                                                              const int8_t* __restrict__ B, int k64, int grid_m,
                                                              int grid_n, int steps, int* __restrict__ sink,
                                                              uint64_t* __restrict__ clocks) {
    __shared__ __attribute__((aligned(1024))) int8_t smem[4 * kStage];
    uint64_t entry;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(entry) : : "memory");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // the product's tile order
    const int total = grid_m * grid_n;
    int pid = blockIdx.x;
    if (total % kXcds == 0) pid = (pid % kXcds) * (total / kXcds) + pid / kXcds;
    const int group_size = 4 * grid_n;
    const int first_m = (pid / group_size) * 4;
    const int gm = min(grid_m - first_m, 4);
    const int tile_m = first_m + (pid % group_size) % gm;
    const int tile_n = (pid % group_size) / gm;

    // wavefront w fills blocks w, w + 8, w + 16, w + 24 of a stage (0-15:
    // A's row groups, 16-31: B's); a block is one row group's tile of the
    // step, 1 KiB contiguous, lane i its bytes 16 i .. 16 i + 15
    const int8_t* g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int blk = wave + 8 * q;
        g[q] = blk < 16 ? A + (int64_t)(tile_m * 16 + blk) * k64 * 16 : B + (int64_t)(tile_n * 16 + blk - 16) * k64 * 16;
    }
    auto issue = [&](int kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dma_load16(g[q], 16 * k64, lane * 16 + kt * 1024,
                       (lds_ptr_t)(smem + (kt & 3) * kStage + (wave + 8 * q) * 1024));
    };

    i32x4 a[2][4], b[2][2];
    i32x16 acc[4][2];
    if constexpr (MFMA) {
        // register operands: bytes of the tile's own first code tiles
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[s][i] = *(const i32x4*)(g[0] + (int64_t)(2 * i + s) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[s][j] = *(const i32x4*)(g[2] + (int64_t)(2 * j + s) * 1024 + lane * 16);
            asm volatile("" ::"v"(a[s][0]), "v"(a[s][1]), "v"(a[s][2]), "v"(a[s][3]), "v"(b[s][0]), "v"(b[s][1]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = i32x16{};
    }
    uint64_t c0, r0, c1, r1;
    __syncthreads();
    read_clocks(c0, r0);
    for (int kt = 0; kt < 3 && kt < steps; ++kt) issue(kt);
    for (int kt = 0; kt < steps; ++kt) {
        // stage kt has landed (the product waits here before its LDS reads)
        if (kt + 2 < steps) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
        else if (kt + 1 < steps) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        if constexpr (MFMA) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
        }
        if (kt + 3 < steps) issue(kt + 3);
    }
    int fold = (int)smem[threadIdx.x * 16];  // a byte of the first stage
    if constexpr (MFMA) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) fold ^= acc[i][j][e];
    }
    sink[(int64_t)blockIdx.x * 512 + threadIdx.x] = fold;
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

// The operand-stream probe (stream_probe_kernel above) for an m x n x k
// product: a and b are m x k and n x k int8 codes on the device in 16 x 64
// tiles (row groups of 16, K in 64-byte chunks, tile (g, c) at
// (g k / 64 + c) KiB); m and n multiples of 256, k a multiple of 64, at
// least 64. mfma: 0 the loads alone, 1 the loads and the matrix
// instructions. sink and clocks as for sqp_mfma_ceiling. Returns 0, -1 for
// a shape outside these limits, or the HIP error of the launch.
extern "C" int sqp_stream_probe(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k, int mfma,
                                int* sink, uint64_t* clocks, void* stream) {
    if (m < kTile || n < kTile || k < 64 || m % kTile || n % kTile || k % 64) return -1;
    const int64_t tiles = (m / kTile) * (n / kTile);
    // a row group's record (16 k bytes) must fit the descriptor's 32-bit count
    if (tiles > (1 << 20) || 16 * k > (int64_t)INT32_MAX) return -1;
    const int gm = (int)(m / kTile), gn = (int)(n / kTile), steps = (int)(k / 64);
    if (mfma)
        hipLaunchKernelGGL(stream_probe_kernel<true>, dim3((unsigned)tiles), dim3(512), 0, (hipStream_t)stream, a, b,
                           (int)k, gm, gn, steps, sink, clocks);
    else
        hipLaunchKernelGGL(stream_probe_kernel<false>, dim3((unsigned)tiles), dim3(512), 0, (hipStream_t)stream, a, b,
                           (int)k, gm, gn, steps, sink, clocks);
    return (int)hipGetLastError();
}

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
