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
//   * one workgroup per BM x BN output tile; its wavefronts form a WGM x WGN
//     grid and each owns a (BM/WGM) x (BN/WGN) block held in registers as
//     32 x 32 tiles of v_mfma_i32_32x32x32_i8 (the 16x16x64 int8 form
//     measures at half the rate on this chip);
//   * K advances in BK = 64-byte steps through a ring of 4 LDS stages filled
//     by direct-to-LDS loads (buffer_load_dwordx4 ... lds: no VGPR staging,
//     no LDS store instructions), issued three steps ahead. On gfx950 a
//     SIMD that issues vector-memory loads loses MFMA cycles to them; the
//     buffer form (a descriptor in scalar registers, one 32-bit offset per
//     lane) costs the MFMA stream fewer of them than the global form (a
//     64-bit address per lane): 58.6 against 62.2 us at 4096^3, the same
//     bits;
//   * a DMA load writes 64 lanes x 16 bytes contiguously, so the LDS rows
//     (64 bytes) cannot be padded; instead chunk c of row r is stored at
//     position c ^ swz(r), swz(r) = (r >> 2) & 3, under which the 16-byte
//     operand reads of a wavefront (32 rows x 2 chunks) measure free of LDS
//     bank conflicts on gfx950;
//   * the 256 x 256 and 128 x 256 tiles run 8 wavefronts, two per SIMD
//     (waves w and w + 4 share one), in ping-pong: the two groups of four
//     alternate between a run of 16 (8) MFMAs on fragments already in
//     registers and the memory work of their next step (LDS fragment reads,
//     their share of a later stage's DMA, the waits), with a workgroup
//     barrier between phases. Interleaving the memory instructions into the
//     MFMA stream of the same wavefronts measured slower;
//   * the 128 x 128 tile (4 wavefronts, one per SIMD) interleaves instead:
//     one barrier per step between the two 32-byte k slices, the next
//     slice's fragments read right after each slice's first MFMA;
//   * rows past m or n are clamped for loading (their results are never
//     stored); a last partial K step goes through registers, zero-filled;
//   * the 1-D grid is remapped so that the tiles dispatched to one XCD (the
//     hardware deals workgroups round-robin over the 8 XCDs) form a compact
//     block sharing A rows and B columns in that XCD's L2;
//   * the epilogue stages each 32-row slab through LDS and writes whole
//     16-byte row chunks with streaming (non-temporal) stores, each slab's
//     row scales loaded one slab ahead;
//   * the same kernel, with the operands' element type as a parameter (K
//     counted in bytes, so the LDS layout and the DMA are unchanged), is the
//     full-precision reference of quantization_error (page
//     "w8a8_smoothquant.py", SmoothQuantW8A8.quantization_error: the plain
//     linear layer on the unquantised operands): bf16 operands on
//     v_mfma_f32_32x32x16_bf16, whose 16-byte fragment is 8 bf16 at k offset
//     8 (l / 32), the int8 fragment's bytes; fp32 operands on four
//     v_mfma_f32_32x32x2_f32 per fragment, the e-th taking element e of
//     every lane's four (the same k permutation in both operands); fp32
//     sums, the bias added in the epilogue, no scales.
//
// Measured at M = N = K = 4096 (bf16 out): the clock under this load is
// power-limited to about 1.7 GHz (int8 MFMA at 32 busy cycles per
// instruction per SIMD); HBM traffic is the per-XCD minimum of the tile
// order.
#include "sq_device.h"

#include <type_traits>

using namespace sq;

namespace {

constexpr int kBK = 64;            // bytes of K per step
constexpr int kStagesPingPong = 4;  // LDS ring depth, 8-wavefront tiles
constexpr int kStagesInterleaved = 4;  // LDS ring depth, 4-wavefront tile
constexpr int kRowLanes = kBK / 16;        // lanes of one DMA load per row
constexpr int kBlockRows = 64 / kRowLanes; // rows per 1 KiB DMA load
constexpr int kXcds = 8;
constexpr int kSlices = kBK / 32;  // 32-byte k slices per step (one MFMA depth each)

// Scheduling-group masks (instruction classes) of sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector memory
// operations are outstanding (vmcnt_imm), and in addition every LDS
// operation has completed (vm_lgkm_imm).
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int vm_lgkm_imm(int n) { return vmcnt_imm(n) & ~(15 << 8); }

// V global loads spread evenly between MFMAs I .. MF-1.
template <int I, int MF, int V>
__device__ __forceinline__ void sched_spread() {
    constexpr int n = MF - 1;
    constexpr int v = I * V / n - (I - 1) * V / n;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, v, 0);
    if constexpr (I + 1 < MF) sched_spread<I + 1, MF, V>();
}
// Order of one k slice: its first MFMA, then all R LDS reads of the next
// slice's fragments (as early as possible: they have the rest of the slice
// to land), then the remaining MFMAs with V global loads spread between them.
template <int MF, int R, int V>
__device__ __forceinline__ void sched_slice() {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
    sched_spread<1, MF, V>();
}

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// Word 3 of a raw buffer descriptor (gfx9 layout): a non-zero data format
// (32-bit), stride 0, so offsets are plain bytes checked against the record
// count.
constexpr int kBufferFlags = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One direct-to-LDS load of 16 bytes per lane: lane i reads byte voff (its
// own) of the `bytes`-long record at base (uniform) and writes LDS at dst +
// 16 i. The descriptor lives in scalar registers. (Kept out of the kernel
// templates: built inside them, the descriptor type makes the host pass
// drop the kernels' launch stubs.)
__device__ __forceinline__ void dma_load16(const int8_t* base, int bytes, int voff, lds_ptr_t dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferFlags),
                                             dst, 16, voff, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// operand element types: int8 codes, or the reference's bf16 / fp32
constexpr int kI8 = 0, kBf16 = 1, kF32 = 2;

// MFMA 32x32x32 i8 operand: lane l holds 16 k-consecutive bytes of row
// (l % 32) at k offset 16 * (l / 32) of a 32-wide k slice; A and B use the
// same mapping, so the hardware's pairing of bytes is the same for both.
// Result: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l % 32.

// ET: operand element type (kI8: the int8 product with the dequantisation;
// kBf16 / kF32: the reference linear). k is the row length in bytes.
// TILED: both operands in 16 x 64 tiles (rows in groups of 16, K in 64-byte
// chunks, tile (g, c) at (g * k / 64 + c) * 1 KiB, each tile row-major; k is
// then the padded row length, a multiple of 64, and the padding is zero):
// every DMA load reads one whole tile, 1 KiB contiguous.
// BPER (row-major only): B's rows are ldb bytes long (a multiple of 64) and
// repeat along k, so B's byte at k offset c is the one at c mod ldb: one
// product sums several A planes against the same B (the straight-through
// backward splits an fp32 operand into three bf16 planes side by side).
// NSPLIT (BPER, fp32 out): gridDim.y independent products of the same shape
// in one launch, product h with A at h * m * k bytes, B at h * n * ldb bytes
// and Y at h * m * n floats (the halves of a contraction split in two).
template <int ET, int BM, int BN, int WGM, int WGN, int OUT, bool TILED, bool BPER = false, int NSPLIT = 1>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int m, int n, int k,
    const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
    int bias_kind, void* __restrict__ Y, int grid_m, int grid_n, int scalar_scales, int ldb) {
    static_assert(!(BPER && TILED), "a periodic B is row-major");
    static_assert(NSPLIT == 1 || (BPER && OUT == 0), "split products: periodic B, fp32 out");
    if constexpr (NSPLIT > 1) {
        const int64_t h = blockIdx.y;
        A += h * m * k;
        B += h * n * ldb;
        Y = (float*)Y + h * m * n;
    }
    constexpr int NW = WGM * WGN;                 // wavefronts (WGM x WGN grid)
    constexpr int kStages = NW == 8 ? kStagesPingPong : kStagesInterleaved;
    static_assert(kStages >= 3 && kStages <= 5, "the prologue's wait covers up to three later stages");
    constexpr int WM = BM / WGM, WN = BN / WGN;   // per-wavefront block
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int STAGE = (BM + BN) * kBK;          // bytes of one LDS stage (A rows, then B rows)
    constexpr int BLOCKS = (BM + BN) / kBlockRows;  // 1 KiB DMA blocks per stage
    constexpr int LOADS = BLOCKS / NW;              // DMA loads per thread per stage
    static_assert(BLOCKS % NW == 0, "stage must split evenly over the wavefronts");
    __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS addresses
    const int wm = wave / WGN, wn = wave % WGN;

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

    // ---- DMA mapping: wave w fills blocks w, w + 4, ...; lane i of a block
    // ---- writes LDS granule i = (row i / 4, position i % 4) and reads the
    // ---- global chunk that position holds.
    // ---- The loads are buffer loads (a descriptor in scalar registers over
    // ---- the block's 16 rows, one 32-bit offset per lane): on gfx950 they
    // ---- cost the MFMA stream of their SIMD far fewer cycles than global
    // ---- loads with a 64-bit address per lane.
    const int8_t* src[LOADS];   // per-lane address (the partial-step tail)
    const int8_t* gbase[LOADS]; // the block's first byte (uniform)
    int voff[LOADS];
    int dst[LOADS];
    bool per[LOADS];            // BPER: the block holds B rows (offsets wrap at ldb)
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int blk = wave + NW * q;
        const bool in_a = blk * kBlockRows < BM;              // the block's 16 rows are all A or all B
        const int row = blk * kBlockRows + lane / kRowLanes;  // row in the A|B stage space
        const int pos = lane % kRowLanes;
        const int chunk = pos ^ swz(row);
        const int8_t* g;  // first byte of the block's 16 rows (uniform)
        if constexpr (TILED) {
            // the block's 16 rows are one row group; groups past the last
            // (tiles past m or n) read the last one, never stored
            if (in_a) g = A + (int64_t)min((m0 >> 4) + blk, (m - 1) >> 4) * k * 16;
            else g = B + (int64_t)min((n0 >> 4) + blk - BM / kBlockRows, (n - 1) >> 4) * k * 16;
            voff[q] = (lane / kRowLanes) * kBK + chunk * 16;
        } else {
            // rows past m or n are clamped to the last one (never stored);
            // every lane's row is at or after the block's clamped first row
            const int r0 = in_a ? min(m0 + blk * kBlockRows, m - 1) : min(n0 + blk * kBlockRows - BM, n - 1);
            const int r = in_a ? min(m0 + row, m - 1) : min(n0 + row - BM, n - 1);
            const int ld = (BPER && !in_a) ? ldb : k;
            g = (in_a ? A : B) + (int64_t)r0 * ld;
            voff[q] = (r - r0) * ld + chunk * 16;
        }
        per[q] = BPER && !in_a;
        src[q] = g + voff[q];
        gbase[q] = g;
        dst[q] = blk * 1024;
    }
    auto issue_stage = [&](int kt, int buf) {
        const int kb = TILED ? kt * 1024 : kt * kBK;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            if constexpr (BPER) {
                // 16 rows of ldb bytes for a B block, the offset wrapped
                const int kq = per[q] ? kb % ldb : kb;
                dma_load16(gbase[q], 16 * (per[q] ? ldb : k), voff[q] + kq, (lds_ptr_t)(smem + buf * STAGE + dst[q]));
            } else {
                // 16 rows of k bytes from the block's first byte: every offset
                // a stage adds stays below that record count
                dma_load16(gbase[q], 16 * k, voff[q] + kb, (lds_ptr_t)(smem + buf * STAGE + dst[q]));
            }
        }
    };
    // a last partial step: the same layout through registers, chunks past k
    // zero-filled
    auto tail_stage = [&](int kt, int buf) {
        const int kb = kt * kBK;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int row = (wave + NW * q) * kBlockRows + lane / kRowLanes;
            const int chunk = (lane % kRowLanes) ^ swz(row);
            i32x4 v = {0, 0, 0, 0};
            if (kb + chunk * 16 < k) v = *(const i32x4*)(src[q] + kb);
            *(i32x4*)(smem + buf * STAGE + dst[q] + lane * 16) = v;
        }
    };

    static_assert(ET == kI8 || OUT != 2, "int32 output is the int8 product's");
    using Acc = std::conditional_t<ET == kI8, i32x16, f32x16>;
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

    // fragment offsets inside a stage: row (.. + fr), k chunk 2 s + lane / 32
    const int fr = lane & 31;
    int foff[kSlices];
#pragma unroll
    for (int s = 0; s < kSlices; ++s) foff[s] = fr * kBK + (((2 * s + (lane >> 5)) ^ swz(fr)) * 16);

    static_assert(kSlices == 2, "the loops below are written for two k slices per step");

    i32x4 fa[TM], fb[TN], ga[TM], gb[TN];  // fragments of slice 0 / slice 1
    auto read_frags = [&](int buf, int s, i32x4 (&xa)[TM], i32x4 (&xb)[TN]) {
        const int8_t* as = smem + buf * STAGE + (wm * WM) * kBK + foff[s];
        const int8_t* bs = smem + buf * STAGE + (BM + wn * WN) * kBK + foff[s];
#pragma unroll
        for (int i = 0; i < TM; ++i) xa[i] = *(const i32x4*)(as + i * 32 * kBK);
#pragma unroll
        for (int j = 0; j < TN; ++j) xb[j] = *(const i32x4*)(bs + j * 32 * kBK);
    };
    auto mfmas = [&](const i32x4 (&xa)[TM], const i32x4 (&xb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (ET == kI8) {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[i], xb[j], acc[i][j], 0, 0, 0);
                } else if constexpr (ET == kBf16) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[i]),
                                                                        __builtin_bit_cast(bf16x8, xb[j]),
                                                                        acc[i][j], 0, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(xa[i][e]),
                                                                         __int_as_float(xb[j][e]), acc[i][j], 0, 0, 0);
                }
            }
    };
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int MF = TM * TN, R = TM + TN;

    const int KF = k / kBK;  // whole steps
    // The epilogue's kernel arguments arrive by scalar loads; scalar loads
    // share the LDS wait counter and may return out of order, so while one
    // is outstanding every LDS wait in the loop would have to drain all LDS
    // reads. Consume them here, before the loop.
    asm volatile("" ::"s"(sa), "s"(sb), "s"(bias), "s"(Y), "s"(bias_kind), "s"(scalar_scales));
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        if (st < KF) issue_stage(st, st);
    if (KF > 0) {
        // stage 0 landed (the later ones issued may be in flight), visible
        // to all
        const int later = min(KF, kStages - 1) - 1;
        if (later >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LOADS));
        else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        barrier();
    }

    if constexpr (NW == 8) {
        // ---- ping-pong: waves w and w + 4 share a SIMD. Group 0 (waves
        // ---- 0-3) and group 1 (waves 4-7) take turns, one phase each,
        // ---- separated by workgroup barriers: while one group issues an
        // ---- uninterrupted run of MFMAs on fragments already in registers,
        // ---- the other reads its next fragments from LDS and issues its
        // ---- share of the DMA of a later stage, so on every SIMD the matrix
        // ---- unit is fed by one wave while the other does the memory work.
        //   group 0: M(0) C(0) M(1) C(1) ... M(KF-1) C(KF-1) | extra barrier
        //   group 1: barrier | M(0) C(0) ... M(KF-1) C(KF-1)
        // M(kt): read both slices of stage kt; issue this wave's loads of
        //        stage kt+3 into the buffer of stage kt-1 (whose last reads,
        //        by group 1 in the previous phase, completed before that
        //        phase's barrier); wait for own LDS reads and own loads of
        //        stage kt+1, which the next M phase (by either group) reads.
        // C(kt): the MFMAs of both slices.
        const bool second = wave >= NW / 2;
        // the wavefront in its MFMA phase runs at raised priority, so that the
        // SIMD's arbiter serves it first whenever both wavefronts are ready
        // (measured 1-3% faster)
        auto mfma_phase = [&] {
            __builtin_amdgcn_s_setprio(1);
            mfmas(fa, fb);
            mfmas(ga, gb);
            __builtin_amdgcn_s_setprio(0);
        };
        if (second) barrier();
        int kt = 0;
        for (; kt + kStages - 1 < KF; ++kt) {
            const int buf = kt % kStages;
            read_frags(buf, 0, fa, fb);
            read_frags(buf, 1, ga, gb);
            issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
            __builtin_amdgcn_s_waitcnt(vm_lgkm_imm((kStages - 2) * LOADS));
            barrier();
            mfma_phase();
            barrier();
        }
        for (; kt < KF; ++kt) {
            const int buf = kt % kStages;
            read_frags(buf, 0, fa, fb);
            read_frags(buf, 1, ga, gb);
            __builtin_amdgcn_s_waitcnt(vm_lgkm_imm(0));
            barrier();
            mfma_phase();
            barrier();
        }
        if (!second) barrier();
    } else {
        // ---- interleaved (one wave per SIMD): step kt, with the slice-0
        // ---- fragments of stage kt in registers:
        //   phase 1: MFMAs of slice 0, while slice 1 of stage kt is read;
        //   barrier: stage kt+1 is complete and visible, and every wavefront
        //            has finished reading stage kt-1's buffer;
        //   phase 2: MFMAs of slice 1, while slice 0 of stage kt+1 is read
        //            and the DMA of stage kt+3 into stage kt-1's buffer is
        //            issued.
        auto wait_barrier = [&](int n_later_stages) {
            if (n_later_stages >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS));
            else if (n_later_stages == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            barrier();
        };
        if (KF > 0) read_frags(0, 0, fa, fb);
        int kt = 0;
        for (; kt + kStages - 1 < KF; ++kt) {
            const int buf = kt % kStages;
            read_frags(buf, 1, ga, gb);
            mfmas(fa, fb);
            sched_slice<MF, R, 0>();
            wait_barrier(1);
            read_frags((kt + 1) % kStages, 0, fa, fb);
            issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
            mfmas(ga, gb);
            sched_slice<MF, R, LOADS>();
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; kt < KF; ++kt) {
            const int buf = kt % kStages;
            read_frags(buf, 1, ga, gb);
            mfmas(fa, fb);
            if (kt + 1 < KF) {
                wait_barrier(KF - 2 - kt);
                read_frags((kt + 1) % kStages, 0, fa, fb);
            }
            mfmas(ga, gb);
        }
    }
    if (!TILED && !BPER && k % kBK) {
        // a last partial step through registers: its buffer was last read
        // kStages steps ago
        __syncthreads();
        tail_stage(KF, KF % kStages);
        __syncthreads();
        read_frags(KF % kStages, 0, fa, fb);
        read_frags(KF % kStages, 1, ga, gb);
        mfmas(fa, fb);
        mfmas(ga, gb);
    }

    // ---- epilogue ---------------------------------------------------------
    // y = f32(acc) * sa[row] * sb[col] (+ bias[col]) in the MFMA layout, then
    // (whole tiles) staged per 32-row slab through this wavefront's own LDS
    // region and written as 16-byte row chunks.
    const int ecol = lane & 31;
    const int erow = (lane >> 5) * 4;
    float swc[TN], bc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = min(n0 + wn * WN + j * 32 + ecol, n - 1);
        swc[j] = 0.0f;
        bc[j] = 0.0f;
        if constexpr (OUT != 2) {
            if constexpr (ET == kI8) swc[j] = sb[scalar_scales ? 0 : col];
            if (bias_kind == 1) bc[j] = ((const float*)bias)[col];
            else if (bias_kind == 2) bc[j] = __uint_as_float((uint32_t)((const uint16_t*)bias)[col] << 16);
        }
    }
    auto value = [&](int i, int j, int r, float sar) -> float {
        float y;
        if constexpr (ET == kI8) y = (float)acc[i][j][r] * sar * swc[j];
        else y = acc[i][j][r];
        if (bias_kind) y = y + bc[j];
        return y;
    };
    constexpr int OB = OUT == 1 ? 2 : 4;            // output bytes per element
    constexpr int PITCH = WN * OB + 32;             // staged row, bytes (bank-spread)
    constexpr int ROW_CHUNKS = WN * OB / 16;        // 16-byte chunks per staged row
    constexpr int SLAB_CHUNKS = 32 * ROW_CHUNKS;
    static_assert(NW * 32 * PITCH <= (int)sizeof(smem), "epilogue staging exceeds LDS");
    const bool whole = (m0 + BM <= m) && (n0 + BN <= n) && (n % (16 / OB) == 0) &&
                       (scalar_scales || ((uintptr_t)sa & 15) == 0) && (((uintptr_t)Y & 15) == 0);
    if (whole) {
        // The row scales of a slab are loaded one slab ahead: the first
        // slab's before the barrier, the next slab's before this slab's
        // stores. Loaded just before their use, behind the scalar-scale
        // branch, each load was waited for in turn, and on this chip that
        // wait also drains the previous slab's stores (the memory counter
        // counts both).
        float sar_all[TM][4][4] = {};
        auto load_slab = [&](int i) {
            if constexpr (OUT != 2 && ET == kI8) {
                if (scalar_scales) {
                    const float v = sa[0];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sar_all[i][q][e] = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = *(const float4*)(sa + m0 + wm * WM + i * 32 + q * 8 + erow);
                        sar_all[i][q][0] = v.x; sar_all[i][q][1] = v.y; sar_all[i][q][2] = v.z; sar_all[i][q][3] = v.w;
                    }
                }
            }
        };
        load_slab(0);
        __syncthreads();  // every wavefront is done with the operand buffers
        int8_t* stage = smem + wave * 32 * PITCH;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rbase = m0 + wm * WM + i * 32;
            if (i + 1 < TM) load_slab(i + 1);
            const float (&sar)[4][4] = sar_all[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (OUT == 1) {
                    // bf16: lanes 2c and 2c+1 hold columns 2c, 2c+1 of the same
                    // rows; one DPP swap of one value per row pair lets the
                    // even lane write (row r, both columns) and the odd lane
                    // (row r+1, both columns) as one 4-byte store each
                    const bool odd = lane & 1;
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const float a0 = value(i, j, r, sar[r >> 2][r & 3]);
                        const float a1 = value(i, j, r + 1, sar[r >> 2][(r & 3) + 1]);
                        const float send = odd ? a0 : a1;
                        const float recv = __int_as_float(
                            __builtin_amdgcn_update_dpp(0, __float_as_int(send), 0xB1, 0xF, 0xF, false));
                        const float lo = odd ? recv : a0, hi = odd ? a1 : recv;
                        const uint32_t packed = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
                                                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
                        const int lr = (r >> 2) * 8 + erow + (r & 3) + (odd ? 1 : 0);
                        *(uint32_t*)(stage + lr * PITCH + (j * 32 + (ecol & ~1)) * OB) = packed;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lr = (r >> 2) * 8 + erow + (r & 3);
                        int8_t* dst = stage + lr * PITCH + (j * 32 + ecol) * OB;
                        if constexpr (OUT == 2) *(int*)dst = acc[i][j][r];
                        else *(float*)dst = value(i, j, r, sar[r >> 2][r & 3]);
                    }
                }
            }
            // the same wavefront reads back what it wrote: LDS keeps its order.
            // The output is written once and not read here: streaming
            // (non-temporal) stores, measured 1-3% faster over the launch
            // (the tiles all end together, so the output burst is exposed)
#pragma unroll
            for (int c = lane; c < SLAB_CHUNKS; c += 64) {
                const int lr = c / ROW_CHUNKS, cc = c % ROW_CHUNKS;
                const i32x4 v = *(const i32x4*)(stage + lr * PITCH + cc * 16);
                int8_t* out = (int8_t*)Y + ((int64_t)(rbase + lr) * n + n0 + wn * WN) * OB + cc * 16;
                __builtin_nontemporal_store(v, (i32x4*)out);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WN + j * 32 + ecol;
        if (col >= n) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + erow + (r & 3);
                if (row >= m) continue;
                const int64_t off = (int64_t)row * n + col;
                if constexpr (OUT == 2) {
                    ((int*)Y)[off] = acc[i][j][r];
                } else {
                    float sar = 0.0f;
                    if constexpr (ET == kI8) sar = sa[scalar_scales ? 0 : row];
                    const float y = value(i, j, r, sar);
                    if constexpr (OUT == 0) ((float*)Y)[off] = y;
                    else ((__bf16*)Y)[off] = (__bf16)y;
                }
            }
        }
    }
}

template <int ET, bool TILED, int BM, int BN, int WGM, int WGN, bool BPER = false, int NSPLIT = 1>
hipError_t launch_tile(const int8_t* xq, const float* sx, int m, const int8_t* wq, const float* sw,
                       int n, int kbytes, const void* bias, int bias_kind, void* y, int out_kind, int scalar_scales,
                       hipStream_t st, int ldb = 0) {
    const int gm = (m + BM - 1) / BM, gn = (n + BN - 1) / BN;
    dim3 grid(gm * gn, NSPLIT), block(64 * WGM * WGN);
    if (out_kind == 0)
        hipLaunchKernelGGL((gemm_kernel<ET, BM, BN, WGM, WGN, 0, TILED, BPER, NSPLIT>), grid, block, 0, st, xq, wq, m,
                           n, kbytes, sx, sw, bias, bias_kind, y, gm, gn, scalar_scales, ldb);
    else if constexpr (!BPER) {
        if (out_kind == 1)
            hipLaunchKernelGGL((gemm_kernel<ET, BM, BN, WGM, WGN, 1, TILED>), grid, block, 0, st, xq, wq, m, n, kbytes,
                               sx, sw, bias, bias_kind, y, gm, gn, scalar_scales, 0);
        else if constexpr (ET == kI8)
            hipLaunchKernelGGL((gemm_kernel<ET, BM, BN, WGM, WGN, 2, TILED>), grid, block, 0, st, xq, wq, m, n, kbytes,
                               sx, sw, bias, bias_kind, y, gm, gn, scalar_scales, 0);
    }
    return hipGetLastError();
}

// Tile choice: the configuration with the least estimated time, whole waves
// of 256 workgroups (one per CU) times the time of one tile, which is its
// area over the configuration's measured speed per unit area on MI355X
// (256 x 256: 1.0, 128 x 256: 0.80, 128 x 128: 0.73, from full-wave runs of
// the int8 product).
template <int ET, bool TILED = false, bool BPER = false>
hipError_t launch_tiled(const int8_t* a, const float* sx, int64_t m, const int8_t* b, const float* sw, int64_t n,
                        int64_t kbytes, const void* bias, int bias_kind, void* y, int out_kind, int scalar_scales,
                        hipStream_t st, int64_t ldb = 0) {
    struct Cfg { int bm, bn; double speed; };
    const Cfg cfgs[] = {{256, 256, 1.0}, {128, 256, 0.80}, {128, 128, 0.73}};
    int best = 0;
    double best_cost = 0.0;
    for (int i = 0; i < 3; ++i) {
        const int64_t tiles = ((m + cfgs[i].bm - 1) / cfgs[i].bm) * ((n + cfgs[i].bn - 1) / cfgs[i].bn);
        const int64_t waves = (tiles + 255) / 256;
        const double cost = (double)waves * cfgs[i].bm * cfgs[i].bn / cfgs[i].speed;
        if (i == 0 || cost < best_cost) {
            best_cost = cost;
            best = i;
        }
    }
    const int mi = (int)m, ni = (int)n, ki = (int)kbytes, lb = (int)ldb;
    switch (best) {
        case 0: return launch_tile<ET, TILED, 256, 256, 2, 4, BPER>(a, sx, mi, b, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st, lb);
        case 1: return launch_tile<ET, TILED, 128, 256, 2, 4, BPER>(a, sx, mi, b, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st, lb);
        default: return launch_tile<ET, TILED, 128, 128, 2, 2, BPER>(a, sx, mi, b, sw, ni, ki, bias, bias_kind, y, out_kind, scalar_scales, st, lb);
    }
}

}  // namespace

hipError_t sq_launch_gemm(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                          const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                          void* y, int out_kind, int scalar_scales, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    // few tokens: the product streams the weights; the tiled kernel would
    // leave most CUs idle
    if (m <= kStreamMaxM)
        return sq_launch_gemm_stream(xq, sx, m, wq, sw, n, k, bias, bias_kind, y, out_kind, scalar_scales, st);
    return launch_tiled<kI8>(xq, sx, m, wq, sw, n, k, bias, bias_kind, y, out_kind, scalar_scales, st);
}

// both operands in 16 x 64 tiles (k the unpadded row length); few tokens
// take the weight-streaming kernel
hipError_t sq_launch_gemm_tiled(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                int scalar_scales, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    if (m <= kStreamMaxM)
        return sq_launch_gemm_stream_tiled(xq, sx, m, wq, sw, n, k, bias, bias_kind, y, out_kind, scalar_scales, st);
    const int64_t k64 = (k + 63) / 64 * 64;
    return launch_tiled<kI8, true>(xq, sx, m, wq, sw, n, k64, bias, bias_kind, y, out_kind, scalar_scales, st);
}

hipError_t sq_launch_reference_gemm(const void* x, const void* w, int bf16, int64_t m, int64_t n, int64_t k,
                                    const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int8_t* a = (const int8_t*)x;
    const int8_t* b = (const int8_t*)w;
    if (bf16) return launch_tiled<kBf16>(a, nullptr, m, b, nullptr, n, 2 * k, bias, bias_kind, y, out_kind, 0, st);
    return launch_tiled<kF32>(a, nullptr, m, b, nullptr, n, 4 * k, bias, bias_kind, y, out_kind, 0, st);
}

// The straight-through backward's products: y[i][j] = sum_c a[i][c] b[j][c mod
// (ldb / 2)] with bf16 a [m][kbytes / 2] and bf16 b [n][ldb / 2] (kbytes and
// ldb multiples of 64, kbytes a multiple of ldb), fp32 sums, fp32 out.
hipError_t sq_launch_gemm_bf16_periodic(const void* a, const void* b, int64_t m, int64_t n, int64_t kbytes,
                                        int64_t ldb, float* y, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    return launch_tiled<kBf16, false, true>((const int8_t*)a, nullptr, m, (const int8_t*)b, nullptr, n, kbytes,
                                            nullptr, 0, y, 0, 0, st, ldb);
}

// The same product with its contraction split in two halves, both in one
// launch of 256 x 256 tiles (the halves fill the compute units where the
// output alone has too few such tiles): y[h] = a[h] b[h] for h = 0, 1, with
// a[h] [m][kbytes / 2] at h * m * kbytes bytes, b[h] [n][ldb / 2] at
// h * n * ldb bytes and y[h] [m][n] at h * m * n floats.
hipError_t sq_launch_gemm_bf16_periodic_split2(const void* a, const void* b, int64_t m, int64_t n, int64_t kbytes,
                                               int64_t ldb, float* y, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    return launch_tile<kBf16, false, 256, 256, 2, 4, true, 2>((const int8_t*)a, nullptr, (int)m, (const int8_t*)b,
                                                              nullptr, (int)n, (int)kbytes, nullptr, 0, y, 0, 0, st,
                                                              (int)ldb);
}
