// sq_wo.hip -- weight-only int8 linear: bf16 activations times int8 weights
// with one scale per output channel, for few tokens (the decode shape); and
// the same weight stream for the W8A8 product of up to 64 tokens on int8
// codes (row-major or tiled).
//
// Follows the torchao page "quantization/subclass.py",
// Int8WeightOnlyQuantizedLinearWeight._quantized_op: the int8 weights are
// converted to the activations' type (bf16, exactly), multiplied with the
// activations, scaled per output channel, then the bias is added:
//   y[t][o] = f32(sum_j x[t][j] * wq[o][j]) * sw[o] (+ bias[o])   -> out type
// Every bf16 x int8 product is exact in fp32; the sum is accumulated in fp32
// by the matrix units.
//
// Design (gfx950). With few tokens every weight byte is used by one
// workgroup only, so the kernel is a stream over the weights and nothing
// needs staging for reuse:
//   * one workgroup of 8 wavefronts per R weight rows, R = ceil(n / 256)
//     (at most 48, more rounds beyond 256 x 48 rows), so that for the decode
//     shapes every compute unit holds one workgroup and streams the same
//     number of rows: no tail round. R need not be a multiple of 16: the
//     last 16-row group of a workgroup is partly masked;
//   * K is cut into 64-element chunks dealt round-robin to the wavefronts;
//     per chunk a lane loads 16 bytes of its weight row (row l % 16, bytes
//     16 (l / 16) .. +16 of the chunk) straight into registers, 64 bytes
//     contiguous per row and instruction, and the 32 bytes of bf16
//     activations at the same k;
//   * the order of the k sum is free, so the chunk's 16 bytes feed two
//     v_mfma_f32_16x16x32_bf16, bytes 0-7 and 8-15 of every lane, the
//     activations split the same way: each lane's k positions map to the
//     same physical k in both operands;
//   * batches of CB chunks (weights and activations) stream through NB
//     register buffers, no LDS; a batch's activations are loaded before its
//     weights, so the in-order memory counter never holds them behind
//     weights that are not needed yet;
//   * loads past the rows or past K read an address another lane of the
//     same instruction reads (no extra memory traffic), so every load is
//     unconditional and the waits are exact; rows past the workgroup's rows
//     and tokens past m only feed outputs that are not stored, and the
//     activations of pieces past K are zeroed where they are used (a zero
//     times a finite int8 adds nothing);
//   * the 8 partial sums of a 16 x 16 output fragment meet in LDS and are
//     added in wavefront order by one wavefront, which applies the scale and
//     the bias;
//   * TILED: the weights in 16 x 64 tiles (16-row groups, K in 64-byte
//     chunks, tile (g, c) at (g * K64 / 64 + c) * 1 KiB, row-major inside,
//     zero padding columns). A chunk's 16 rows x 64 bytes are then one
//     tile, so each weight load instruction reads 1 KiB contiguously
//     instead of 16 separate 64-byte pieces. A workgroup owns whole groups
//     (the groups spread evenly over the workgroups, G or G - 1 each);
//   * I8: the W8A8 product for few tokens (page "w8a8_smoothquant.py",
//     SmoothQuantW8A8.forward, integer route) on int8 activation codes:
//     per chunk a lane loads 16 code bytes of each token group (tiled: one
//     1 KiB tile per instruction, like the weights; row-major: 16 rows x 64
//     bytes) and one v_mfma_i32_16x16x64_i8 takes the chunk (lane l: row
//     l % 16, bytes 16 (l / 16) .. +16, the tile's own order). The int32
//     sums are exact; the epilogue is the GEMM's, f32(acc) * sx[t] * sw[o]
//     (+ bias[o]), or the raw int32 sums (OUT = 2).
//   * FUSED (I8, TILED): the activation quantisation of the same call runs in
//     this kernel (page "w8a8_smoothquant.py", SmoothQuantW8A8.forward:
//     X / s, per-token int8, then the product). Workgroup b quantises tokens
//     b, b + grid, ... (bit-identical to the row quantiser) into the
//     caller's tiled code buffer, then publishes each with a per-token flag
//     (release at agent scope). Every workgroup issues its first weight
//     loads, then waits (acquire) until every token's flag holds this
//     call's epoch; the wait is bounded, and a workgroup that runs out of
//     polls quantises the missing tokens itself (the same bytes: the race
//     between identical writes is benign), so no workgroup can hang on
//     another. The epoch lives in the caller's workspace next to the
//     flags: every workgroup reads it at its start, and the last workgroup
//     to finish (a done counter) advances it and resets the counter, so
//     successive calls and graph replays see fresh flags.
#include <atomic>
#include <type_traits>

#include "sq_device.h"

using namespace sq;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;    // K elements per chunk
constexpr int kWaves = 8;     // wavefronts per workgroup
constexpr int kMaxRows = 48;  // weight rows per workgroup, at most

// 8 int8 (two dwords) -> 8 bf16, exactly (every int8 is a bf16)
__device__ __forceinline__ bf16x8 widen(uint32_t lo, uint32_t hi) {
    bf16x8 out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t word = i < 4 ? lo : hi;
        const int v = (int)(int8_t)(word >> (8 * (i & 3)));
        out[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint((float)v) >> 16));
    }
    return out;
}

// The fused path's synchronisation words in the caller's workspace (zero
// before the first call): epoch, done counter, one flag per token.
struct FuseSync {
    unsigned long long epoch;
    unsigned long long done;
    unsigned long long fallbacks;  // workgroups that ran out of polls, ever (a statistic)
    unsigned long long pad;
    unsigned long long flag[64];
};

// One token row of the per-token activation quantiser, by the 512 threads
// of a workgroup, bit-identical to the row quantiser's arithmetic (thread t
// owns the 8-channel chunks t, t + 512, ..., at most kProdChunks of them,
// held in registers: the row is read once):
//   x~ = x / s (exact division; the IEEE division where the fast quotient
//   leaves its proven range), scale = max(max |x~|, 1e-8) / 127,
//   codes = round_half_even(x~ / scale) into the 16 x 64 tiles of q (padding
//   columns zero).
constexpr int kProdChunks = 4;  // 512 threads x 4 chunks x 8 = 16384 channels
template <bool BF16>
__device__ void produce_row(const void* x, const float* __restrict__ s, int64_t row, int64_t k, int8_t* q,
                            float* scale_out, float* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t k8 = k >> 3, k64 = (k + 63) & ~(int64_t)63;
    auto in_range = [](float q0) {
        const float a0 = __builtin_fabsf(q0);
        return a0 >= 0x1p-50f && a0 <= 0x1p120f;
    };
    float v[kProdChunks][8], sv[kProdChunks][8];
#pragma unroll
    for (int c = 0; c < kProdChunks; ++c) {
        const int64_t j8 = (int64_t)c * 64 * kWaves + tid;
        if (j8 < k8) {
            load8<BF16>(x, row * k + j8 * 8, v[c]);
            load8<false>(s, j8 * 8, sv[c]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[c][i] = 0.0f;
                sv[c][i] = 1.0f;
            }
        }
    }
    // the quotients; the IEEE division where any of the thread's quotients
    // leaves the fast range (as the row quantiser decides it)
    float xs[kProdChunks][8], yv[kProdChunks][8];
    float qmax = 0.0f;
    bool y_bad = false;
#pragma unroll
    for (int c = 0; c < kProdChunks; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            yv[c][i] = recip_rn(sv[c][i]);
            y_bad |= __builtin_isnan(yv[c][i]);
            xs[c][i] = div_rn(v[c][i], sv[c][i], yv[c][i]);
            qmax = fmaxf(qmax, __builtin_fabsf(v[c][i] * yv[c][i]));
        }
    if (y_bad || !(qmax <= 0x1p120f)) {
#pragma unroll
        for (int c = 0; c < kProdChunks; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q0 = v[c][i] * yv[c][i];
                if (!in_range(q0) && q0 != 0.0f) xs[c][i] = v[c][i] / sv[c][i];
            }
    }
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < kProdChunks; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, __builtin_fabsf(xs[c][i]));
    mx = wave_max_nonneg(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();  // red is reused by the next row
    const float scale = row_scale(fmaxf(mx, kFloor));
    const float rs = row_scale_recip(scale);
#pragma unroll
    for (int c = 0; c < kProdChunks; ++c) {
        const int64_t j8 = (int64_t)c * 64 * kWaves + tid;
        if (j8 >= (k64 >> 3)) continue;
        u32x2 codes = {0u, 0u};
        if (j8 < k8) {
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = __float_as_uint(div_rn(xs[c][i], scale, rs) + kMagic);
            codes = u32x2{pack_low_bytes(b[0], b[1], b[2], b[3]), pack_low_bytes(b[4], b[5], b[6], b[7])};
        }
        *(u32x2*)(q + ((row >> 4) * (k64 >> 6) + (j8 >> 3)) * 1024 + (row & 15) * 64 + (j8 & 7) * 8) = codes;
    }
    if (tid == 0) scale_out[row] = scale;
}

// FUSE: 0 none; 1, 2: the activation quantisation of the call runs here
// (FUSED above) from bf16 (1) or fp32 (2) activations xf with smoothing
// factor sf; X and sa are then the tiled code and scale buffers it fills.
struct FuseArgs {
    const void* xf;
    const float* sf;
    FuseSync* sync;
    int wait_polls;
};

// v_mfma_f32_16x16x32_bf16 operands: lane l holds 8 k-consecutive bf16 of
// row (l % 16) at k offset 8 * (l / 16); result lane l, register r -> row
// 4 * (l / 16) + r (token), column l % 16 (weight row).
template <int TM, int G, int CB, int NB, int OUT, bool TILED, bool I8, int FUSE = 0>
__global__ __launch_bounds__(64 * kWaves) void wo_kernel(const void* X, const int8_t* Bw, int m, int n, int k,
                                                         int rows, const float* __restrict__ sa,
                                                         const float* __restrict__ sb, const void* __restrict__ bias,
                                                         int bias_kind, void* __restrict__ Y, int scalar_scales,
                                                         FuseArgs fa) {
    static_assert(I8 || OUT != 2, "raw int32 sums only for the int8 product");
    static_assert(FUSE == 0 || (I8 && TILED), "the fused quantisation writes tiled int8 codes");
    typedef typename std::conditional<I8, i32x4, f32x4>::type acc_t;
    constexpr int XV = I8 ? 1 : 2;  // 16-byte activation loads per token group and chunk
    __shared__ acc_t red[kWaves][TM * G][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned long long epoch = 0;
    if constexpr (FUSE != 0) {
        // this call's epoch (stable while the kernel runs: only the last
        // workgroup to finish advances it)
        // (the previous call's update is visible: kernels on a stream are
        // ordered)
        epoch = __hip_atomic_load(&fa.sync->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float* fred = (float*)&red[0][0][0];
        for (int tok = blockIdx.x; tok < m; tok += gridDim.x) {
            produce_row<FUSE == 1>(fa.xf, fa.sf, tok, k, (int8_t*)X, (float*)sa, fred);
            // the workgroup's codes are complete (the barrier orders every
            // thread's stores before thread 0's release, which makes them
            // visible to every compute unit before the flag)
            __syncthreads();
            // system scope: the flag is written through to memory, where the
            // other compute units' polls read it (each XCD's L2 would keep
            // serving them a stale copy at agent scope)
            if (threadIdx.x == 0)
                __hip_atomic_store(&fa.sync->flag[tok], epoch + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    const int r16 = lane & 15, grp = lane >> 4;
    const int nchunks = (k + kChunk - 1) / kChunk;
    int row0;
    const int8_t* wrow[G];
    if constexpr (TILED) {
        // groups [g0, g1) of the ceil(n / 16); a group past g1 reads group
        // g1 - 1 (another lane's addresses), never stored
        const int ng = (n + 15) / 16;
        const int g0 = (int)((int64_t)blockIdx.x * ng / gridDim.x);
        const int g1 = (int)((int64_t)(blockIdx.x + 1) * ng / gridDim.x);
        row0 = g0 * 16;
        rows = (g1 - g0) * 16;
#pragma unroll
        for (int g = 0; g < G; ++g)
            wrow[g] = Bw + (int64_t)min(g0 + g, g1 - 1) * nchunks * 1024 + r16 * 64 + grp * 16;
    } else {
        // row pointers: a row past the workgroup's rows reads the last row,
        // a token past m the last token (addresses another lane of the
        // instruction reads); their sums land in outputs that are not stored
        row0 = blockIdx.x * rows;
        const int rend = min(row0 + rows, n);
#pragma unroll
        for (int g = 0; g < G; ++g) wrow[g] = Bw + (int64_t)min(row0 + g * 16 + r16, rend - 1) * k;
    }
    // activation rows: bf16, a token past m reads the last token; int8
    // tiles, the lane's position in token group t's first tile (tokens past
    // m are the group's padding rows, never stored)
    const int8_t* xrow[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        if constexpr (I8 && TILED) xrow[t] = (const int8_t*)X + (int64_t)t * nchunks * 1024 + r16 * 64 + grp * 16;
        else if constexpr (I8) xrow[t] = (const int8_t*)X + (int64_t)min(t * 16 + r16, m - 1) * k;
        else xrow[t] = (const int8_t*)((const uint16_t*)X + (int64_t)min(t * 16 + r16, m - 1) * k);
    }

    // chunks of this wavefront: wave, wave + 8, ...; every wavefront runs
    // the same number of batches; pieces past K read the last 16 elements
    // of the row (tiled weights: the last chunk's tile) and their
    // activations are zeroed where they are used
    const int per_wave = (nchunks + kWaves - 1) / kWaves;
    // batches, padded to a multiple of NB (the loop handles NB at a time; a
    // padding batch holds only pieces past K)
    const int nb = ((per_wave + CB - 1) / CB + NB - 1) / NB * NB;
    auto koff = [&](int b, int j, bool& ok) {
        const int off = (wave + kWaves * (b * CB + j)) * kChunk + grp * 16;
        ok = off < k;  // k is a multiple of 16: a piece is whole or absent
        return ok ? off : k - 16;
    };
    // byte offset of a batch piece in a weight row (tiled: of the chunk's
    // tile from the lane's position in the group's first tile)
    auto woff = [&](int b, int j) {
        if constexpr (TILED) {
            return min(wave + kWaves * (b * CB + j), nchunks - 1) * 1024;
        } else {
            bool ok;
            return koff(b, j, ok);
        }
    };

    // NB register buffers, each with a batch of weights and the matching
    // activations
    struct Batch {
        u32x4 w[G][CB];
        u32x4 x[TM][CB][XV];
    };
    Batch bufs[NB];
    acc_t acc[TM][G];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[t][g] = acc_t{0, 0, 0, 0};

    // activations first: the memory counter is in order, and a batch's
    // activations (cache hits) must not wait behind its weights
    auto load = [&](Batch& buf, int b) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if constexpr (I8) {
                const int off = woff(b, j);
#pragma unroll
                for (int t = 0; t < TM; ++t) buf.x[t][j][0] = *(const u32x4*)(xrow[t] + off);
            } else {
                bool ok;
                const int off = koff(b, j, ok);
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    buf.x[t][j][0] = *(const u32x4*)((const uint16_t*)xrow[t] + off);
                    buf.x[t][j][1] = *(const u32x4*)((const uint16_t*)xrow[t] + off + 8);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const int off = woff(b, j);
#pragma unroll
            for (int g = 0; g < G; ++g) buf.w[g][j] = *(const u32x4*)(wrow[g] + off);
        }
    };
    auto compute = [&](const Batch& buf, int b) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            bool ok;
            koff(b, j, ok);
            if constexpr (I8) {
                i32x4 xa[TM];
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    xa[t] = __builtin_bit_cast(i32x4, ok ? buf.x[t][j][0] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const i32x4 wv = __builtin_bit_cast(i32x4, buf.w[g][j]);
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        acc[t][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[t], wv, acc[t][g], 0, 0, 0);
                }
                continue;
            }
            bf16x8 xa[TM], xb[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                xa[t] = __builtin_bit_cast(bf16x8, ok ? buf.x[t][j][0] : u32x4{0u, 0u, 0u, 0u});
                xb[t] = __builtin_bit_cast(bf16x8, ok ? buf.x[t][j][1] : u32x4{0u, 0u, 0u, 0u});
            }
            if constexpr (!I8) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const bf16x8 wlo = widen(buf.w[g][j][0], buf.w[g][j][1]);
                    const bf16x8 whi = widen(buf.w[g][j][2], buf.w[g][j][3]);
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[t], wlo, acc[t][g], 0, 0, 0);
                        acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[t], whi, acc[t][g], 0, 0, 0);
                    }
                }
            }
        }
    };

    // Every path issues the same loads in the same order and the loop has a
    // single exit, its last pair peeled: a load issued on one path only (or
    // a second exit, which the control-flow structurizer turns into a path
    // that skips the loads) leaves the compiler's wait counts at their most
    // pessimistic. An empty asm with a memory clobber closes every group of
    // loads (X and Bw are not restrict-qualified, so the clobber holds for
    // them; it keeps the prologue's and the loop's loads in their blocks),
    // and a scheduling barrier keeps the compute that follows, register work
    // included, behind them: the scheduler would otherwise place each load
    // just before its use.
    auto fence = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (FUSE != 0) {
        // the first batches' weights stream while the tokens are quantised
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int off = woff(i, j);
#pragma unroll
                for (int g = 0; g < G; ++g) bufs[i].w[g][j] = *(const u32x4*)(wrow[g] + off);
            }
        fence();
        // wavefront 0 waits, bounded, for every token's flag of this epoch
        // (relaxed polls from memory, system scope: an acquire per poll would
        // invalidate the caches the producers work from; one acquire
        // follows the wait)
        __shared__ int missing;
        if (wave == 0) {
            bool ready = false;
            for (int poll = 0;; ++poll) {
                ready = true;
                if (lane < m)
                    ready = __hip_atomic_load(&fa.sync->flag[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
                            epoch + 1;
                if (__builtin_amdgcn_ballot_w64(!ready) == 0 || poll >= fa.wait_polls) break;
                __builtin_amdgcn_s_sleep(2);
            }
            const unsigned long long late = __builtin_amdgcn_ballot_w64(!ready);
            if (lane == 0) missing = late != 0;
        }
        __syncthreads();
        if (missing) {
            // out of polls: quantise every token not yet published here (the
            // same bytes its producer writes) and publish it
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(&fa.sync->fallbacks, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float* fred = (float*)&red[0][0][0];
            __shared__ int done_tok;
            for (int tok = 0; tok < m; ++tok) {
                if (threadIdx.x == 0)
                    done_tok = __hip_atomic_load(&fa.sync->flag[tok], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
                               epoch + 1;
                __syncthreads();
                const int skip = done_tok;
                __syncthreads();
                if (skip) continue;
                produce_row<FUSE == 1>(fa.xf, fa.sf, tok, k, (int8_t*)X, (float*)sa, fred);
                __syncthreads();
                if (threadIdx.x == 0)
                    __hip_atomic_store(&fa.sync->flag[tok], epoch + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
        // acquire the published codes (the flags observed above) before any
        // wavefront reads them
        if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int off = woff(i, j);
#pragma unroll
                for (int t = 0; t < TM; ++t) bufs[i].x[t][j][0] = *(const u32x4*)(xrow[t] + off);
            }
        fence();
    } else {
#pragma unroll
        for (int i = 0; i < NB; ++i) load(bufs[i], i);
        fence();
    }
    int b = 0;
    for (; b + NB < nb; b += NB) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            compute(bufs[i], b + i);
            load(bufs[i], b + i + NB);
            fence();
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) compute(bufs[i], b + i);

    // ---- the wavefronts' partial sums meet in LDS; fragment f = t * G + g
    // ---- is summed in wavefront order by wavefront f % 8
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int g = 0; g < G; ++g) red[wave][t * G + g][lane] = acc[t][g];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < TM * G; ++f) {
        if (f % kWaves != wave) continue;
        const int t = f / G, g = f % G;
        acc_t s = red[0][f][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) s += red[w][f][lane];
        const int o = row0 + g * 16 + r16;
        if (g * 16 + r16 >= rows || o >= n) continue;
        float swo = 0.0f, bo = 0.0f;
        if constexpr (OUT != 2) {
            swo = sb[I8 && scalar_scales ? 0 : o];
            if (bias_kind == 1) bo = ((const float*)bias)[o];
            else if (bias_kind == 2) bo = __uint_as_float((uint32_t)((const uint16_t*)bias)[o] << 16);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = t * 16 + grp * 4 + r;
            if (tok >= m) continue;
            const int64_t off = (int64_t)tok * n + o;
            if constexpr (OUT == 2) {
                ((int*)Y)[off] = s[r];
            } else {
                float y;
                if constexpr (I8) y = (float)s[r] * sa[scalar_scales ? 0 : tok] * swo;
                else y = s[r] * swo;
                if (bias_kind) y = y + bo;
                if constexpr (OUT == 0) ((float*)Y)[off] = y;
                else ((__bf16*)Y)[off] = (__bf16)y;
            }
        }
    }
    if constexpr (FUSE != 0) {
        // the last workgroup to finish advances the epoch (every workgroup
        // has read it by then) and resets the counter for the next call
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned long long prev =
                __hip_atomic_fetch_add(&fa.sync->done, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (prev == gridDim.x - 1) {
                __hip_atomic_store(&fa.sync->done, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&fa.sync->epoch, epoch + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// grid: row-major weights, ceil(n / rows) workgroups of `rows` rows; tiled
// weights, `rows` is the workgroup count (the groups spread over them)
template <int TM, int G, int CB, int NB, bool TILED, bool I8, int FUSE = 0>
hipError_t launch_wo(const void* x, const float* sx, int m, const int8_t* wq, const float* sw, int n, int k,
                     int rows, const void* bias, int bias_kind, void* y, int out_kind, int scalar_scales,
                     hipStream_t st, FuseArgs fa = FuseArgs{}) {
    const dim3 grid(TILED ? rows : (n + rows - 1) / rows), block(64 * kWaves);
    if (out_kind == 0)
        hipLaunchKernelGGL((wo_kernel<TM, G, CB, NB, 0, TILED, I8, FUSE>), grid, block, 0, st, x, wq, m, n, k, rows,
                           sx, sw, bias, bias_kind, y, scalar_scales, fa);
    else if (out_kind == 1)
        hipLaunchKernelGGL((wo_kernel<TM, G, CB, NB, 1, TILED, I8, FUSE>), grid, block, 0, st, x, wq, m, n, k, rows,
                           sx, sw, bias, bias_kind, y, scalar_scales, fa);
    else if constexpr (I8)
        hipLaunchKernelGGL((wo_kernel<TM, G, CB, NB, 2, TILED, I8, FUSE>), grid, block, 0, st, x, wq, m, n, k, rows,
                           sx, sw, bias, bias_kind, y, scalar_scales, fa);
    return hipGetLastError();
}

// One chunk per batch, two register buffers: measured on the decode shapes,
// larger batches leave more compute after the last bytes arrive and more
// buffers only lengthen the queues (both slower).
template <int TM, bool TILED, bool I8, int FUSE = 0>
hipError_t launch_wo_t(int groups, const void* x, const float* sx, int m, const int8_t* wq, const float* sw, int n,
                       int k, int rows, const void* bias, int bias_kind, void* y, int out_kind, int scalar_scales,
                       hipStream_t st, FuseArgs fa = FuseArgs{}) {
    switch (groups) {
        case 1: return launch_wo<TM, 1, 1, 2, TILED, I8, FUSE>(x, sx, m, wq, sw, n, k, rows, bias, bias_kind, y, out_kind, scalar_scales, st, fa);
        case 2: return launch_wo<TM, 2, 1, 2, TILED, I8, FUSE>(x, sx, m, wq, sw, n, k, rows, bias, bias_kind, y, out_kind, scalar_scales, st, fa);
        default: return launch_wo<TM, 3, 1, 2, TILED, I8, FUSE>(x, sx, m, wq, sw, n, k, rows, bias, bias_kind, y, out_kind, scalar_scales, st, fa);
    }
}

// Tokens in chunks of up to 64, each chunk streaming the weights once: the
// kernel is built for the decode shape. bf16 activations are [m][k]; int8
// codes are 16 x 64 tiles (a 64-token chunk is 4 whole groups).
template <bool TILED, bool I8>
hipError_t wo_chunks(const void* x, const float* sx, int64_t m, int64_t k, const int8_t* wq, const float* sw,
                     int64_t n, int rows, int groups, const void* bias, int bias_kind, void* y, int out_kind,
                     int scalar_scales, hipStream_t st) {
    const int ob = out_kind == 1 ? 2 : 4;
    const int ni = (int)n, ki = (int)k;
    const int64_t k64 = (k + 63) / 64 * 64;
    for (int64_t r0 = 0; r0 < m; r0 += 64) {
        const int mc = (int)((m - r0 < 64) ? m - r0 : 64);
        const void* xc = I8 ? (const void*)((const int8_t*)x + r0 * (TILED ? k64 : k))
                            : (const void*)((const uint16_t*)x + r0 * k);
        const float* sxc = (I8 && !scalar_scales) ? sx + r0 : sx;
        void* yc = (int8_t*)y + r0 * n * ob;
        hipError_t e;
        switch ((mc + 15) / 16) {
            case 1: e = launch_wo_t<1, TILED, I8>(groups, xc, sxc, mc, wq, sw, ni, ki, rows, bias, bias_kind, yc, out_kind, scalar_scales, st); break;
            case 2: e = launch_wo_t<2, TILED, I8>(groups, xc, sxc, mc, wq, sw, ni, ki, rows, bias, bias_kind, yc, out_kind, scalar_scales, st); break;
            case 3: e = launch_wo_t<3, TILED, I8>(groups, xc, sxc, mc, wq, sw, ni, ki, rows, bias, bias_kind, yc, out_kind, scalar_scales, st); break;
            default: e = launch_wo_t<4, TILED, I8>(groups, xc, sxc, mc, wq, sw, ni, ki, rows, bias, bias_kind, yc, out_kind, scalar_scales, st); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


// compute units of the current device, asked once per device
int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// tiled weights: the ceil(n / 16) row groups spread evenly over the
// workgroups, at most 3 groups each, as few rounds as that allows
void tiled_grid(int64_t n, int& wgs, int& groups) {
    const int64_t cus = compute_units();
    const int64_t ng = (n + 15) / 16;
    const int64_t rounds = (ng + cus * 3 - 1) / (cus * 3);
    const int64_t w = ng < cus * rounds ? ng : cus * rounds;
    wgs = (int)w;
    groups = (int)((ng + w - 1) / w);
}

}  // namespace

// Tokens are processed in chunks of up to 64 (each chunk streams the
// weights once): the kernel is built for the decode shape. Rows per
// workgroup: the rows spread evenly over the compute units in as few rounds
// as keep a workgroup at 48 rows or fewer, and at least 16.
hipError_t sq_launch_wo_linear(const void* x, int64_t m, int64_t k, const int8_t* wq, const float* sw, int64_t n,
                               const void* bias, int bias_kind, void* y, int out_kind, hipStream_t st) {
    const int64_t cus = compute_units();
    const int64_t rounds = (n + cus * kMaxRows - 1) / (cus * kMaxRows);
    int rows = (int)((n + cus * rounds - 1) / (cus * rounds));
    if (rows < 16) rows = 16;
    return wo_chunks<false, false>(x, nullptr, m, k, wq, sw, n, rows, (rows + 15) / 16, bias, bias_kind, y,
                                   out_kind, 0, st);
}

hipError_t sq_launch_wo_linear_tiled(const void* x, int64_t m, int64_t k, const int8_t* wq, const float* sw,
                                     int64_t n, const void* bias, int bias_kind, void* y, int out_kind,
                                     hipStream_t st) {
    int wgs, groups;
    tiled_grid(n, wgs, groups);
    return wo_chunks<true, false>(x, nullptr, m, k, wq, sw, n, wgs, groups, bias, bias_kind, y, out_kind, 0, st);
}

// the W8A8 product for m <= 64 on row-major codes
hipError_t sq_launch_gemm_stream(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq, const float* sw,
                                 int64_t n, int64_t k, const void* bias, int bias_kind, void* y, int out_kind,
                                 int scalar_scales, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int64_t cus = compute_units();
    const int64_t rounds = (n + cus * kMaxRows - 1) / (cus * kMaxRows);
    int rows = (int)((n + cus * rounds - 1) / (cus * rounds));
    if (rows < 16) rows = 16;
    return wo_chunks<false, true>(xq, sx, m, k, wq, sw, n, rows, (rows + 15) / 16, bias, bias_kind, y, out_kind,
                                  scalar_scales, st);
}

// the W8A8 product for m <= 64 on tiled codes (both operands in 16 x 64 tiles)
hipError_t sq_launch_gemm_stream_tiled(const int8_t* xq, const float* sx, int64_t m, const int8_t* wq,
                                       const float* sw, int64_t n, int64_t k, const void* bias, int bias_kind,
                                       void* y, int out_kind, int scalar_scales, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    int wgs, groups;
    tiled_grid(n, wgs, groups);
    return wo_chunks<true, true>(xq, sx, m, k, wq, sw, n, wgs, groups, bias, bias_kind, y, out_kind, scalar_scales,
                                 st);
}

// The W8A8 linear for m <= 64 in one launch (FUSED above): the activation
// codes and scales of x are written to xq (tiled) and sx by the kernel
// itself, then the weight stream multiplies them. sync: the workspace's
// synchronisation words (zero before the first call).
hipError_t sq_launch_linear_stream_fused(const void* x, int bf16, const float* s, int64_t m, int64_t k,
                                         int8_t* xq, float* sx, const int8_t* wq, const float* sw, int64_t n,
                                         const void* bias, int bias_kind, void* y, int out_kind, void* sync,
                                         int wait_polls, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    if (m > kStreamMaxM) return hipErrorInvalidValue;
    int wgs, groups;
    tiled_grid(n, wgs, groups);
    const FuseArgs fa{x, s, (FuseSync*)sync, wait_polls};
    const int mi = (int)m, ni = (int)n, ki = (int)k;
    switch ((mi + 15) / 16) {
        case 1:
            return bf16 ? launch_wo_t<1, true, true, 1>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa)
                        : launch_wo_t<1, true, true, 2>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa);
        case 2:
            return bf16 ? launch_wo_t<2, true, true, 1>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa)
                        : launch_wo_t<2, true, true, 2>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa);
        case 3:
            return bf16 ? launch_wo_t<3, true, true, 1>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa)
                        : launch_wo_t<3, true, true, 2>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa);
        default:
            return bf16 ? launch_wo_t<4, true, true, 1>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa)
                        : launch_wo_t<4, true, true, 2>(groups, xq, sx, mi, wq, sw, ni, ki, wgs, bias, bias_kind, y,
                                                        out_kind, 0, st, fa);
    }
}

size_t sq_stream_fused_sync_bytes() { return sizeof(FuseSync); }
