// diag.hip -- diagnostic kernels that bound the pipelined GEMM from above,
// and a wait-profile build of the GEMM itself.  None of them is part of the
// GEMM path: nothing in pgemm_gemm calls them.
//
// Page "Software pipelines and asynchronous copies" (section "Worked example:
// Choosing between two and four stages", last point) warns that a timing
// difference alone does not show the cause; these measure the two resources
// whose limits set the GEMM's ceiling on this part:
//
//   mfma_ceiling_kernel  the matrix cores alone: every SIMD runs two waves (or
//                        one) of back-to-back MFMAs on independent
//                        accumulators, 16x16 blocks (the GEMM's) or 32x32
//                        blocks, operands from random (or zero) register
//                        data, no memory traffic.  Random operands draw more
//                        power than zeros, and the part lowers its clock for
//                        them; one wave per SIMD shows what a single issuing
//                        wave can keep busy.
//   lds_stream_kernel    the producer alone: the exact LDS-DMA pieces of a
//                        GEMM tile class (same raster, same 1-KiB blocks,
//                        same ring depth and ready barrier per K tile), no
//                        fragment reads, no MFMA.  Its rate is the most the
//                        ring can feed the consumer from L2.
//   wait profile         the GEMM kernel of a DIRECT variant built with
//                        ProbeCfg: shader-clock stamps split each ready edge
//                        into its vmcnt wait (tile landed) and its barrier
//                        wait, per wave (page "Software pipelines and
//                        asynchronous copies", introduction: stalls mapped to
//                        the wait before the next panel).
#include <hip/hip_runtime.h>

#include <cstdio>

#include "pgemm.h"
#include "pgemm_kernel.hpp"

namespace pgemm {
namespace diag {

constexpr int kAcc = 16;  // independent 16x16 accumulators per wave (eight 32x32 ones: the same flops)

// 32-bit integer mixing function (the MurmurHash3 finalizer).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

// A float uniform in [-1, 1) from 24 random bits.
__device__ __forceinline__ float unit(uint32_t h) { return (float)(h >> 8) * (2.0f / 16777216.0f) - 1.0f; }

// One 32-bit operand word of random data in the dtype's format.
template <int D>
__device__ __forceinline__ int operand_word(uint32_t h0, uint32_t h1) {
    if constexpr (D == DT_BF16) {
        const uint32_t lo = __builtin_bit_cast(uint32_t, unit(h0)) >> 16;
        const uint32_t hi = __builtin_bit_cast(uint32_t, unit(h1)) >> 16;
        return (int)(lo | (hi << 16));
    } else if constexpr (D == DT_F16) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)unit(h0));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)unit(h1));
        return (int)(lo | (hi << 16));
    } else if constexpr (D == DT_I8) {
        return (int)h0;  // four random int8 values
    } else {
        return __builtin_bit_cast(int, unit(h0));
    }
}

// The two members of a tile configuration that mfma_block reads.
template <int D>
struct DiagCfg {
    static constexpr int Dt = D;
    typedef Traits<D> T;
};

// Accumulator of a 32x32 MFMA block: 16 values per lane.
template <int D>
struct Acc32 {
    typedef __attribute__((ext_vector_type(16))) float T;
};
template <>
struct Acc32<DT_I8> {
    typedef __attribute__((ext_vector_type(16))) int T;
};

// One 32x32 MFMA block (K 16 for fp16/bf16, 32 for int8): twice the flops of
// the 16x16 block of mfma_block.
template <int D>
__device__ __forceinline__ void mfma_block32(typename Acc32<D>::T& acc, const i32x4& a, const i32x4& b) {
    if constexpr (D == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0,
                                                      0, 0);
    } else if constexpr (D == DT_F16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0,
                                                     0);
    } else {
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
    }
}

// NT threads (NT / 256 waves per SIMD), BLK: 16 (sixteen 16x16 accumulators)
// or 32 (eight 32x32 ones, fp16/bf16/int8 only).
template <int D, int NT, int BLK>
__global__ void __launch_bounds__(NT) mfma_ceiling_kernel(int iters, uint32_t seed, int zero, float* out,
                                                          long long* clock) {
    const long long rt0 = (long long)__builtin_amdgcn_s_memrealtime();
    const long long cy0 = (long long)__builtin_amdgcn_s_memtime();
    // 96 KiB of LDS that nothing but an impossible branch touches: it keeps
    // one workgroup per CU, so every SIMD holds exactly NT / 256 of these
    // waves.
    __shared__ char hold[98304];
    if (iters < 0) hold[threadIdx.x] = 0;
    typedef typename Traits<D>::Acc Acc;
    i32x4 a[4], b[4];
    const uint32_t base = seed ^ ((uint32_t)blockIdx.x << 16) ^ ((uint32_t)threadIdx.x << 5);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t k = base + (uint32_t)(q * 4 + e) * 2u;
            a[q][e] = zero ? 0 : operand_word<D>(mix32(k), mix32(k ^ 0x5bd1e995u));
            b[q][e] = zero ? 0 : operand_word<D>(mix32(k + 1u), mix32((k + 1u) ^ 0x5bd1e995u));
        }
    float s = 0.0f;
    if constexpr (BLK == 16) {
        Acc acc[kAcc];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = Acc{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j) mfma_block<DiagCfg<D>>(acc[j], a[j & 3], b[j >> 2]);
        }
        // keep every accumulator live: one value per wave
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += (float)acc[j][e];
    } else {
        typedef typename Acc32<D>::T A32;
        A32 acc[kAcc / 2];
#pragma unroll
        for (int j = 0; j < kAcc / 2; ++j) acc[j] = A32{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kAcc / 2; ++j) mfma_block32<D>(acc[j], a[j & 3], b[j >> 2]);
        }
#pragma unroll
        for (int j = 0; j < kAcc / 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += (float)acc[j][e];
    }
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * (NT / 64) + (threadIdx.x >> 6)] = s;
    if (clock != nullptr && threadIdx.x == 0) {
        // wave 0's shader and 100 MHz clocks at its start and end
        const long long cy1 = (long long)__builtin_amdgcn_s_memtime();
        const long long rt1 = (long long)__builtin_amdgcn_s_memrealtime();
        long long* o = clock + (int64_t)blockIdx.x * kClockWords;
        o[0] = cy0;
        o[1] = rt0;
        o[2] = cy1;
        o[3] = rt1;
    }
}

// Flops of one mfma_block call.
constexpr int64_t block_flops(int d) { return d == DT_F32 ? 2 * 16 * 16 * 16 : d == DT_I8 ? 2 * 16 * 16 * 64 : 2 * 16 * 16 * 32; }

// The producer of tile class C alone: K tiles 0 .. S-2 in the prologue, then
// per K tile t the pieces of tile t+S-1 and the ready barrier of tile t.
// Pieces past the last K tile load nothing (every lane out of range).
template <class C>
__global__ void __launch_bounds__(C::NT) lds_stream_kernel(KernelArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    char PGEMM_LDS* smem = (char PGEMM_LDS*)smem_raw;
    const WgTiles w = wg_tiles(g);
    if (w.count == 0) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int m0, n0;
    wg_tile_origin<C>(g, w, 0, m0, n0);
    const int nK = (g.K + C::BK - 1) / C::BK;
#pragma unroll
    for (int p = 0; p < C::S - 1; ++p) issue_dma<C>(g, m0, n0, p, smem + p * C::STAGE_BYTES, wave, lane);
    int ahead = (C::S - 1) % C::S;
    for (int t = 0; t < nK; ++t) {
        issue_dma<C>(g, m0, n0, t + C::S - 1, smem + ahead * C::STAGE_BYTES, wave, lane);
        ahead = ahead + 1 == C::S ? 0 : ahead + 1;
        wait_barrier<C::LPS * (C::S - 1)>();  // K tile t has landed for every wave
    }
    __builtin_amdgcn_s_waitcnt(0);
}

struct StreamVariant {
    int dtype, bm, bn, bk, stages;
    const void* fn;
    int threads, stage_bytes;
};

#define PGEMM_STREAM(D, BM, BN, BK, S, WGM, WGN)                                                        \
    StreamVariant {                                                                                    \
        D, BM, BN, BK, S, reinterpret_cast<const void*>(&lds_stream_kernel<Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>>), \
            Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>::NT, Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>::STAGE_BYTES \
    }

// The tile classes of the benchmark's plans (and the ring depths of the
// bf16 256 x 256 x 32 class).
static const StreamVariant k_streams[] = {
    PGEMM_STREAM(DT_BF16, 256, 256, 64, 2, 2, 4), PGEMM_STREAM(DT_BF16, 256, 256, 32, 2, 2, 4),
    PGEMM_STREAM(DT_BF16, 256, 256, 32, 3, 2, 4), PGEMM_STREAM(DT_BF16, 256, 256, 32, 4, 2, 4),
    PGEMM_STREAM(DT_F16, 256, 256, 64, 2, 2, 4),  PGEMM_STREAM(DT_I8, 256, 256, 128, 2, 2, 4),
    PGEMM_STREAM(DT_F32, 128, 64, 16, 2, 2, 2),   PGEMM_STREAM(DT_F32, 256, 256, 32, 2, 2, 4),
};

struct ProbeVariant {
    int dtype, bm, bn, bk, stages;
    const void* fn;
    int threads, nw;
};

#define PGEMM_PROBE(D, BM, BN, BK, S, WGM, WGN)                                                          \
    ProbeVariant {                                                                                       \
        D, BM, BN, BK, S,                                                                                \
            reinterpret_cast<const void*>(&gemm_kernel<ProbeCfg<Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>>, false>), \
            Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>::NT, WGM * WGN                                  \
    }

// The planner's 4096^3 classes at one and two stages, and the bf16
// 256 x 256 x 32 class at every depth.
static const ProbeVariant k_probes[] = {
    PGEMM_PROBE(DT_BF16, 256, 256, 64, 1, 2, 4), PGEMM_PROBE(DT_BF16, 256, 256, 64, 2, 2, 4),
    PGEMM_PROBE(DT_BF16, 256, 256, 32, 1, 2, 4), PGEMM_PROBE(DT_BF16, 256, 256, 32, 2, 2, 4),
    PGEMM_PROBE(DT_BF16, 256, 256, 32, 3, 2, 4), PGEMM_PROBE(DT_BF16, 256, 256, 32, 4, 2, 4),
    PGEMM_PROBE(DT_BF16, 128, 128, 64, 2, 2, 2), PGEMM_PROBE(DT_BF16, 128, 128, 64, 3, 2, 2),
    PGEMM_PROBE(DT_F16, 256, 256, 64, 1, 2, 4),  PGEMM_PROBE(DT_F16, 256, 256, 64, 2, 2, 4),
    PGEMM_PROBE(DT_I8, 256, 256, 128, 1, 2, 4),  PGEMM_PROBE(DT_I8, 256, 256, 128, 2, 2, 4),
    PGEMM_PROBE(DT_F32, 128, 64, 16, 1, 2, 2),   PGEMM_PROBE(DT_F32, 128, 64, 16, 2, 2, 2),
    PGEMM_PROBE(DT_F32, 256, 256, 32, 1, 2, 4),  PGEMM_PROBE(DT_F32, 256, 256, 32, 2, 2, 4),
};

// The parts ladder: the GEMM kernel of a DIRECT class built with parts of
// its steady state left out (PartsCfg), from the matrix cores alone up to
// the whole K loop.
struct PartsVariant {
    int dtype, bm, bn, bk, stages, parts;
    const void* fn;
    int threads;
};

#define PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PT)                                                              \
    PartsVariant {                                                                                                 \
        D, BM, BN, BK, S, PT,                                                                                      \
            reinterpret_cast<const void*>(&gemm_kernel<PartsCfg<Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>, PT>, false>), \
            Cfg<D, BM, BN, BK, S, WGM, WGN, PROD_DIRECT>::NT                                                       \
    }
#define PGEMM_PARTS(D, BM, BN, BK, S, WGM, WGN)                                                                    \
    PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, 0), PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PART_AREADS),           \
        PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PART_BREADS),                                                     \
        PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PART_AREADS | PART_BREADS),                                       \
        PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PART_AREADS | PART_BREADS | PART_BARRIER),                        \
        PGEMM_PARTS1(D, BM, BN, BK, S, WGM, WGN, PART_ALL)

// The planner's 4096^3 classes.
static const PartsVariant k_parts[] = {
    PGEMM_PARTS(DT_BF16, 256, 256, 64, 2, 2, 4),
    PGEMM_PARTS(DT_F16, 256, 256, 64, 2, 2, 4),
    PGEMM_PARTS(DT_I8, 256, 256, 128, 2, 2, 4),
    PGEMM_PARTS(DT_F32, 128, 64, 16, 2, 2, 2),
};

}  // namespace diag
}  // namespace pgemm

using namespace pgemm;
using namespace pgemm::diag;

template <int D, int NT>
static const void* ceiling_fn(int block) {
    if constexpr (D == DT_F32) {
        return reinterpret_cast<const void*>(&mfma_ceiling_kernel<D, NT, 16>);
    } else {
        return block == 32 ? reinterpret_cast<const void*>(&mfma_ceiling_kernel<D, NT, 32>)
                           : reinterpret_cast<const void*>(&mfma_ceiling_kernel<D, NT, 16>);
    }
}

template <int NT>
static const void* ceiling_fn(int dtype, int block) {
    return dtype == PGEMM_F32    ? ceiling_fn<DT_F32, NT>(block)
           : dtype == PGEMM_F16  ? ceiling_fn<DT_F16, NT>(block)
           : dtype == PGEMM_BF16 ? ceiling_fn<DT_BF16, NT>(block)
                                 : ceiling_fn<DT_I8, NT>(block);
}

extern "C" int pgemm_diag_mfma_ceiling(int dtype, int zero_operands, int waves_per_simd, int block, int iters,
                                       int grid, uint32_t seed, float* out, int64_t* flops, int64_t* clock,
                                       void* stream) {
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if ((zero_operands != 0 && zero_operands != 1) || (waves_per_simd != 1 && waves_per_simd != 2) ||
        (block != 16 && block != 32) || (block == 32 && dtype == PGEMM_F32) || iters < 0 || iters > (1 << 24) ||
        grid < 1 || grid > 65536 || out == nullptr || ((uintptr_t)out & 3) != 0 || ((uintptr_t)clock & 7) != 0)
        return PGEMM_ERR_INVALID_ARG;
    const int threads = 256 * waves_per_simd;
    const void* fn = waves_per_simd == 1 ? ceiling_fn<256>(dtype, block) : ceiling_fn<512>(dtype, block);
    if (flops) *flops = (int64_t)grid * (threads / 64) * iters * kAcc * block_flops(dtype);
    long long* clk = reinterpret_cast<long long*>(clock);
    void* args[] = {&iters, &seed, &zero_operands, &out, &clk};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        std::fprintf(stderr, "pgemm: launch of the MFMA ceiling kernel failed: %s (%d)\n", hipGetErrorString(e), (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}

extern "C" int pgemm_diag_lds_stream(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                     int64_t ldb, int dtype, int tile_m, int tile_n, int tile_k, int stages,
                                     int64_t* lds_bytes, void* stream) {
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || lda < K || ldb < N) return PGEMM_ERR_INVALID_ARG;
    const int es = dtype == PGEMM_F32 ? 4 : dtype == PGEMM_I8 ? 1 : 2;
    // the aligned case: both operands 16-byte aligned, rows of whole 16-byte chunks
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || (lda * es) % 16 || (ldb * es) % 16 || (K * es) % 16 ||
        (N * es) % 16)
        return PGEMM_ERR_INVALID_ARG;
    if (M > 0x7fffff00 || N > 0x7fffff00 || K > 0x7fffff00 || (double)lda * es * 256.0 >= 2147483648.0 ||
        (double)ldb * es * 128.0 >= 2147483648.0)
        return PGEMM_ERR_TOO_LARGE;
    const StreamVariant* v = nullptr;
    for (const StreamVariant& s : k_streams)
        if (s.dtype == dtype && s.bm == tile_m && s.bn == tile_n && s.bk == tile_k && s.stages == stages) v = &s;
    if (!v) return PGEMM_ERR_INFEASIBLE_PLAN;
    KernelArgs a{};
    a.A = A;
    a.B = B;
    a.lda = lda;
    a.ldb = ldb;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)((M + v->bm - 1) / v->bm);
    a.tiles_n = (int)((N + v->bn - 1) / v->bn);
    a.group_m = 4;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > 0x7ffffff0) return PGEMM_ERR_TOO_LARGE;
    const int grid = (int)((tiles + 7) / 8 * 8);
    if (lds_bytes) *lds_bytes = tiles * ((K + v->bk - 1) / v->bk) * v->stage_bytes;
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(v->fn, dim3(grid), dim3(v->threads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        std::fprintf(stderr, "pgemm: launch of the LDS stream kernel failed: %s (%d)\n", hipGetErrorString(e), (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}

extern "C" int pgemm_diag_wait_profile(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                       int64_t ldb, void* C, int64_t ldc, int dtype, int tile_m, int tile_n,
                                       int tile_k, int stages, int64_t* out, int64_t out_len, void* stream) {
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !C || lda < K || ldb < N || ldc < N || !out ||
        ((uintptr_t)out & 7) != 0)
        return PGEMM_ERR_INVALID_ARG;
    const int es = dtype == PGEMM_F32 ? 4 : dtype == PGEMM_I8 ? 1 : 2;
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)C & 3) || (lda * es) % 16 || (ldb * es) % 16 ||
        (K * es) % 16 || (N * es) % 16)
        return PGEMM_ERR_INVALID_ARG;
    if (M > 0x7fffff00 || N > 0x7fffff00 || K > 0x7fffff00 || (double)lda * es * 256.0 >= 2147483648.0 ||
        (double)ldb * es * 128.0 >= 2147483648.0 || (double)ldc * 4.0 * 256.0 >= 2147483648.0)
        return PGEMM_ERR_TOO_LARGE;
    const ProbeVariant* v = nullptr;
    for (const ProbeVariant& p : k_probes)
        if (p.dtype == dtype && p.bm == tile_m && p.bn == tile_n && p.bk == tile_k && p.stages == stages) v = &p;
    if (!v) return PGEMM_ERR_INFEASIBLE_PLAN;
    KernelArgs a{};
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)((M + v->bm - 1) / v->bm);
    a.tiles_n = (int)((N + v->bn - 1) / v->bn);
    a.group_m = 4;
    a.alpha = 1.0f;
    a.ialpha = 1;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > 0x7ffffff0) return PGEMM_ERR_TOO_LARGE;
    const int grid = (int)((tiles + 7) / 8 * 8);
    // every workgroup with a tile writes kProbeWords entries per wave; idle ones write nothing
    if (out_len < (int64_t)grid * v->nw * kProbeWords) return PGEMM_ERR_INVALID_ARG;
    a.probe = reinterpret_cast<long long*>(out);
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(v->fn, dim3(grid), dim3(v->threads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        std::fprintf(stderr, "pgemm: launch of the wait-profile kernel failed: %s (%d)\n", hipGetErrorString(e),
                     (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}

extern "C" int pgemm_diag_parts(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                int64_t ldb, void* C, int64_t ldc, int dtype, int tile_m, int tile_n, int tile_k,
                                int stages, int parts, int64_t* clock, int64_t clock_len, void* stream) {
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !C || lda < K || ldb < N || ldc < N || !clock ||
        ((uintptr_t)clock & 7) != 0 || parts < 0 || parts > PART_ALL)
        return PGEMM_ERR_INVALID_ARG;
    const int es = dtype == PGEMM_F32 ? 4 : dtype == PGEMM_I8 ? 1 : 2;
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)C & 3) || (lda * es) % 16 || (ldb * es) % 16 ||
        (K * es) % 16 || (N * es) % 16)
        return PGEMM_ERR_INVALID_ARG;
    if (M > 0x7fffff00 || N > 0x7fffff00 || K > 0x7fffff00 || (double)lda * es * 256.0 >= 2147483648.0 ||
        (double)ldb * es * 128.0 >= 2147483648.0 || (double)ldc * 4.0 * 256.0 >= 2147483648.0)
        return PGEMM_ERR_TOO_LARGE;
    const PartsVariant* v = nullptr;
    for (const PartsVariant& p : k_parts)
        if (p.dtype == dtype && p.bm == tile_m && p.bn == tile_n && p.bk == tile_k && p.stages == stages &&
            p.parts == parts)
            v = &p;
    if (!v) return PGEMM_ERR_INFEASIBLE_PLAN;
    KernelArgs a{};
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)((M + v->bm - 1) / v->bm);
    a.tiles_n = (int)((N + v->bn - 1) / v->bn);
    a.group_m = 4;
    a.alpha = 1.0f;
    a.ialpha = 1;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > 0x7ffffff0) return PGEMM_ERR_TOO_LARGE;
    const int grid = (int)((tiles + 7) / 8 * 8);
    // every workgroup with a tile writes kClockWords entries; idle ones write nothing
    if (clock_len < (int64_t)grid * kClockWords) return PGEMM_ERR_INVALID_ARG;
    a.probe = reinterpret_cast<long long*>(clock);
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(v->fn, dim3(grid), dim3(v->threads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        std::fprintf(stderr, "pgemm: launch of the parts-ladder kernel failed: %s (%d)\n", hipGetErrorString(e),
                     (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}
