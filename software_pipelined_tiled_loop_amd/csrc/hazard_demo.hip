// Consume-before-reuse hazard demonstrator (page "Software pipelines and
// asynchronous copies", sections "Producer-consumer synchronization" and
// "Practice"): a two-stage tiled copy-and-reduce of an int32 array into row
// sums, with the correct stage protocol and a variant that drops only the
// reuse barrier.  Index functions and the tile geometry: hazard_demo.hpp.
//
// Per tile t (stage s = t % 2), every wave:
//   1. issues the global loads of tile t+2 into registers,
//   2. (the delayed wave only) sleeps,
//   3. reads and reduces its four rows of tile t from stage s,
//   4. REUSE_WAIT: waits at the reuse barrier until every wave has read stage s,
//   5. writes tile t+2 into stage s,
//   6. waits at the readiness barrier, after which stage s holds tile t+2 for
//      every wave and stage 1-s (written one tile earlier) holds tile t+1.
// Without step 4 a wave that reaches step 5 early overwrites rows that a
// slower wave has not read yet; the slower wave then sums tile t+2 in place of
// tile t.  Both variants execute the same addresses, and every barrier they
// keep is executed by all four waves the same number of times.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>

#include "hazard_demo.hpp"
#include "pgemm.h"

namespace hazard {

// A native 4 x int32 vector: copies of it stay in registers (HIP's int4 is a
// struct whose copies through memory are not split into registers).
typedef int v4i __attribute__((ext_vector_type(4)));

template <bool REUSE_WAIT>
__global__ void __launch_bounds__(NTH)
    copy_reduce_kernel(const int* __restrict__ X, int64_t ldx, int nT, int* __restrict__ sums, int delay_wave,
                       int delay_cycles, long long* trace, int trace_wg) {
    __shared__ v4i stage[2][CHUNKS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int* base = X + (int64_t)blockIdx.x * RB * ldx;
    const bool traced = trace != nullptr && (int)blockIdx.x == trace_wg;

    v4i st[CPT];
    uint32_t part[ROWS_PER_WAVE] = {0u, 0u, 0u, 0u};

    auto load = [&](int t) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = prod_chunk(tid, j);
            st[j] = *(const v4i*)(base + x_offset(ldx, chunk_row(c), t, chunk_col(c)));
        }
    };
    auto put = [&](int s) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) stage[s][prod_chunk(tid, j)] = st[j];
    };
    auto stamp = [&](int t, int e) {
        if (traced) {
            asm volatile("" ::: "memory");
            const long long now = (long long)__builtin_amdgcn_s_memtime();
            if (lane == 0) trace[trace_index(wave, nT, t, e)] = now;
            asm volatile("" ::: "memory");
        }
    };

    if (nT > 0) {
        // Prologue: tiles 0 and 1 into stages 0 and 1.
        load(0);
        put(0);
        if (nT > 1) {
            load(1);
            put(1);
        }
        __syncthreads();
    }
    for (int t = 0; t < nT; ++t) {
        const int s = t & 1;
        const bool refill = t + 2 < nT;
        // Past the last tile the load re-reads tile t (in bounds, never
        // written to LDS): unconditional, it stays in flight under the reads.
        load(refill ? t + 2 : t);
        stamp(t, 0);
        if (wave == delay_wave) {
            // s_sleep takes an immediate: 127 x 64 clocks per long sleep, then
            // 64-clock steps for the rest
            for (int i = 0; i < delay_cycles / 8128; ++i) __builtin_amdgcn_s_sleep(127);
            for (int i = 0; i < delay_cycles % 8128 / 64; ++i) __builtin_amdgcn_s_sleep(1);
        }
        stamp(t, 1);
        v4i v[ROWS_PER_WAVE];
#pragma unroll
        for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) v[rr] = stage[s][cons_chunk(wave, lane, rr)];
#pragma unroll
        for (int rr = 0; rr < ROWS_PER_WAVE; ++rr)
            part[rr] += (uint32_t)v[rr].x + (uint32_t)v[rr].y + (uint32_t)v[rr].z + (uint32_t)v[rr].w;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of stage s are complete
        stamp(t, 2);
        if constexpr (REUSE_WAIT) __syncthreads();  // consume-before-reuse edge
        stamp(t, 3);
        if (refill) put(s);  // stage s now holds tile t+2
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stamp(t, 4);
        __syncthreads();  // readiness edge
        stamp(t, 5);
    }
    // Exact wave reduction of each row's 64 lane partials (integer, so the
    // order does not matter).
#pragma unroll
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part[rr] += (uint32_t)__shfl_xor((int)part[rr], off);
    if (lane == 0) {
#pragma unroll
        for (int rr = 0; rr < ROWS_PER_WAVE; ++rr)
            sums[(int64_t)blockIdx.x * RB + ROWS_PER_WAVE * wave + rr] = (int)part[rr];
    }
}

}  // namespace hazard

extern "C" int pgemm_hazard_copy_reduce(const int32_t* X, int64_t rows, int64_t cols, int64_t ldx, int32_t* row_sums,
                                        int reuse_wait, int delay_wave, int delay_cycles, int64_t* trace,
                                        int64_t trace_len, int trace_wg, void* stream) {
    using namespace hazard;
    if (rows < 0 || rows % RB != 0 || cols < 0 || cols % TC != 0 || ldx < cols || ldx % 4 != 0)
        return PGEMM_ERR_INVALID_ARG;
    if (reuse_wait != 0 && reuse_wait != 1) return PGEMM_ERR_INVALID_ARG;
    if (delay_wave < -1 || delay_wave >= NWAVE || delay_cycles < 0 || delay_cycles > 10000000)
        return PGEMM_ERR_INVALID_ARG;
    if (rows == 0) return PGEMM_OK;
    if (row_sums == nullptr || (cols > 0 && (X == nullptr || ((uintptr_t)X & 15) != 0))) return PGEMM_ERR_INVALID_ARG;
    if (rows / RB > INT_MAX || cols / TC > INT_MAX / (NWAVE * EV)) return PGEMM_ERR_TOO_LARGE;
    const int grid = (int)(rows / RB);
    const int nT = (int)(cols / TC);
    if (trace != nullptr &&
        (trace_len < (int64_t)NWAVE * EV * nT || trace_wg < 0 || trace_wg >= grid || ((uintptr_t)trace & 7) != 0))
        return PGEMM_ERR_INVALID_ARG;

    const int* x = reinterpret_cast<const int*>(X);
    int* sums = reinterpret_cast<int*>(row_sums);
    long long* tr = reinterpret_cast<long long*>(trace);
    void* args[] = {&x, &ldx, (void*)&nT, &sums, &delay_wave, &delay_cycles, &tr, &trace_wg};
    const void* fn = reuse_wait ? reinterpret_cast<const void*>(&copy_reduce_kernel<true>)
                                : reinterpret_cast<const void*>(&copy_reduce_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(NTH), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        std::fprintf(stderr, "pgemm: launch of the hazard copy-reduce (grid %d) failed: %s (%d)\n", grid,
                     hipGetErrorString(e), (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}
