// variants.hpp -- the table of compiled kernel variants (host side).
#pragma once

#include <hip/hip_runtime.h>
#include "pgemm_kernel.hpp"

namespace pgemm {

typedef hipError_t (*LaunchFn)(const KernelArgs&, int grid, hipStream_t);

struct VariantDesc {
    int dtype, bm, bn, bk, stages, wgm, wgn, producer;
    int threads, lds_bytes;
    LaunchFn launch;             // one workgroup per output tile
    LaunchFn launch_persistent;  // fewer workgroups, each looping over its tiles
};

// hipLaunchKernel returns this launch's own status; reading the runtime's
// last-error slot instead could report an earlier, unrelated failure.
template <class C, bool STREAM>
hipError_t launch_variant(const KernelArgs& a, int grid, hipStream_t s) {
    KernelArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<C, STREAM>), dim3(grid), dim3(C::NT), args, 0,
                           s);
}

#define PGEMM_VARIANT(D, BM, BN, BK, S, WGM, WGN, P)                                      \
    VariantDesc {                                                                         \
        D, BM, BN, BK, S, WGM, WGN, P, Cfg<D, BM, BN, BK, S, WGM, WGN, P>::NT,             \
            Cfg<D, BM, BN, BK, S, WGM, WGN, P>::LDS_BYTES,                                 \
            &launch_variant<Cfg<D, BM, BN, BK, S, WGM, WGN, P>, false>,                    \
            &launch_variant<Cfg<D, BM, BN, BK, S, WGM, WGN, P>, true>                      \
    }

// Per-dtype tables, each defined in its own translation unit.
const VariantDesc* variants_f32(int* n);
const VariantDesc* variants_f16(int* n);
const VariantDesc* variants_bf16(int* n);
const VariantDesc* variants_i8(int* n);

}  // namespace pgemm
