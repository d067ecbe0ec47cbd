// Host-only driver of the C ABI for the address and undefined-behaviour
// sanitizers: every path that returns before a launch -- the planner over a
// grid of shapes, dtypes, depths and options, argument validation of both
// entry points, the models, the variant table and the status strings.  No
// GPU is touched: every gemm call here is refused by validation first.
// Prints "OK <calls>".
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/pgemm.h"

static int calls = 0;

#define EXPECT(cond)                                                  \
    do {                                                              \
        ++calls;                                                      \
        if (!(cond)) {                                                \
            std::printf("FAIL line %d: %s\n", __LINE__, #cond);       \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main() {
    const int64_t dims[] = {0, 1, 15, 16, 17, 255, 256, 257, 1000, 4096, 4097, 100000, 1 << 20};
    for (int dtype = -1; dtype <= 4; ++dtype)
        for (int64_t M : dims)
            for (int64_t N : {(int64_t)1, (int64_t)256, (int64_t)3968, (int64_t)65536})
                for (int64_t K : dims)
                    for (int stages = -1; stages <= 5; ++stages)
                        for (int aligned = 0; aligned <= 1; ++aligned) {
                            pgemm_plan_info info;
                            const int r = pgemm_plan(M, N, K, dtype, stages, aligned, nullptr, &info);
                            ++calls;
                            if (r == PGEMM_OK) {
                                EXPECT(info.tile_m > 0 && info.tile_n > 0 && info.tile_k > 0);
                                EXPECT(info.stages >= 1 && info.stages <= 4);
                                EXPECT(info.grid % 8 == 0 && info.grid > 0);
                                EXPECT(info.lds_bytes <= 163840);
                            } else {
                                EXPECT(r < 0 && pgemm_strerror(r) != nullptr);
                            }
                        }
    // forced options, valid and invalid
    for (int producer = -1; producer <= 4; ++producer)
        for (int tm : {0, 128, 256, 64})
            for (int tk : {0, 16, 32, 64, 128})
                for (int workgroups : {-8, 0, 1, 8, 4096})
                    for (int waves : {-1, 0, 4, 8, 16}) {
                        pgemm_opts o;
                        std::memset(&o, 0, sizeof(o));
                        o.producer = producer;
                        o.tile_m = tm;
                        o.tile_n = tm;
                        o.tile_k = tk;
                        o.workgroups = workgroups;
                        o.waves = waves;
                        o.skew = (tk == 128) ? 65 : 0;
                        for (int dtype = 0; dtype <= 3; ++dtype) {
                            pgemm_plan_info info;
                            const int r = pgemm_plan(4096, 4096, 4096, dtype, 0, producer != 3, &o, &info);
                            EXPECT(r == PGEMM_OK || r < 0);
                        }
                    }
    // gemm entry points: every call fails validation before any launch
    const uintptr_t fake = (uintptr_t)1 << 20;
    const void* A = (const void*)fake;
    void* C = (void*)fake;
    EXPECT(pgemm_gemm(-1, 8, 8, 1.0, A, 8, A, 8, 0.0, C, 8, PGEMM_F32, 0, nullptr) == PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_gemm(8, 8, 8, 1.0, A, 7, A, 8, 0.0, C, 8, PGEMM_F32, 0, nullptr) == PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_gemm(8, 8, 8, 1.0, A, 8, A, 8, 0.0, C, 8, 9, 0, nullptr) == PGEMM_ERR_UNSUPPORTED_DTYPE);
    EXPECT(pgemm_gemm(8, 8, 8, 1.0, A, 8, A, 8, 0.0, C, 8, PGEMM_F32, 7, nullptr) == PGEMM_ERR_BAD_STAGES);
    EXPECT(pgemm_gemm(8, 8, 8, 0.5, A, 8, A, 8, 0.0, C, 8, PGEMM_I8, 0, nullptr) == PGEMM_ERR_NONINTEGRAL_SCALAR);
    EXPECT(pgemm_gemm(8, 8, 8, 1.0, nullptr, 8, A, 8, 0.0, C, 8, PGEMM_F32, 0, nullptr) == PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_gemm(0, 8, 8, 1.0, nullptr, 8, nullptr, 8, 0.0, nullptr, 8, PGEMM_F32, 0, nullptr) == PGEMM_OK);
    EXPECT(pgemm_gemm(8, 8, 8, 1.0, A, 8, A, 8, 0.0, C, (int64_t)1 << 40, PGEMM_F32, 0, nullptr) ==
           PGEMM_ERR_TOO_LARGE);
    pgemm_opts bad;
    std::memset(&bad, 0, sizeof(bad));
    bad.reserved[0] = 1;
    EXPECT(pgemm_gemm_ex(8, 8, 8, 1.0, A, 8, A, 8, 0.0, C, 8, PGEMM_F32, 0, &bad, nullptr) == PGEMM_ERR_INVALID_ARG);
    // hazard demonstrator validation
    const int32_t* X = (const int32_t*)fake;
    int32_t* S = (int32_t*)fake;
    EXPECT(pgemm_hazard_copy_reduce(X, 15, 256, 256, S, 1, -1, 0, nullptr, 0, 0, nullptr) == PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_hazard_copy_reduce(X, 16, 256, 256, S, 2, -1, 0, nullptr, 0, 0, nullptr) == PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_hazard_copy_reduce(X, 32, 512, 512, S, 1, -1, 0, (int64_t*)fake, 47, 0, nullptr) ==
           PGEMM_ERR_INVALID_ARG);
    EXPECT(pgemm_hazard_copy_reduce(nullptr, 0, 256, 256, nullptr, 1, -1, 0, nullptr, 0, 0, nullptr) == PGEMM_OK);
    // models, including degenerate arguments
    EXPECT(pgemm_model_uncovered_cycles(500, 220, 2) == 280);
    EXPECT(pgemm_model_uncovered_cycles(500, 0, 4) == 500);
    EXPECT(pgemm_model_lds_bytes(128, 64, 16, 2, 4, 2) == 24832);
    EXPECT(pgemm_model_global_loads_per_output(128, 64, 4096) == 96);
    EXPECT(pgemm_model_compute_load_ratio(0, 0, 0, 0) == 0);
    EXPECT(pgemm_model_compute_load_ratio(256, 256, 64, 2) == 128);
    // variant table and strings
    const int nv = pgemm_num_variants();
    EXPECT(nv > 0);
    for (int i = -2; i < nv + 2; ++i) {
        pgemm_plan_info info;
        int dt = -1;
        const int r = pgemm_variant_info(i, &info, &dt);
        EXPECT((i >= 0 && i < nv) ? (r == PGEMM_OK && dt >= 0 && dt <= 3) : r < 0);
    }
    for (int s = -10; s <= 2; ++s) EXPECT(pgemm_strerror(s) != nullptr);
    EXPECT(pgemm_version() > 0);
    std::printf("OK %d\n", calls);
    return 0;
}
