// kern_f16.hip -- compiled variants for f16 inputs (fp32 accumulation, fp32 C).
#include "variants.hpp"

namespace pgemm {

#define V(BM, BN, BK, S, WGM, WGN, P) PGEMM_VARIANT(DT_F16, BM, BN, BK, S, WGM, WGN, P)
static const VariantDesc k_table[] = {
    // 256 x 256 tiles, 8 waves of 128 x 64 (two waves per SIMD)
    V(256, 256, 32, 1, 2, 4, PROD_DIRECT),   V(256, 256, 32, 2, 2, 4, PROD_DIRECT),
    V(256, 256, 32, 3, 2, 4, PROD_DIRECT),   V(256, 256, 32, 4, 2, 4, PROD_DIRECT),
    V(256, 256, 32, 1, 2, 4, PROD_REGISTER), V(256, 256, 32, 2, 2, 4, PROD_REGISTER),
    V(256, 256, 32, 3, 2, 4, PROD_REGISTER), V(256, 256, 32, 4, 2, 4, PROD_REGISTER),
    V(256, 256, 64, 1, 2, 4, PROD_DIRECT),   V(256, 256, 64, 2, 2, 4, PROD_DIRECT),
    // 128 x 128 tiles, 4 waves of 64 x 64
    V(128, 128, 64, 1, 2, 2, PROD_DIRECT),   V(128, 128, 64, 2, 2, 2, PROD_DIRECT),
    V(128, 128, 64, 3, 2, 2, PROD_DIRECT),   V(128, 128, 64, 4, 2, 2, PROD_DIRECT),
    V(128, 128, 64, 2, 2, 2, PROD_REGISTER),
    // generic producer for misaligned operands
    V(128, 128, 64, 1, 2, 2, PROD_GENERIC),  V(128, 128, 64, 2, 2, 2, PROD_GENERIC),
    V(128, 128, 64, 3, 2, 2, PROD_GENERIC),  V(128, 128, 64, 4, 2, 2, PROD_GENERIC),
    V(256, 256, 32, 1, 2, 4, PROD_GENERIC), V(256, 256, 32, 2, 2, 4, PROD_GENERIC),
    // one producer per operand: the misaligned operand through registers, the other by LDS-DMA
    V(256, 256, 32, 2, 2, 4, PROD_STAGED_A), V(256, 256, 32, 2, 2, 4, PROD_STAGED_B),
    V(256, 256, 64, 2, 2, 4, PROD_STAGED_A), V(256, 256, 64, 2, 2, 4, PROD_STAGED_B),
};
#undef V

const VariantDesc* variants_f16(int* n) {
    *n = (int)(sizeof(k_table) / sizeof(k_table[0]));
    return k_table;
}

}  // namespace pgemm
