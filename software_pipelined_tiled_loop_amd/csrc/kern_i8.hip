// kern_i8.hip -- compiled variants for int8 inputs (int32 accumulation, int32 C).
#include "variants.hpp"

namespace pgemm {

#define V(BM, BN, BK, S, WGM, WGN, P) PGEMM_VARIANT(DT_I8, BM, BN, BK, S, WGM, WGN, P)
static const VariantDesc k_table[] = {
    // 256 x 256 tiles, 8 waves of 128 x 64
    V(256, 256, 64, 1, 2, 4, PROD_DIRECT),    V(256, 256, 64, 2, 2, 4, PROD_DIRECT),
    V(256, 256, 64, 3, 2, 4, PROD_DIRECT),    V(256, 256, 64, 4, 2, 4, PROD_DIRECT),
    V(256, 256, 64, 1, 2, 4, PROD_REGISTER),  V(256, 256, 64, 2, 2, 4, PROD_REGISTER),
    V(256, 256, 64, 3, 2, 4, PROD_REGISTER),  V(256, 256, 64, 4, 2, 4, PROD_REGISTER),
    V(256, 256, 128, 1, 2, 4, PROD_DIRECT),   V(256, 256, 128, 2, 2, 4, PROD_DIRECT),
    // 128 x 128 tiles, 4 waves of 64 x 64
    V(128, 128, 128, 1, 2, 2, PROD_DIRECT),   V(128, 128, 128, 2, 2, 2, PROD_DIRECT),
    V(128, 128, 128, 3, 2, 2, PROD_DIRECT),   V(128, 128, 128, 4, 2, 2, PROD_DIRECT),
    V(128, 128, 128, 1, 2, 2, PROD_GENERIC),  V(128, 128, 128, 2, 2, 2, PROD_GENERIC),
    V(128, 128, 128, 3, 2, 2, PROD_GENERIC),  V(128, 128, 128, 4, 2, 2, PROD_GENERIC),
    V(256, 256, 64, 1, 2, 4, PROD_GENERIC), V(256, 256, 64, 2, 2, 4, PROD_GENERIC),
    // one producer per operand: the misaligned operand through registers, the other by LDS-DMA
    V(256, 256, 64, 2, 2, 4, PROD_STAGED_A),  V(256, 256, 64, 2, 2, 4, PROD_STAGED_B),
    V(256, 256, 128, 2, 2, 4, PROD_STAGED_A), V(256, 256, 128, 2, 2, 4, PROD_STAGED_B),
};
#undef V

const VariantDesc* variants_i8(int* n) {
    *n = (int)(sizeof(k_table) / sizeof(k_table[0]));
    return k_table;
}

}  // namespace pgemm
