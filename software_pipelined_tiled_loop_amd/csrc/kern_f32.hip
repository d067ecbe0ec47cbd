// kern_f32.hip -- compiled variants for fp32 inputs (fp32 MFMA, fp32 C).
#include "variants.hpp"

namespace pgemm {

#define V(BM, BN, BK, S, WGM, WGN, P) PGEMM_VARIANT(DT_F32, BM, BN, BK, S, WGM, WGN, P)
static const VariantDesc k_table[] = {
    // the 128 x 64 x 16 tile class of the pages' SGEMM kernel (4 waves of 64 x 32)
    V(128, 64, 16, 1, 2, 2, PROD_DIRECT),     V(128, 64, 16, 2, 2, 2, PROD_DIRECT),
    V(128, 64, 16, 3, 2, 2, PROD_DIRECT),     V(128, 64, 16, 4, 2, 2, PROD_DIRECT),
    V(128, 64, 16, 1, 2, 2, PROD_REGISTER),   V(128, 64, 16, 2, 2, 2, PROD_REGISTER),
    // 256 x 256 tiles, 8 waves of 128 x 64
    V(256, 256, 32, 1, 2, 4, PROD_DIRECT),    V(256, 256, 32, 2, 2, 4, PROD_DIRECT),
    // 128 x 128 tiles, 4 waves of 64 x 64
    V(128, 128, 32, 1, 2, 2, PROD_DIRECT),    V(128, 128, 32, 2, 2, 2, PROD_DIRECT),
    V(128, 128, 32, 3, 2, 2, PROD_DIRECT),    V(128, 128, 32, 4, 2, 2, PROD_DIRECT),
    V(128, 128, 32, 1, 2, 2, PROD_GENERIC),   V(128, 128, 32, 2, 2, 2, PROD_GENERIC),
    V(128, 128, 32, 3, 2, 2, PROD_GENERIC),   V(128, 128, 32, 4, 2, 2, PROD_GENERIC),
    V(128, 64, 16, 1, 2, 2, PROD_GENERIC),    V(128, 64, 16, 2, 2, 2, PROD_GENERIC),
    V(256, 256, 32, 1, 2, 4, PROD_GENERIC),   V(256, 256, 32, 2, 2, 4, PROD_GENERIC),
    // one producer per operand: the misaligned operand through registers, the other by LDS-DMA
    V(128, 64, 16, 2, 2, 2, PROD_STAGED_A),   V(128, 64, 16, 2, 2, 2, PROD_STAGED_B),
    V(256, 256, 32, 2, 2, 4, PROD_STAGED_A),  V(256, 256, 32, 2, 2, 4, PROD_STAGED_B),
};
#undef V

const VariantDesc* variants_f32(int* n) {
    *n = (int)(sizeof(k_table) / sizeof(k_table[0]));
    return k_table;
}

}  // namespace pgemm
