// table_f32.hip -- tile-table entries with fp32 operands (instantiates their kernels).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "kernels.h"

namespace htk {

static const KernelEntry g_f32[] = {
    HT_TILED("f32_ak_bk_128x128x32_w2x2_m32_vec", DT_F32, 1, 1, 1, 128, 128, 32, 2, 2, 32),
    HT_TILED("f32_ak_bn_128x128x32_w2x2_m32_vec", DT_F32, 1, 0, 1, 128, 128, 32, 2, 2, 32),
    HT_TILED("f32_am_bk_128x128x32_w2x2_m32_vec", DT_F32, 0, 1, 1, 128, 128, 32, 2, 2, 32),
    HT_TILED("f32_am_bn_128x128x32_w2x2_m32_vec", DT_F32, 0, 0, 1, 128, 128, 32, 2, 2, 32),
    HT_TILED("f32_ak_bk_64x64x32_w2x2_m16_vec", DT_F32, 1, 1, 1, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_ak_bn_64x64x32_w2x2_m16_vec", DT_F32, 1, 0, 1, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_am_bk_64x64x32_w2x2_m16_vec", DT_F32, 0, 1, 1, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_am_bn_64x64x32_w2x2_m16_vec", DT_F32, 0, 0, 1, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_ak_bk_64x64x32_w2x2_m16_narrow", DT_F32, 1, 1, 0, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_ak_bn_64x64x32_w2x2_m16_narrow", DT_F32, 1, 0, 0, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_am_bk_64x64x32_w2x2_m16_narrow", DT_F32, 0, 1, 0, 64, 64, 32, 2, 2, 16),
    HT_TILED("f32_am_bn_64x64x32_w2x2_m16_narrow", DT_F32, 0, 0, 0, 64, 64, 32, 2, 2, 16),
};

const KernelEntry* table_f32(int* n) {
  *n = (int)(sizeof(g_f32) / sizeof(g_f32[0]));
  return g_f32;
}

}  // namespace htk
