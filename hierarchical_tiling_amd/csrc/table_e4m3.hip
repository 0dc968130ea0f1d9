// table_e4m3.hip -- tile-table entries with fp8 e4m3 operands (instantiates their kernels).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "kernels.h"

namespace htk {

static const KernelEntry g_e4m3[] = {
    HT_TILED("e4m3_ak_bk_256x256x128_w2x2_m32_vec", DT_F8, 1, 1, 1, 256, 256, 128, 2, 2, 32),
    HT_TILED("e4m3_ak_bk_128x128x128_w2x2_m32_vec", DT_F8, 1, 1, 1, 128, 128, 128, 2, 2, 32),
    HT_TILED("e4m3_ak_bk_64x64x128_w2x2_m16_vec", DT_F8, 1, 1, 1, 64, 64, 128, 2, 2, 16),
    HT_TILED("e4m3_ak_bk_128x128x128_w2x2_m32_narrow", DT_F8, 1, 1, 0, 128, 128, 128, 2, 2, 32),
    HT_TILED("e4m3_ak_bn_128x128x128_w2x2_m32_narrow", DT_F8, 1, 0, 0, 128, 128, 128, 2, 2, 32),
    HT_TILED("e4m3_am_bk_128x128x128_w2x2_m32_narrow", DT_F8, 0, 1, 0, 128, 128, 128, 2, 2, 32),
    HT_TILED("e4m3_am_bn_128x128x128_w2x2_m32_narrow", DT_F8, 0, 0, 0, 128, 128, 128, 2, 2, 32),
    HT_TILED("e4m3_ak_bk_64x64x128_w2x2_m16_narrow", DT_F8, 1, 1, 0, 64, 64, 128, 2, 2, 16),
    HT_TILED("e4m3_ak_bn_64x64x128_w2x2_m16_narrow", DT_F8, 1, 0, 0, 64, 64, 128, 2, 2, 16),
    HT_TILED("e4m3_am_bk_64x64x128_w2x2_m16_narrow", DT_F8, 0, 1, 0, 64, 64, 128, 2, 2, 16),
    HT_TILED("e4m3_am_bn_64x64x128_w2x2_m16_narrow", DT_F8, 0, 0, 0, 64, 64, 128, 2, 2, 16),
    HT_DMA("e4m3_ak_bk_256x256x64_w2x2_m32_dma4", DT_F8, 256, 256, 2, 2, 32, 4, 1, 4),
    HT_DMA("e4m3_ak_bk_256x256x128_w2x2_m32_dma2", DT_F8, 256, 256, 2, 2, 32, 2, 1, 8),
    HT_RING("e4m3_ak_bk_256x256x128_w2x4_m32_ring", DT_F8, 2, 4, 32, 2),
    HT_RING("e4m3_ak_bk_256x256x128_w2x4_m32_ring1", DT_F8, 2, 4, 32, 1),
    HT_SKINNY_DMA("e4m3_ak_bk_16x32_w4_skinny_dma", DT_F8, 4, 2, 3, 2),
    HT_SKINNY("e4m3_ak_bk_16x32_w4_skinny", DT_F8, 4, 1, 2, 2, 2),
};

const KernelEntry* table_e4m3(int* n) {
  *n = (int)(sizeof(g_e4m3) / sizeof(g_e4m3[0]));
  return g_e4m3;
}

}  // namespace htk
