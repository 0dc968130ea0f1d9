// table_f16.hip -- tile-table entries with fp16 operands (instantiates their kernels).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "kernels.h"

namespace htk {

static const KernelEntry g_f16[] = {
    HT_TILED("f16_ak_bk_256x256x64_w2x2_m32_vec", DT_F16, 1, 1, 1, 256, 256, 64, 2, 2, 32),
    HT_TILED("f16_ak_bk_128x128x64_w2x2_m32_vec", DT_F16, 1, 1, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_ak_bn_256x256x64_w2x2_m32_vec", DT_F16, 1, 0, 1, 256, 256, 64, 2, 2, 32),
    HT_TILED("f16_ak_bn_128x128x64_w2x2_m32_vec", DT_F16, 1, 0, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bk_128x128x64_w2x2_m32_vec", DT_F16, 0, 1, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bn_128x128x64_w2x2_m32_vec", DT_F16, 0, 0, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_ak_bk_64x64x64_w2x2_m16_vec", DT_F16, 1, 1, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_ak_bn_64x64x64_w2x2_m16_vec", DT_F16, 1, 0, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bk_64x64x64_w2x2_m16_vec", DT_F16, 0, 1, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bn_64x64x64_w2x2_m16_vec", DT_F16, 0, 0, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_ak_bk_128x128x64_w2x2_m32_narrow", DT_F16, 1, 1, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_ak_bk_64x64x64_w2x2_m16_narrow", DT_F16, 1, 1, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_ak_bn_64x64x64_w2x2_m16_narrow", DT_F16, 1, 0, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bk_64x64x64_w2x2_m16_narrow", DT_F16, 0, 1, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bn_64x64x64_w2x2_m16_narrow", DT_F16, 0, 0, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_ak_bn_128x128x64_w2x2_m32_narrow", DT_F16, 1, 0, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bk_128x128x64_w2x2_m32_narrow", DT_F16, 0, 1, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bn_128x128x64_w2x2_m32_narrow", DT_F16, 0, 0, 0, 128, 128, 64, 2, 2, 32),
    // 2-byte rows at any element alignment: realigned 16-byte loads
    HT_TILED("f16_ak_bk_128x128x64_w2x2_m32_realign", DT_F16, 1, 1, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_ak_bn_128x128x64_w2x2_m32_realign", DT_F16, 1, 0, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bk_128x128x64_w2x2_m32_realign", DT_F16, 0, 1, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_am_bn_128x128x64_w2x2_m32_realign", DT_F16, 0, 0, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("f16_ak_bk_64x64x64_w2x2_m16_realign", DT_F16, 1, 1, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_ak_bn_64x64x64_w2x2_m16_realign", DT_F16, 1, 0, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bk_64x64x64_w2x2_m16_realign", DT_F16, 0, 1, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("f16_am_bn_64x64x64_w2x2_m16_realign", DT_F16, 0, 0, 2, 64, 64, 64, 2, 2, 16),
    HT_DMA("f16_ak_bk_256x256x32_w2x2_m32_dma4", DT_F16, 256, 256, 2, 2, 32, 4, 1, 4),
    HT_DMA("f16_ak_bk_256x256x64_w2x2_m32_dma2", DT_F16, 256, 256, 2, 2, 32, 2, 1, 8),
    HT_DMA("f16_ak_bk_256x256x64_w2x4_m32_dma2", DT_F16, 256, 256, 2, 4, 32, 2, 1, 8),
    HT_RING("f16_ak_bk_256x256x64_w2x4_m32_ring", DT_F16, 2, 4, 32, 2),
    HT_RING_SK("f16_ak_bk_256x256x64_w2x4_m16_ring", DT_F16, 2, 4, 16, 2),
    HT_RING_BN_SK("f16_ak_bn_256x256x64_w2x4_m16_ring", DT_F16, 2, 4, 16, 2),
    HT_SKINNY_DMA("f16_ak_bk_16x32_w4_skinny_dma", DT_F16, 4, 2, 3, 2),
    HT_SKINNY("f16_ak_bk_16x32_w8_skinny", DT_F16, 8, 1, 2, 2, 4),
};

const KernelEntry* table_f16(int* n) {
  *n = (int)(sizeof(g_f16) / sizeof(g_f16[0]));
  return g_f16;
}

}  // namespace htk
