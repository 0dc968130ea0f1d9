// table_bf16_dma.hip -- tile-table entries with bf16 operands, DMA-fed kernels (instantiates their kernels).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "kernels.h"

namespace htk {

static const KernelEntry g_bf16_dma[] = {
    HT_DMA("bf16_ak_bk_256x256x32_w2x2_m32_dma4", DT_BF16, 256, 256, 2, 2, 32, 4, 1, 4),
    HT_DMA("bf16_ak_bk_256x256x32_w2x2_m32_dma5", DT_BF16, 256, 256, 2, 2, 32, 5, 1, 4),
    HT_DMA("bf16_ak_bk_256x128x32_w2x2_m32_dma3_o2", DT_BF16, 256, 128, 2, 2, 32, 3, 2, 4),
    HT_DMA("bf16_ak_bk_128x256x32_w2x2_m32_dma3_o2", DT_BF16, 128, 256, 2, 2, 32, 3, 2, 4),
    HT_DMA("bf16_ak_bk_256x128x32_w4x1_m32_dma3_o2", DT_BF16, 256, 128, 4, 1, 32, 3, 2, 4),
    HT_DMA("bf16_ak_bk_256x256x64_w2x2_m32_dma2", DT_BF16, 256, 256, 2, 2, 32, 2, 1, 8),
    HT_DMA("bf16_ak_bk_256x128x64_w2x2_m32_dma3", DT_BF16, 256, 128, 2, 2, 32, 3, 1, 8),
    HT_DMA("bf16_ak_bk_256x256x32_w2x4_m32_dma5", DT_BF16, 256, 256, 2, 4, 32, 5, 1, 4),
    HT_DMA("bf16_ak_bk_256x256x32_w4x2_m32_dma5", DT_BF16, 256, 256, 4, 2, 32, 5, 1, 4),
    HT_DMA("bf16_ak_bk_256x256x64_w2x4_m32_dma2", DT_BF16, 256, 256, 2, 4, 32, 2, 1, 8),
    HT_RING("bf16_ak_bk_256x256x64_w2x4_m32_ring", DT_BF16, 2, 4, 32, 2),
    HT_RING_SK("bf16_ak_bk_256x256x64_w2x4_m16_ring", DT_BF16, 2, 4, 16, 2),
    HT_RING("bf16_ak_bk_256x256x64_w2x4_m16_ring1", DT_BF16, 2, 4, 16, 1),
    HT_RING_BN_SK("bf16_ak_bn_256x256x64_w2x4_m16_ring", DT_BF16, 2, 4, 16, 2),
    HT_SKINNY_DMA("bf16_ak_bk_16x32_w4_skinny_dma", DT_BF16, 4, 2, 3, 2),
    HT_SKINNY("bf16_ak_bk_16x32_w8_skinny", DT_BF16, 8, 1, 2, 2, 4),
};

const KernelEntry* table_bf16_dma(int* n) {
  *n = (int)(sizeof(g_bf16_dma) / sizeof(g_bf16_dma[0]));
  return g_bf16_dma;
}

}  // namespace htk
