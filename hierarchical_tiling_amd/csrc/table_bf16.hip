// table_bf16.hip -- tile-table entries with bf16 operands, register-staged loads (instantiates their kernels).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "kernels.h"

namespace htk {

static const KernelEntry g_bf16[] = {
    HT_TILED("bf16_ak_bk_256x256x64_w2x2_m32_vec", DT_BF16, 1, 1, 1, 256, 256, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bk_128x128x64_w2x2_m32_vec", DT_BF16, 1, 1, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bk_256x256x64_w2x4_m32_vec", DT_BF16, 1, 1, 1, 256, 256, 64, 2, 4, 32),
    HT_TILED("bf16_ak_bn_256x256x64_w2x2_m32_vec", DT_BF16, 1, 0, 1, 256, 256, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bn_128x128x64_w2x2_m32_vec", DT_BF16, 1, 0, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bk_128x128x64_w2x2_m32_vec", DT_BF16, 0, 1, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bn_128x128x64_w2x2_m32_vec", DT_BF16, 0, 0, 1, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bk_64x64x64_w2x2_m16_vec", DT_BF16, 1, 1, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_ak_bn_64x64x64_w2x2_m16_vec", DT_BF16, 1, 0, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bk_64x64x64_w2x2_m16_vec", DT_BF16, 0, 1, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bn_64x64x64_w2x2_m16_vec", DT_BF16, 0, 0, 1, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_ak_bk_128x128x64_w2x2_m32_narrow", DT_BF16, 1, 1, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bk_64x64x64_w2x2_m16_narrow", DT_BF16, 1, 1, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_ak_bn_64x64x64_w2x2_m16_narrow", DT_BF16, 1, 0, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bk_64x64x64_w2x2_m16_narrow", DT_BF16, 0, 1, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bn_64x64x64_w2x2_m16_narrow", DT_BF16, 0, 0, 0, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_ak_bn_128x128x64_w2x2_m32_narrow", DT_BF16, 1, 0, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bk_128x128x64_w2x2_m32_narrow", DT_BF16, 0, 1, 0, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bn_128x128x64_w2x2_m32_narrow", DT_BF16, 0, 0, 0, 128, 128, 64, 2, 2, 32),
    // 2-byte rows at any element alignment: realigned 16-byte loads
    HT_TILED("bf16_ak_bk_128x128x64_w2x2_m32_realign", DT_BF16, 1, 1, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bn_128x128x64_w2x2_m32_realign", DT_BF16, 1, 0, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bk_128x128x64_w2x2_m32_realign", DT_BF16, 0, 1, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_am_bn_128x128x64_w2x2_m32_realign", DT_BF16, 0, 0, 2, 128, 128, 64, 2, 2, 32),
    HT_TILED("bf16_ak_bk_64x64x64_w2x2_m16_realign", DT_BF16, 1, 1, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_ak_bn_64x64x64_w2x2_m16_realign", DT_BF16, 1, 0, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bk_64x64x64_w2x2_m16_realign", DT_BF16, 0, 1, 2, 64, 64, 64, 2, 2, 16),
    HT_TILED("bf16_am_bn_64x64x64_w2x2_m16_realign", DT_BF16, 0, 0, 2, 64, 64, 64, 2, 2, 16),
};

const KernelEntry* table_bf16(int* n) {
  *n = (int)(sizeof(g_bf16) / sizeof(g_bf16[0]));
  return g_bf16;
}

}  // namespace htk
