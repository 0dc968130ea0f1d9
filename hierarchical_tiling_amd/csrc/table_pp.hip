// table_pp.hip -- tile-table entries of the ping-pong kernel (instantiates it).
// Entry fields and the selection rule are described in gemm_internal.h and api.cpp.
#include "pingpong.h"

namespace htk {

static const KernelEntry g_pp[] = {
    HT_PP("bf16_ak_bk_256x256x64_w2x4_m16_pp", DT_BF16),
    HT_PP("f16_ak_bk_256x256x64_w2x4_m16_pp", DT_F16),
    HT_PP("e4m3_ak_bk_256x256x128_w2x4_m16_pp", DT_F8),
    HT_PP_BN("bf16_ak_bn_256x256x64_w2x4_m16_pp", DT_BF16),
    HT_PP_BN("f16_ak_bn_256x256x64_w2x4_m16_pp", DT_F16),
};

const KernelEntry* table_pp(int* n) {
  *n = (int)(sizeof(g_pp) / sizeof(g_pp[0]));
  return g_pp;
}

}  // namespace htk
