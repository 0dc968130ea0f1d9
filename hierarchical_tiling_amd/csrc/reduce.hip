// reduce.hip -- launcher of the split-K reduction (the second kernel of a split-K run).
#include "kernels.h"

namespace htk {

hipError_t launch_splitk_reduce(const KParams& p, int out_type, hipStream_t s) {
  const int64_t mn = p.M * p.N;
  const unsigned blocks = (unsigned)min((mn + 255) / 256, (int64_t)4096);
  if (blocks == 0) return hipSuccess;
  switch (out_type) {
    case DT_F32: hipLaunchKernelGGL(gemm_splitk_reduce<DT_F32>, dim3(blocks), dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL(gemm_splitk_reduce<DT_F16>, dim3(blocks), dim3(256), 0, s, p); break;
    case DT_BF16: hipLaunchKernelGGL(gemm_splitk_reduce<DT_BF16>, dim3(blocks), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace htk
