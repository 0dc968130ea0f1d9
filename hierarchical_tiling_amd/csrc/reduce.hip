// reduce.hip -- second kernels: the split-K and split-tail reductions, and the fixed-order sum of
// the row sums-of-squares partials.
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

hipError_t launch_tail_reduce(const KParams& p, int out_type, hipStream_t s) {
  if (p.tail_tiles <= 0) return hipSuccess;
  const int64_t area = (int64_t)p.tile_bm * p.tile_bn;
  const dim3 grid((unsigned)p.tail_tiles, (unsigned)min((area + 255) / 256, (int64_t)32));
  switch (out_type) {
    case DT_F32: hipLaunchKernelGGL(gemm_tail_reduce<DT_F32>, grid, dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL(gemm_tail_reduce<DT_F16>, grid, dim3(256), 0, s, p); break;
    case DT_BF16: hipLaunchKernelGGL(gemm_tail_reduce<DT_BF16>, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// out[m] = sum of the tiles_n partials of row m, in plane order.
__global__ __launch_bounds__(256) void gemm_row_sumsq_reduce(const float* ws, float* out,
                                                               int64_t M, int tiles_n) {
  for (int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x; m < M; m += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int t = 0; t < tiles_n; ++t) s += ws[t * M + m];
    out[m] = s;
  }
}

hipError_t launch_row_sumsq_reduce(const float* ws, float* out, int64_t M, int tiles_n,
                                   hipStream_t s) {
  const unsigned blocks = (unsigned)min((M + 255) / 256, (int64_t)1024);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_row_sumsq_reduce, dim3(blocks), dim3(256), 0, s, ws, out, M, tiles_n);
  return hipGetLastError();
}

}  // namespace htk
