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

hipError_t launch_sk_fixup(const KParams& p, int out_type, hipStream_t s) {
  if (p.sk_tiles <= 0) return hipSuccess;
  const int64_t area = (int64_t)p.tile_bm * p.tile_bn;
  const dim3 grid((unsigned)p.sk_tiles, (unsigned)min((area + 255) / 256, (int64_t)32));
  switch (out_type) {
    case DT_F32: hipLaunchKernelGGL(gemm_sk_fixup<DT_F32>, grid, dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL(gemm_sk_fixup<DT_F16>, grid, dim3(256), 0, s, p); break;
    case DT_BF16: hipLaunchKernelGGL(gemm_sk_fixup<DT_BF16>, grid, dim3(256), 0, s, p); break;
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

// Grouped tile table: two block-wide scans over the G + 1 offsets (a running maximum, then a
// sum of tile counts), each thread taking a contiguous run of entries.
__global__ __launch_bounds__(1024) void gemm_group_scan(const int32_t* off, int G, int M, int bm,
                                                       int tiles_n, int32_t* lo, int64_t* base) {
  __shared__ int smax[1024];
  __shared__ int64_t ssum[1024];
  const int t = threadIdx.x;
  const int per = (G + 1 + 1023) / 1024;
  const int b = min(t * per, G + 1), e = min(b + per, G + 1);
  int m = 0;
  for (int i = b; i < e; ++i) m = max(m, off[i]);
  smax[t] = m;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive scan of the chunk maxima
    const int v = t >= d ? smax[t - d] : 0;
    __syncthreads();
    smax[t] = max(smax[t], v);
    __syncthreads();
  }
  int run = t > 0 ? smax[t - 1] : 0;      // running maximum before this chunk
  int prev = min(run, M);                 // effective offset of the entry before this chunk
  int64_t sum = 0;                        // tiles of the groups that end in this chunk
  for (int i = b; i < e; ++i) {
    run = max(run, off[i]);
    const int eff = min(run, M);
    lo[i] = eff;
    if (i > 0) sum += (int64_t)((eff - prev + bm - 1) / bm) * tiles_n;
    prev = eff;
  }
  ssum[t] = sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive scan of the chunk sums
    const int64_t v = t >= d ? ssum[t - d] : 0;
    __syncthreads();
    ssum[t] += v;
    __syncthreads();
  }
  int64_t acc = t > 0 ? ssum[t - 1] : 0;
  prev = b > 0 ? min(smax[t > 0 ? t - 1 : 0], M) : 0;
  for (int i = b; i < e; ++i) {
    const int eff = lo[i];
    if (i > 0) acc += (int64_t)((eff - prev + bm - 1) / bm) * tiles_n;
    base[i] = acc;
    prev = eff;
  }
}

hipError_t launch_group_scan(const int32_t* offsets, int G, int64_t M, int bm, int tiles_n,
                             int32_t* lo, int64_t* base, hipStream_t s) {
  hipLaunchKernelGGL(gemm_group_scan, dim3(1), dim3(1024), 0, s, offsets, G, (int)M, bm, tiles_n,
                     lo, base);
  return hipGetLastError();
}

}  // namespace htk
