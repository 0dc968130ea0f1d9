// repack.hip -- copies an operand that the 16-byte loaders cannot read (a leading dimension or
// base that is not 16-byte aligned, or an fp8 operand that is not K-contiguous) into a K-major,
// 16-byte aligned, zero-padded copy in the caller's workspace, so that the aligned kernels (DMA
// rings, 16-byte loaders) run on it ("CUTLASS" (stanleyjacob.dev), Part II: operands that miss
// the alignment the fast kernels need take a slower path; here that path is one extra pass over
// the operand's bytes, which for the problem sizes where the library chooses it costs far less
// than running the whole product with element-wise loads).
//
// dst[r * Kp + k] = src(r, k) for k < K and 0 for K <= k < Kp, with src(r, k) at element offset
// r * s_row + k * s_k.  A workgroup moves a 64 x 64 tile through LDS: reads walk the source's
// contiguous direction (neighbouring lanes, neighbouring elements), writes are 16-byte row chunks
// of dst.  Bound by HBM: each source byte is read once and each destination byte written once.
#include "kernels.h"

namespace htk {

struct RepackParams {
  const void* src;
  void* dst;
  int64_t rows, K, Kp;     // dst is rows x Kp
  int64_t s_row, s_k;      // source element strides
};

template <int SZ, bool KCONTIG>
__global__ __launch_bounds__(256) void gemm_repack_kernel(const RepackParams p) {
  typedef typename std::conditional<SZ == 1, uint8_t, typename std::conditional<SZ == 2, uint16_t, uint32_t>::type>::type T;
  constexpr int TILE = 64, VE = 16 / SZ;
  __shared__ T tile[TILE][TILE + 4 / SZ];  // one dword of padding per row
  const int64_t r0 = (int64_t)blockIdx.y * TILE, k0 = (int64_t)blockIdx.x * TILE;
  const T* src = (const T*)p.src;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TILE * TILE / 256; ++i) {
    const int q = tid + 256 * i;
    const int a = q / TILE, b = q % TILE;   // b along the source's contiguous direction
    const int r = KCONTIG ? a : b, k = KCONTIG ? b : a;
    const int64_t gr = r0 + r, gk = k0 + k;
    tile[r][k] = gr < p.rows && gk < p.K ? src[gr * p.s_row + gk * p.s_k] : T(0);
  }
  __syncthreads();
  constexpr int CPR = TILE / VE;  // 16-byte chunks per tile row
#pragma unroll
  for (int i = 0; i < TILE * CPR / 256; ++i) {
    const int q = tid + 256 * i;
    const int r = q / CPR, c = q % CPR;
    const int64_t gr = r0 + r, gk = k0 + c * VE;
    if (gr >= p.rows || gk >= p.Kp) continue;
    u32x4 v = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < VE; ++e) v[e * SZ / 4] |= (u32)tile[r][c * VE + e] << (8 * ((e * SZ) % 4));
    *(u32x4*)((char*)p.dst + (gr * p.Kp + gk) * SZ) = v;
  }
}

// 2-byte elements, K-contiguous source at any element alignment: each thread writes one 16-byte
// chunk of dst from the realigned 16 bytes (plus the next dword) of the source row, elements at
// k >= K cleared; no LDS.  The descriptor spans the whole source rounded up to a dword.
__device__ __forceinline__ void repack_rows16(const RepackParams& p, int64_t bx) {
  const int64_t cpr = p.Kp / 8;                              // chunks per dst row
  const int64_t q = bx * 256 + threadIdx.x;
  if (q >= p.rows * cpr) return;
  const int64_t r = q / cpr, c = q - r * cpr;
  const char* base = (const char*)((uintptr_t)p.src & ~uintptr_t(3));
  const uint32_t delta = (uint32_t)((const char*)p.src - base);
  const int64_t ext = (delta + ((p.rows - 1) * p.s_row + p.K) * 2 + 3) & ~int64_t(3);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, ext);
  const int64_t k = c * 8;
  const uint32_t off = delta + (uint32_t)((r * p.s_row + k) * 2);
  const uint32_t emask = k >= p.K ? 0u : (k + 8 <= p.K ? 0xffu : ((1u << (p.K - k)) - 1u));
  const Raw16 w = raw16(rsrc, emask ? (off & ~3u) : kOobOffset);
  *(u32x4*)((char*)p.dst + (r * p.Kp + k) * 2) = realign16(w, off & 2u, emask);
}
__global__ __launch_bounds__(256) void gemm_repack_rows16(const RepackParams p) {
  repack_rows16(p, blockIdx.x);
}

// 2-byte elements, row-contiguous source (element (r, k) at r + k * s_k) at any alignment: a
// 64 (k) x 64 (r) tile is read as realigned 16-byte chunks of 8 consecutive r at one k, written
// into LDS transposed (element by element), and stored as 16-byte chunks of dst rows.
constexpr int kColsTile = 64, kColsPitch = kColsTile + 2;  // LDS row = one r, 64 k values
__device__ __forceinline__ void repack_cols16(const RepackParams& p, int64_t bx, int64_t by,
                                              uint16_t (*tile)[kColsPitch]) {
  constexpr int TILE = kColsTile;
  const int64_t r0 = by * TILE, k0 = bx * TILE;
  const char* base = (const char*)((uintptr_t)p.src & ~uintptr_t(3));
  const uint32_t delta = (uint32_t)((const char*)p.src - base);
  const int64_t ext = (delta + ((p.K - 1) * p.s_k + p.rows) * 2 + 3) & ~int64_t(3);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, ext);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;        // 512 chunks: 64 k rows x 8 chunks of 8 r
    const int kk = q / 8, rc = q % 8;
    const int64_t gk = k0 + kk, gr = r0 + rc * 8;
    const uint32_t off = delta + (uint32_t)((gk * p.s_k + gr) * 2);
    const uint32_t emask = gk >= p.K || gr >= p.rows ? 0u
                           : (gr + 8 <= p.rows ? 0xffu : ((1u << (p.rows - gr)) - 1u));
    const Raw16 w = raw16(rsrc, emask ? (off & ~3u) : kOobOffset);
    const u32x4 v = realign16(w, off & 2u, emask);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[rc * 8 + e][kk] = (uint16_t)(v[e / 2] >> (16 * (e % 2)));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;        // 512 chunks: 64 dst rows x 8 chunks of 8 k
    const int r = q / 8, c = q % 8;
    const int64_t gr = r0 + r, gk = k0 + c * 8;
    if (gr >= p.rows || gk >= p.Kp) continue;
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = (u32)tile[r][c * 8 + 2 * d] | ((u32)tile[r][c * 8 + 2 * d + 1] << 16);
    *(u32x4*)((char*)p.dst + (gr * p.Kp + gk) * 2) = v;
  }
}
__global__ __launch_bounds__(256) void gemm_repack_cols16(const RepackParams p) {
  __shared__ uint16_t tile[kColsTile][kColsPitch];
  repack_cols16(p, blockIdx.x, blockIdx.y, tile);
}

// Both operands of a product in one launch (2-byte elements, each source K- or row-contiguous):
// workgroups [0, na) copy the first operand, the rest the second, so the two copies share the
// GPU instead of running one after the other.  kind 0: realigned row copy (K-contiguous source),
// 1: LDS transpose (row-contiguous source).
struct RepackJob {
  RepackParams p;
  int kind;
  int64_t gx;      // workgroups along K (transposes: the grid's x extent)
  int64_t blocks;  // workgroups of this job
};
__global__ __launch_bounds__(256) void gemm_repack_pair16(const RepackJob a, const RepackJob b) {
  __shared__ uint16_t tile[kColsTile][kColsPitch];
  const int64_t x = blockIdx.x;
  const bool first = x < a.blocks;
  const RepackJob& j = first ? a : b;
  const int64_t l = first ? x : x - a.blocks;
  if (j.kind == 0) repack_rows16(j.p, l);
  else repack_cols16(j.p, l % j.gx, l / j.gx, tile);
}

namespace {
// The pair kernel's job for one operand, or kind -1 when it needs the generic copy.
RepackJob job16(const void* src, void* dst, int64_t rows, int64_t K, int64_t Kp, int64_t s_row,
                int64_t s_k) {
  RepackJob j{{src, dst, rows, K, Kp, s_row, s_k}, -1, 0, 0};
  const bool kc = s_k == 1;
  const int64_t span = kc ? (rows - 1) * s_row + K : (K - 1) * s_k + rows;
  if (rows <= 0 || Kp <= 0 || span * 2 >= (int64_t(1) << 31) - 64) return j;
  if (kc) {
    j.kind = 0;
    j.blocks = (rows * (Kp / 8) + 255) / 256;
  } else if (s_row == 1) {
    j.kind = 1;
    j.gx = (Kp + 63) / 64;
    j.blocks = j.gx * ((rows + 63) / 64);
  }
  return j;
}
}  // namespace

hipError_t launch_repack_pair(const void* a_src, void* a_dst, int64_t a_rows, int64_t a_srow,
                              int64_t a_sk, const void* b_src, void* b_dst, int64_t b_rows,
                              int64_t b_srow, int64_t b_sk, int64_t K, int64_t Kp, int esize,
                              hipStream_t s) {
  if (esize == 2) {
    const RepackJob a = a_src ? job16(a_src, a_dst, a_rows, K, Kp, a_srow, a_sk) : RepackJob{{}, 0, 1, 0};
    const RepackJob b = b_src ? job16(b_src, b_dst, b_rows, K, Kp, b_srow, b_sk) : RepackJob{{}, 0, 1, 0};
    if (a.kind >= 0 && b.kind >= 0 && a.blocks + b.blocks > 0) {
      hipLaunchKernelGGL(gemm_repack_pair16, dim3((unsigned)(a.blocks + b.blocks)), dim3(256), 0, s, a, b);
      return hipGetLastError();
    }
  }
  hipError_t err = hipSuccess;
  if (a_src) err = launch_repack(a_src, a_dst, a_rows, K, Kp, a_srow, a_sk, esize, s);
  if (err == hipSuccess && b_src) err = launch_repack(b_src, b_dst, b_rows, K, Kp, b_srow, b_sk, esize, s);
  return err;
}

hipError_t launch_repack(const void* src, void* dst, int64_t rows, int64_t K, int64_t Kp,
                         int64_t s_row, int64_t s_k, int esize, hipStream_t s) {
  if (rows <= 0 || Kp <= 0) return hipSuccess;
  RepackParams p{src, dst, rows, K, Kp, s_row, s_k};
  const dim3 grid((unsigned)((Kp + 63) / 64), (unsigned)((rows + 63) / 64));
  const bool kc = s_k == 1;
  // the realigned 16-byte paths address the source with 32-bit offsets
  const int64_t span = kc ? (rows - 1) * s_row + K : (K - 1) * s_k + rows;
  if (esize == 2 && span * 2 < (int64_t(1) << 31) - 64) {
    if (kc) {
      const int64_t chunks = rows * (Kp / 8);
      hipLaunchKernelGGL(gemm_repack_rows16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, p);
      return hipGetLastError();
    }
    if (s_row == 1) {
      hipLaunchKernelGGL(gemm_repack_cols16, grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  switch (esize * 2 + (kc ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((gemm_repack_kernel<1, false>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((gemm_repack_kernel<1, true>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_repack_kernel<2, false>), grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL((gemm_repack_kernel<2, true>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_repack_kernel<4, false>), grid, dim3(256), 0, s, p); break;
    case 9: hipLaunchKernelGGL((gemm_repack_kernel<4, true>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace htk
