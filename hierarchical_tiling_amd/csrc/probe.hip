// probe.hip -- the index probe: runs one MFMA atom on the device and reports where the hardware
// put each value, so that the atoms' layouts (atom_maps.h) can be compared bit for bit with the
// layout helper's evaluation of the same layouts ("A10 - CuTe, CUTLASS & CuTile", section 3.3:
// the (thread, value) -> (m, n) map of a fragment; section 6 Pitfall 2: fragment bugs are
// silent, so the map is checked directly).  One wave; every index stays inside the atom's tile.
#include "../../include/htgemm.h"
#include "kernels.h"

namespace htk {

namespace {

// Element bits of the small values the probe uses: 0 and powers of two up to 32 (exact in every
// operand type).
template <int DT> __device__ uint32_t enc(int v) {
  if (v == 0) return 0;
  int e = 0;
  while ((1 << e) < v) ++e;
  if constexpr (DT == DT_F32) return (uint32_t)(127 + e) << 23;
  if constexpr (DT == DT_F16) return (uint32_t)(15 + e) << 10;
  if constexpr (DT == DT_BF16) return (uint32_t)(127 + e) << 7;
  return (uint32_t)(7 + e) << 3;  // OCP e4m3
}

// Place element bits `bits` at element position `e` of a run of 16-byte chunks.
template <int DT> __device__ void put(u32x4* chunks, int e, uint32_t bits) {
  constexpr int SZ = Ty<DT>::SZ, PER = 4 / SZ;  // elements per dword
  const int dw = e / PER, sh = (e % PER) * 8 * SZ;
  u32x4& c = chunks[dw / 4];
  c[dw % 4] |= bits << sh;
}

// Inputs that encode the output position in D: A(m, k) and B(k, n) non-zero for k < 10 only,
// with D(m, n) = sum over k of A B = m + 32 n exactly.
__device__ int a_val(int m, int k) { return k < 5 ? ((m >> k) & 1) : (k < 10 ? 32 : 0); }
__device__ int b_val(int k, int n) { return k < 5 ? (1 << k) : (k < 10 ? ((n >> (k - 5)) & 1) << (k - 5) : 0); }

template <int DT, int MI>
__global__ __launch_bounds__(64) void gemm_probe_kernel(int32_t* out) {
  typedef Atom<DT, MI> At;
  typedef typename At::acc_t acc_t;
  typedef Maps<DT, MI> Mp;
  constexpr int SZ = Ty<DT>::SZ, VE = 16 / SZ, CH = 8, BKE = CH * VE;
  constexpr int G = At::G, UPL = CH / G, S = UPL / At::UNITS, VPL = Mp::M.vpl, NACC = At::NACC;
  __shared__ u32x4 As[MI * CH], Bs[MI * CH];
  __shared__ int stat[4];
  const int lane = threadIdx.x;
  for (int i = lane; i < GEMM_PROBE_INTS; i += 64) out[i] = -2;

  // ---- accumulator map through the kernels' LDS tiles, swizzle and fragment addressing ----
  for (int q = lane; q < MI * CH; q += 64) {
    const int row = q / CH, c = q % CH;
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    for (int e = 0; e < VE; ++e) {
      const int k = c * VE + e;
      put<DT>(&a, e, enc<DT>(a_val(row, k)));
      put<DT>(&b, e, enc<DT>(b_val(k, row)));
    }
    As[lds_slot<CH>(row, c)] = a;
    Bs[lds_slot<CH>(row, c)] = b;
  }
  __syncthreads();
  static_assert(BKE >= 10, "one k-tile holds every non-zero k");
  const int frow = frag_row<DT, MI>(lane), fgrp = frag_chunk<DT, MI>(lane);
  acc_t acc = acc_t{};
  static_for<S>([&](auto sub) {
    u32x4 fa[At::UNITS], fb[At::UNITS];
    static_for<At::UNITS>([&](auto x) {
      const int c = fgrp + G * (sub * At::UNITS + x);
      fa[x] = As[lds_slot<CH>(frow, c)];
      fb[x] = Bs[lds_slot<CH>(frow, c)];
    });
    static_for<At::PER_UNIT>([&](auto u) { At::mma(acc, fa, fb, u); });
  });
  static_for<NACC>([&](auto r) {
    const int d = (int)acc[(int)r];
    out[lane + 64 * r] = d % 32 + MI * (d / 32);
    out[2048 + lane + 64 * r] = acc_row<DT, MI>(lane, r) + MI * acc_col<DT, MI>(lane, r);
  });

  // ---- operand slots: one-hot A in slot (L, V) ----
  const uint32_t one = enc<DT>(1);
  u32x4 ones[At::UNITS];
  static_for<At::UNITS>([&](auto x) {
    ones[x] = u32x4{0, 0, 0, 0};
    for (int e = 0; e < VE; ++e) put<DT>(&ones[x], e, one);
  });
  for (int L = 0; L < 64; ++L) {
    for (int V = 0; V < VPL; ++V) {
      u32x4 fa[At::UNITS];
      static_for<At::UNITS>([&](auto x) { fa[x] = u32x4{0, 0, 0, 0}; });
      if (lane == L) put<DT>(fa, V, one);
      const int kL = lane_offset(Mp::M.op, L) / MI + value_offset(Mp::M.op, V) / MI;
      for (int pass = 0; pass < 2; ++pass) {
        // pass 0: B all ones; pass 1: B one exactly in the slots labelled with A's k
        u32x4 fb[At::UNITS];
        if (pass == 0) {
          static_for<At::UNITS>([&](auto x) { fb[x] = ones[x]; });
        } else {
          static_for<At::UNITS>([&](auto x) { fb[x] = u32x4{0, 0, 0, 0}; });
          for (int v = 0; v < VPL; ++v)
            if (lane_offset(Mp::M.op, lane) / MI + value_offset(Mp::M.op, v) / MI == kL) put<DT>(fb, v, one);
        }
        if (lane == 0) { stat[0] = 1 << 30; stat[1] = -1; stat[2] = 0; stat[3] = 0; }
        __syncthreads();
        acc_t d = acc_t{};
        At::mma(d, fa, fb, 0);
        static_for<NACC>([&](auto r) {
          const float v = d[(int)r];
          if (v != 0.f) {
            atomicMin(&stat[0], acc_row<DT, MI>(lane, r));
            atomicMax(&stat[1], acc_row<DT, MI>(lane, r));
            atomicAdd(&stat[2], v == 1.f ? 1 : 1000);
          }
        });
        __syncthreads();
        if (lane == 0) {
          const bool one_row = stat[0] == stat[1];
          if (pass == 0) out[4096 + L + 64 * V] = one_row && stat[2] == MI ? stat[0] : -1;
          else out[6144 + L + 64 * V] = one_row && stat[2] <= MI ? stat[2] : -1;
        }
        __syncthreads();
      }
    }
  }
}

template <int DT, int MI> hipError_t launch_probe(int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL((gemm_probe_kernel<DT, MI>), dim3(1), dim3(64), 0, s, out);
  return hipGetLastError();
}

}  // namespace

}  // namespace htk

extern "C" int gemm_probe_atom(int dtype, int mi, int32_t* out, void* stream) {
  using namespace htk;
  if (!out || (mi != 16 && mi != 32)) return GEMM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (dtype * 2 + (mi == 32)) {
    case DT_F32 * 2: e = launch_probe<DT_F32, 16>(out, s); break;
    case DT_F32 * 2 + 1: e = launch_probe<DT_F32, 32>(out, s); break;
    case DT_F16 * 2: e = launch_probe<DT_F16, 16>(out, s); break;
    case DT_F16 * 2 + 1: e = launch_probe<DT_F16, 32>(out, s); break;
    case DT_BF16 * 2: e = launch_probe<DT_BF16, 16>(out, s); break;
    case DT_BF16 * 2 + 1: e = launch_probe<DT_BF16, 32>(out, s); break;
    case DT_F8 * 2: e = launch_probe<DT_F8, 16>(out, s); break;
    case DT_F8 * 2 + 1: e = launch_probe<DT_F8, 32>(out, s); break;
    default: return GEMM_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}
