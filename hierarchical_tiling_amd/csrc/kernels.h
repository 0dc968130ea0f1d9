// kernels.h -- gfx950 (MI355X, CDNA4) kernels of the hierarchically tiled GEMM.  The table_*.hip
// files instantiate them per operand type (one translation unit each, so they build in parallel).
//
//   D = act(alpha * (A @ B) + beta * C + bias),  fp32 accumulation.
//
// The decomposition follows the pages' tile hierarchy ("CUTLASS", stanleyjacob.dev, Part I
// "The mental model" and Part IV "The full life of one GEMM"; "A10 - CuTe, CUTLASS & CuTile",
// section 3.2): the output is cut into workgroup tiles (BM x BN) that stream K in BK steps
// through LDS; each wave owns a wave tile held in accumulator registers; each wave tile is a
// grid of MFMA atoms.  What is MI355X-specific here:
//
//  * Atoms are CDNA4 MFMA instructions on 64-lane waves: v_mfma_f32_32x32x16_{bf16,f16},
//    v_mfma_f32_32x32x64_f8f6f4 (OCP e4m3), v_mfma_f32_32x32x2_f32 and their 16x16 forms.
//    For each atom, lane l holds row (l % MI) of the A tile and column (l % MI) of the B tile,
//    and a contiguous run of k; A and B place the same k in the same lane slot, so the k order
//    inside an atom never matters.  The 32x32 accumulator holds, in register r of lane l,
//    row 8*(r/4) + 4*(l/32) + r%4 and column l % 32; the 16x16 one row 4*(l/16) + r.
//  * LDS tiles are stored K-contiguous: one row per m (for A) or n (for B), BK*esize = 128
//    bytes, i.e. eight 16-byte chunks.  Chunk c of row r lives at chunk slot c ^ (r & 7): the
//    XOR swizzle of "A10", section 3.4 (Swizzle<3,4,3> in byte addressing), which puts the
//    eight rows that one ds_read_b128 phase reads at the same logical chunk into eight
//    different 16-byte bank groups, and also makes the row-wise 16-byte stores conflict free.
//  * The K mainloop is double buffered ("CUTLASS", Part IV Stage 4): the global loads of
//    k-tile t+1 are issued into registers before the MFMAs of tile t, and written into the other
//    LDS stage after them, with one barrier per k-tile ("CuTe DSL / CUDA Tile" post, "Pipelining
//    hides a wait": the slower of load and compute sets the interval).
//  * Workgroup ids are remapped so that each of the 8 XCDs (each with its own L2) gets a
//    contiguous range of tiles, walked in groups of GROUP_M tile rows ("CUTLASS", Part IV
//    Stage 2: the tile scheduler swizzles the grid for L2 reuse).
//  * Edges: rows past M or N are clamped to the last valid row on load (their results are never
//    stored), the K tail is zero-filled, and stores are predicated.  MFMA issue is never
//    predicated: it is wave-wide, so every lane always executes it ("A10", section 6,
//    Pitfall 1: guards around a collective matrix instruction must be uniform).
//  * A narrow-load variant reads element by element with full predication, for leading
//    dimensions or pointers that are not 16-byte aligned ("CUTLASS", Part II: misaligned
//    operands fall back to a slow path).
//  * The epilogue applies alpha, beta*C, bias[n] and the activation in fp32 on the accumulator
//    registers and rounds to the output type once ("CUTLASS", Part IV Stage 5).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "atom_maps.h"
#include "gemm_internal.h"

namespace htk {

typedef uint8_t u8;
typedef uint16_t u16;
typedef uint32_t u32;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// Element types
// ------------------------------------------------------------------------------------------
template <int DT> struct Ty;
template <> struct Ty<DT_F32> { typedef u32 T; static constexpr int SZ = 4; typedef float O; };
template <> struct Ty<DT_F16> { typedef u16 T; static constexpr int SZ = 2; typedef u16 O; };
template <> struct Ty<DT_BF16> { typedef u16 T; static constexpr int SZ = 2; typedef u16 O; };
template <> struct Ty<DT_F8> { typedef u8 T; static constexpr int SZ = 1; typedef u16 O; };

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __builtin_bit_cast(float, u32(b) << 16); }
__device__ __forceinline__ float f16_to_f32(u16 h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ u16 f32_to_bf16(float x) { return __builtin_bit_cast(u16, (__bf16)x); }
__device__ __forceinline__ u16 f32_to_f16(float x) { return __builtin_bit_cast(u16, (_Float16)x); }

// Output (C, D, bias) element access by output dtype.
template <int ODT> struct Out;
template <> struct Out<DT_F32> {
  __device__ static float load(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
  __device__ static float from_bits(u32 b) { return __builtin_bit_cast(float, b); }
};
template <> struct Out<DT_F16> {
  __device__ static float load(const void* p, int64_t i) { return f16_to_f32(((const u16*)p)[i]); }
  __device__ static void store(void* p, int64_t i, float v) { ((u16*)p)[i] = f32_to_f16(v); }
  __device__ static float from_bits(u32 b) { return f16_to_f32((u16)b); }
};
template <> struct Out<DT_BF16> {
  __device__ static float load(const void* p, int64_t i) { return bf16_to_f32(((const u16*)p)[i]); }
  __device__ static void store(void* p, int64_t i, float v) { ((u16*)p)[i] = f32_to_bf16(v); }
  __device__ static float from_bits(u32 b) { return bf16_to_f32((u16)b); }
};

// Compile-time loop: the body sees its index as a constant, so register arrays indexed by it
// stay in registers (a runtime index would force the array into scratch memory).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Output element bits.
template <int ODT> struct OutBits { typedef u16 T; };
template <> struct OutBits<DT_F32> { typedef u32 T; };
__device__ __forceinline__ u16 to_bits(float v, std::integral_constant<int, DT_BF16>) { return f32_to_bf16(v); }
__device__ __forceinline__ u16 to_bits(float v, std::integral_constant<int, DT_F16>) { return f32_to_f16(v); }
__device__ __forceinline__ u32 to_bits(float v, std::integral_constant<int, DT_F32>) { return __builtin_bit_cast(u32, v); }

// ------------------------------------------------------------------------------------------
// MFMA atoms.  G: lane groups along k (64 / MI); UNITS: 16-byte chunks per lane per operand per
// instruction; PER_UNIT: instructions fed by one chunk; NACC: accumulator floats per lane.
// ------------------------------------------------------------------------------------------
template <int DT, int MI> struct Atom;

template <> struct Atom<DT_BF16, 32> {
  static constexpr int G = 2, UNITS = 1, PER_UNIT = 1, NACC = 16;
  typedef f32x16 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
template <> struct Atom<DT_BF16, 16> {
  static constexpr int G = 4, UNITS = 1, PER_UNIT = 1, NACC = 4;
  typedef f32x4 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
template <> struct Atom<DT_F16, 32> {
  static constexpr int G = 2, UNITS = 1, PER_UNIT = 1, NACC = 16;
  typedef f32x16 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                               __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
  }
};
template <> struct Atom<DT_F16, 16> {
  static constexpr int G = 4, UNITS = 1, PER_UNIT = 1, NACC = 4;
  typedef f32x4 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[0]),
                                               __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
  }
};
// fp8: format code 0 selects OCP E4M3 for both operands; scale operands left neutral (0).
template <> struct Atom<DT_F8, 32> {
  static constexpr int G = 2, UNITS = 2, PER_UNIT = 1, NACC = 16;
  typedef f32x16 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    i32x8 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
    i32x8 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  }
};
template <> struct Atom<DT_F8, 16> {
  static constexpr int G = 4, UNITS = 2, PER_UNIT = 1, NACC = 4;
  typedef f32x4 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int) {
    i32x8 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
    i32x8 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  }
};
template <> struct Atom<DT_F32, 32> {
  static constexpr int G = 2, UNITS = 1, PER_UNIT = 4, NACC = 16;
  typedef f32x16 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int sub) {
    // Bit-cast the whole chunk, then pick the element: this compiler folds a scalar bit-cast
    // of an extracted u32 vector element to element 0.
    const f32x4 av = __builtin_bit_cast(f32x4, a[0]), bv = __builtin_bit_cast(f32x4, b[0]);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[sub], bv[sub], c, 0, 0, 0);
  }
};
template <> struct Atom<DT_F32, 16> {
  static constexpr int G = 4, UNITS = 1, PER_UNIT = 4, NACC = 4;
  typedef f32x4 acc_t;
  __device__ static void mma(acc_t& c, const u32x4* a, const u32x4* b, int sub) {
    const f32x4 av = __builtin_bit_cast(f32x4, a[0]), bv = __builtin_bit_cast(f32x4, b[0]);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(av[sub], bv[sub], c, 0, 0, 0);
  }
};

// Positions taken from the atom's layouts (atom_maps.h), so the kernels' fragment addressing and
// accumulator placement are the layout functions the host checks against the layout helper and
// the index probe checks against the hardware.
template <int DT, int MI> struct Maps {
  static constexpr int idx = atom_index(DT, MI);
  static_assert(idx >= 0, "no layout for this atom");
  static constexpr AtomMaps M = kAtomMaps[idx];
  // values of one lane's contiguous k run per instruction (16 bytes, or one f32)
  static constexpr int RUN = M.vpl < 16 / dtype_size(DT) ? M.vpl : 16 / dtype_size(DT);
  // the accumulator registers of a lane all lie in one column (offsets of the value modes stay
  // below MI), so the column of a lane's accumulators is taken once per lane
  static constexpr bool one_column() {
    for (int r = 0; r < M.nacc; ++r)
      if (value_offset(M.acc, r) >= MI) return false;
    return true;
  }
  static_assert(one_column(), "accumulator values of a lane span one column");
};
// Offset of layout WHICH (0: operand, 1: accumulator) of atom IDX at a lane, with the shape and
// stride as compile-time constants: a sum of ((l / P_i) % S_i) * D_i over the lane modes (P_i the
// product of the shapes before mode i).
template <int IDX, int WHICH> struct LaneOffset {
  static constexpr const AtomLayout& L() { return WHICH == 0 ? kAtomMaps[IDX].op : kAtomMaps[IDX].acc; }
  static constexpr int prod(int i) {
    int p = 1;
    for (int j = 0; j < i; ++j) p *= L().shape[j];
    return p;
  }
  template <int I> __device__ static __forceinline__ int term(unsigned l) {
    constexpr int P = prod(I);
    if constexpr (I >= L().n || P >= 64) return 0;  // past the lane modes
    else return (int)((l / (unsigned)P) % (unsigned)L().shape[I]) * L().stride[I];
  }
  __device__ static __forceinline__ int at(unsigned l) {
    return term<0>(l) + term<1>(l) + term<2>(l) + term<3>(l);
  }
};
template <int DT, int MI> struct MapRefs {
  typedef LaneOffset<atom_index(DT, MI), 0> op;
  typedef LaneOffset<atom_index(DT, MI), 1> acc;
};
// Row (within the MI x MI block) and column of accumulator register r of lane l.
template <int DT, int MI, class R> __device__ __forceinline__ int acc_row(int l, R) {
  constexpr int vo = value_offset(Maps<DT, MI>::M.acc, R::value);
  const int lo = MapRefs<DT, MI>::acc::at((unsigned)l);
  return (int)((unsigned)(lo + vo) % (unsigned)MI);
}
template <int DT, int MI, class R> __device__ __forceinline__ int acc_col(int l, R) {
  constexpr int vo = value_offset(Maps<DT, MI>::M.acc, R::value);
  const int lo = MapRefs<DT, MI>::acc::at((unsigned)l);
  return (int)((unsigned)(lo + vo) / (unsigned)MI);
}
// Operand fragments: the row of A (column of B) lane l supplies, and the 16-byte chunk of an LDS
// row holding the start of its first k run (chunks of later runs and substeps follow every
// 64 / MI chunks).
template <int DT, int MI> __device__ __forceinline__ int frag_row(int l) {
  const int lo = MapRefs<DT, MI>::op::at((unsigned)l);
  return (int)((unsigned)lo % (unsigned)MI);
}
template <int DT, int MI> __device__ __forceinline__ int frag_chunk(int l) {
  const int lo = MapRefs<DT, MI>::op::at((unsigned)l);
  return (int)((unsigned)lo / (unsigned)(MI * Maps<DT, MI>::RUN));
}

// ------------------------------------------------------------------------------------------
// Workgroup -> output tile.  Dispatch hands consecutive workgroup ids to the 8 XCDs in turn;
// the remap gives XCD x the contiguous tile range [start(x), start(x) + count(x)), and tiles
// are walked GROUP_M tile rows at a time so concurrently resident neighbours share A and B.
// A split-tail launch covers the tile order from p.tile_base on.
// ------------------------------------------------------------------------------------------
// Tile t of the tile order: GROUP_M tile rows at a time, column by column within a group.
__device__ __forceinline__ void tile_walk(const KParams& p, int t, int& tm, int& tn) {
  const int width = p.group_m * p.tiles_n;
  const int group = t / width;
  const int first = group * p.group_m;
  const int gsz = min(p.tiles_m - first, p.group_m);
  const int within = t - group * width;
  tm = first + within % gsz;
  tn = within / gsz;
}
__device__ __forceinline__ void tile_of(const KParams& p, int pid, int nwg, int& tm, int& tn) {
  const int per = nwg >> 3, extra = nwg & 7;
  const int xcd = pid & 7, local = pid >> 3;
  tile_walk(p, xcd * per + min(xcd, extra) + local + p.tile_base, tm, tn);
}

// ReLU that keeps NaN (max(0, NaN) is NaN, as in the oracle's definition).
__device__ __forceinline__ float relu(float v) { return v > 0.f ? v : (v == v ? 0.f : v); }

// GELU(x) = x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, the exact (erf) form.  erf is taken
// from Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26 (Hastings):
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1 / (1 + p z),  z >= 0,
// with |error| <= 1.5e-7, and erf(-z) = -erf(z).  With z = |x| / sqrt 2 the upper tail is
//   q = (1 - erf(z)) / 2 = t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) / 2 * 2^(-x^2 log2(e) / 2),
// and Phi(x) = 1 - q for x >= 0, q for x < 0.  Halved coefficients, folded constants and the
// hardware reciprocal and base-2 exponential (each within 1 ulp) keep it to 12 plain and two
// transcendental instructions with no branches; the error stays near the formula's 1.5e-7, far
// below the 2^-9 (bf16) / 2^-12 (fp16) output rounding.
__device__ __forceinline__ float gelu(float x) {
  const float t = __builtin_amdgcn_rcpf(
      __builtin_fmaf(0.3275911f * 0.70710678118654752f, __builtin_fabsf(x), 1.0f));
  float h = __builtin_fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  h = __builtin_fmaf(h, t, 0.5f * 1.421413741f);
  h = __builtin_fmaf(h, t, 0.5f * -0.284496736f);
  h = __builtin_fmaf(h, t, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(x * x * (-0.5f * 1.4426950408889634f));
  const float q = h * t * e;
  return x * (x >= 0.f ? 1.0f - q : q);
}

// SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), with the hardware base-2 exponential and reciprocal
// (each within 1 ulp).  For x below about -88, e^-x overflows to infinity and the result is -0,
// where the exact value is below 1e-36 in magnitude.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

__device__ __forceinline__ float activate(int act, float v) {
  if (act == 1) return relu(v);
  if (act == 2) return gelu(v);
  if (act == 3) return silu(v);
  return v;
}

// The problem of a batched launch that this workgroup computes ("CUTLASS, CuTe, and CUDA Tile",
// "Assembling a CUTLASS kernel": the problem shape's fourth mode L is a batch of independent
// problems): problem blockIdx.z moves each operand base by its byte stride; everything else
// (shape, strides, alpha, beta, bias and the scale vectors) is shared.
__device__ __forceinline__ KParams batch_view(const KParams& p) {
  KParams q = p;
  if (p.batch > 1 && !p.offsets && !p.problems) {
    const int64_t z = blockIdx.z;
    q.A = (const char*)p.A + z * p.a_bstride;
    q.B = (const char*)p.B + z * p.b_bstride;
    if (p.has_c) q.C = (const char*)p.C + z * p.c_bstride;
    q.D = (char*)p.D + z * p.d_bstride;
  }
  return q;
}

// The kernel argument read again from the kernarg segment (the kernel's only argument, at offset
// 0).  The pointer passes through an empty asm, so these loads cannot be merged with those made
// at entry: values needed only after the main loop are loaded there instead of occupying SGPRs
// across it.
typedef __attribute__((address_space(4))) const KParams kparams_const_t;
__device__ __forceinline__ KParams reload_args() {
  kparams_const_t* q = (kparams_const_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *(const KParams*)q;
}

// The problem and tile of a workgroup of a tile kernel.  Plain and batched launches: tile
// blockIdx.x of gridDim.x.  A grouped launch with ragged M (mixture-of-experts: "CUTLASS",
// Part V, a grouped GEMM in which each expert is one problem of a batch of differently shaped
// problems) shares A's, C's and D's row space among the groups: group e owns rows
// [lo[e], lo[e+1]) and multiplies them by its own B, and the grid enumerates the tiles of every
// group in order.  lo (the caller's offsets clamped into [0, M] and made non-decreasing) and the
// groups' first tiles come from gemm_group_scan; a workgroup finds its group by binary search.
// Returns false for a workgroup past the last group's tiles (the grid is sized for the most
// tiles any split of M can need); such a workgroup exits before its first barrier.
//
// A grouped launch of independent problems ("CUTLASS", Part III: many problems of irregular
// shapes in one launch) takes every operand, shape and leading dimension from the problem's
// table entry; the strides' directions, the types and the epilogue stay those of the launch.
__device__ __forceinline__ int find_group(const int64_t* base, int G, int64_t x) {
  int e = 0, hi_e = G;  // base[e] <= x < base[hi_e]
  while (hi_e - e > 1) {
    const int mid = (e + hi_e) >> 1;
    if (base[mid] <= x) e = mid; else hi_e = mid;
  }
  return e;
}
template <int BM>
__device__ __forceinline__ bool problem_view(const KParams& in, KParams& p, int& pid, int& nwg) {
  p = batch_view(in);
  pid = blockIdx.x;
  nwg = gridDim.x;
  if (in.problems) {
    const int64_t x = blockIdx.x;
    if (x >= in.group_base[in.batch]) return false;
    const int e = find_group(in.group_base, in.batch, x);
    const GroupProblem& q = in.problems[e];
    p.A = q.A;
    p.B = q.B;
    p.C = in.has_c ? q.C : nullptr;
    p.D = q.D;
    p.bias = q.bias;
    p.M = q.M;
    p.N = q.N;
    p.K = q.K;
    p.k_per_split = (int)q.K;
    p.lda = q.lda;
    p.ldb = q.ldb;
    if (in.c_sn == 1) p.c_sm = q.ldc; else p.c_sn = q.ldc;
    if (in.d_sn == 1) p.d_sm = q.ldd; else p.d_sn = q.ldd;
    p.c_span = q.c_span;
    p.tiles_m = q.tiles_m;
    p.tiles_n = q.tiles_n;
    pid = (int)(x - in.group_base[e]);
    nwg = q.tiles_m * q.tiles_n;
    return true;
  }
  if (!in.offsets) return true;
  const int64_t x = blockIdx.x;
  const int G = in.batch;
  if (x >= in.group_base[G]) return false;
  const int e = find_group(in.group_base, G, x);
  const int lo = in.group_lo[e], hi = in.group_lo[e + 1];
  const int tm = (hi - lo + BM - 1) / BM;
  p.A = (const char*)in.A + lo * in.a_row_bytes;
  p.B = (const char*)in.B + e * in.b_bstride;
  if (in.has_c) {
    p.C = (const char*)in.C + lo * in.c_row_bytes;
    if (in.c_span > 0) p.c_span = in.c_span - lo * in.c_row_bytes;
  }
  p.D = (char*)in.D + lo * in.d_row_bytes;
  if (in.has_row_scale) p.row_scale = in.row_scale + lo;
  p.M = hi - lo;
  p.tiles_m = tm;
  pid = (int)(x - in.group_base[e]);
  nwg = tm * in.tiles_n;
  return true;
}

// Epilogue of one output element (row, col) from its fp32 sum, for the kernels that finish
// element by element: y = act((alpha * row_scale[row] * col_scale[col] * sum + beta * C) + bias).
template <int ODT>
__device__ __forceinline__ float finish_elem(const KParams& p, int64_t row, int64_t col, float sum) {
  typedef Out<ODT> O;
  float v = p.alpha * sum;
  if (p.has_row_scale) v *= p.row_scale[row];
  if (p.has_col_scale) v *= p.col_scale[col];
  if (p.has_c) v += p.beta * O::load(p.C, row * p.c_sm + col * p.c_sn);
  if (p.has_bias) v += O::load(p.bias, col);
  return activate(p.act, v);
}

// ------------------------------------------------------------------------------------------
// Split-K ("CUTLASS", Part III: a problem with too few output tiles to fill the GPU splits its K
// loop across several workgroups, whose partial sums are reduced afterwards).  Workgroup row
// blockIdx.y takes the K slice [k_begin, k_begin + k_len); operand pointers are advanced to
// k_begin so the mainloops see a problem of depth k_len.  Each slice writes its raw fp32 sums to
// its own M x N plane of the workspace; gemm_splitk_reduce adds the planes in a fixed order and
// applies the epilogue, so results do not depend on scheduling.
// ------------------------------------------------------------------------------------------
struct KRange {
  int64_t begin, len;
};
__device__ __forceinline__ KRange k_range(const KParams& p) {
  if (p.split_k <= 1) return {0, p.K};
  const int64_t b = (int64_t)blockIdx.y * p.k_per_split;
  return {b, max((int64_t)0, min((int64_t)p.k_per_split, p.K - b))};
}
// operand base advanced by k elements along K (KMAJ: K is the unit-stride direction)
template <int DT, bool KMAJ>
__device__ __forceinline__ const void* advance_k(const void* base, int64_t ld, int64_t k) {
  return (const char*)base + (KMAJ ? k : k * ld) * Ty<DT>::SZ;
}
// raw fp32 partial sums of this workgroup's tile into plane blockIdx.y of the workspace
template <int DT, int MI, int BM, int BN, int WTM, int WTN, int RM, int RN, class AccT>
__device__ __forceinline__ void store_partial(const KParams& p, const AccT (&acc)[RM][RN],
                                              int64_t m0, int64_t n0, int wm, int wn, int lane,
                                              int slot = -1) {
  typedef Atom<DT, MI> At;
  // whole-problem split: plane blockIdx.y of M x N; split tail: the compact BM x BN slot of
  // tail workgroup blockIdx.x in plane blockIdx.y; Stream-K: compact slot `slot`
  const bool tail = slot >= 0 || p.tail_tiles > 0;
  float* w = slot >= 0 ? p.workspace + (int64_t)slot * (BM * BN)
             : tail ? p.workspace + ((int64_t)blockIdx.y * p.tail_tiles + blockIdx.x) * (BM * BN)
                    : p.workspace + (int64_t)blockIdx.y * p.M * p.N;
  static_for<RM>([&](auto i) {
    static_for<RN>([&](auto j) {
      static_for<At::NACC>([&](auto r) {
        const int64_t col = n0 + wn * WTN + j * MI + acc_col<DT, MI>(lane, r);
        const int64_t row = m0 + wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
        if (row < p.M && col < p.N)
          w[tail ? (row - m0) * BN + (col - n0) : row * p.N + col] = acc[i][j][(int)r];
      });
    });
  });
}
// D = act(alpha * sum_s W[s] + beta * C + bias) elementwise, the planes added in order s = 0, 1, ...
template <int ODT>
__global__ __launch_bounds__(256) void gemm_splitk_reduce(const KParams p_) {
  const KParams p = batch_view(p_);
  typedef Out<ODT> O;
  const int64_t MN = p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < MN; e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / p.N, col = e - row * p.N;
    float sum = 0.f;
    for (int s = 0; s < p.split_k; ++s) sum += p.workspace[s * MN + e];
    O::store(p.D, row * p.d_sm + col * p.d_sn, finish_elem<ODT>(p, row, col, sum));
  }
}

// Second kernel of a split tail.  Block (x, y) takes tail tile x -- found with the same tile
// order as tail workgroup x of the first kernel -- and elements y, y + gridDim.y, ... of it:
// D = act(alpha * sum_s W[s] + beta * C + bias), the split_k partials added in order.
template <int ODT>
__global__ __launch_bounds__(256) void gemm_tail_reduce(const KParams p) {
  typedef Out<ODT> O;
  int tm, tn;
  tile_of(p, blockIdx.x, gridDim.x, tm, tn);
  const int64_t m0 = (int64_t)tm * p.tile_bm, n0 = (int64_t)tn * p.tile_bn;
  const int64_t area = (int64_t)p.tile_bm * p.tile_bn, plane = area * p.tail_tiles;
  const float* w = p.workspace + (int64_t)blockIdx.x * area;
  const int bn = p.tile_bn;
  for (int e = blockIdx.y * 256 + threadIdx.x; e < (int)area; e += gridDim.y * 256) {
    const int64_t row = m0 + e / bn, col = n0 + e % bn;
    if (row >= p.M || col >= p.N) continue;
    float sum = 0.f;
    for (int s = 0; s < p.split_k; ++s) sum += w[s * plane + e];
    O::store(p.D, row * p.d_sm + col * p.d_sn, finish_elem<ODT>(p, row, col, sum));
  }
}

// ------------------------------------------------------------------------------------------
// Stream-K ("CUTLASS", Part IV Stage 2: a tile scheduler that splits K across blocks so every
// processor gets an equal share of the work, then reduces the partial sums; Stream-K, Osama et
// al. 2023, cited there): P persistent workgroups share the I = tiles * nkt k-tile iterations of
// the Stream-K tiles; workgroup w takes iterations [I w / P, I (w+1) / P), walking them tile by
// tile.  A tile whose iterations one workgroup covers whole is finished by it; the pieces of a
// tile shared by several workgroups go to slots of the workspace (slot 2w for the first tile of
// workgroup w, 2w + 1 for its last) and a second pass adds them in workgroup (so K) order and
// applies the epilogue -- the pages' separate-reduction form of the second phase.
// ------------------------------------------------------------------------------------------
__host__ __device__ __forceinline__ int64_t sk_start(int64_t I, int P, int64_t w) { return I * w / P; }
// the workgroup whose range holds iteration i: the largest w with sk_start(w) <= i
__host__ __device__ __forceinline__ int sk_owner(int64_t I, int P, int64_t i) {
  const int64_t w = ((i + 1) * P + I - 1) / I - 1;
  return (int)(w < 0 ? 0 : (w >= P ? P - 1 : w));
}
template <int ODT>
__global__ __launch_bounds__(256) void gemm_sk_fixup(const KParams p) {
  typedef Out<ODT> O;
  const int64_t t = blockIdx.x, nkt = p.sk_nkt, I = (int64_t)p.sk_tiles * nkt;
  const int P = p.sk_wgs;
  const int wlo = sk_owner(I, P, t * nkt), whi = sk_owner(I, P, (t + 1) * nkt - 1);
  if (wlo == whi) return;  // finished by its one workgroup
  int tm, tn;
  tile_walk(p, (int)(p.tile_base + t), tm, tn);
  const int64_t m0 = (int64_t)tm * p.tile_bm, n0 = (int64_t)tn * p.tile_bn;
  const int64_t area = (int64_t)p.tile_bm * p.tile_bn;
  // the tile's pieces in workgroup order: one thread per workgroup finds its slot (-1: an empty
  // range, which holds no piece); at most P workgroups share a tile
  __shared__ int slots[256];
  const int n = whi - wlo + 1;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int64_t s0 = sk_start(I, P, wlo + i);
    slots[i] = s0 == sk_start(I, P, wlo + i + 1) ? -1 : 2 * (wlo + i) + (s0 / nkt == t ? 0 : 1);
  }
  __syncthreads();
  const int bn = p.tile_bn;
  for (int e = blockIdx.y * 256 + threadIdx.x; e < (int)area; e += gridDim.y * 256) {
    const int64_t row = m0 + e / bn, col = n0 + e % bn;
    if (row >= p.M || col >= p.N) continue;
    float sum = 0.f;
    for (int i = 0; i < n; ++i)
      if (slots[i] >= 0) sum += p.workspace[slots[i] * area + e];
    O::store(p.D, row * p.d_sm + col * p.d_sn, finish_elem<ODT>(p, row, col, sum));
  }
}

// ------------------------------------------------------------------------------------------
// Tile loaders: global -> registers -> swizzled LDS.
// LDS row r (an m of A or an n of B) holds BK elements as CH = BK*SZ/16 chunks.
// Every loader has the same interface: init() once per tile, load<PRED>(k0) for the k-tile at
// k0 (PRED: zero-fill elements at k >= K), store() into one LDS stage.
// ------------------------------------------------------------------------------------------
// Chunk slot of (row, chunk): Swizzle<3,0,4> on the chunk offset row * 8 + chunk, i.e. the XOR
// key is (row >> 1) & 7 (atom_maps.h).  A ds_read_b128 phase serves 16 lanes = 256 bytes = all
// 64 banks; the 16 lanes of an MFMA fragment read are 16 consecutive rows at one logical chunk,
// and with this key their 16-byte chunks land on 16 different 16-byte bank groups (rows 2m and
// 2m+1 differ in the 128-byte half, rows 2m..2m+14 in the XOR).  A 16-lane phase of the row-wise
// tile store covers two whole rows, also conflict free.  Rows longer than 128 bytes (CH a
// multiple of 8) keep the key of their first 8 chunks in every 8-chunk group.
template <int CH> __device__ __forceinline__ int lds_slot(int row, int chunk) {
  static_assert(CH % 8 == 0, "rows must be a multiple of 128 bytes");
  return row * CH + (chunk & ~7) + (swizzled_slot<8>(row, chunk & 7) - row * 8);
}

// Buffer descriptor over `bytes` bytes from `base` (gfx9 raw buffer: stride 0).  Loads whose
// VGPR offset (plus instruction offset) is at or past `bytes` return zero and touch no memory.
// The SGPR offset is added to the address but is not part of that range check, so it may only
// carry offsets that stay inside a valid row (the k position); row offsets go in the base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  bytes = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// K-contiguous operand, 16-byte buffer loads.  The descriptor starts at the tile's first row
// and ends at the operand's last element; the row offset of each load is in the (range-checked)
// VGPR offset, so rows past the end read as zero, and the k advance is the scalar offset.  The
// descriptor is rebuilt from uniform scalars at every load (SALU work): kept in the loader
// object, the compiler can no longer prove it uniform and wraps each load in a readfirstlane
// loop.  Needs (R*ld + K)*SZ < 2^31 (checked on the host).
template <int DT, int R, int BKE, int NT>
struct LoadKMajorVec {
  static constexpr int SZ = Ty<DT>::SZ, VE = 16 / SZ, CH = BKE * SZ / 16;
  static constexpr int N = R * CH / NT;
  static_assert(R * CH % NT == 0 && NT % CH == 0, "tile chunks must divide over the threads");
  u32x4 r[N];
  const char* tile;   // first byte of this tile's first row (uniform)
  int64_t ld, span, K;
  uint32_t voff;      // this thread's chunk within a group of NT/CH rows: row tid/CH, chunk tid%CH
  int kc;             // element offset of this thread's chunk within a k-tile
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0, int64_t rows,
                                       int64_t K_, int tid) {
    tile = (const char*)base + row0 * ld_ * SZ;
    ld = ld_;
    span = ((rows - row0 - 1) * ld_ + K_) * SZ;  // bytes from the tile start to the last element
    K = K_;
    voff = (uint32_t)((tid / CH) * ld_ * SZ + (tid % CH) * 16);
    kc = (tid % CH) * VE;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
    const uint32_t row_step = (uint32_t)((NT / CH) * ld * SZ);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(tile, span);
    const bool ok = !PRED || k0 + kc < K;
    const uint32_t vo = ok ? voff : voff - kc * SZ;  // an invalid k chunk reads its row start
#pragma unroll
    for (int i = 0; i < N; ++i) {
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vo + i * row_step, (int)(k0 * SZ), 0);
      r[i] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, row = q / CH, c = q % CH;
      lds[lds_slot<CH>(row, c)] = r[i];
    }
  }
};

// Row-contiguous (M- or N-contiguous) operand, 16-byte loads of VE rows at one k, transposed
// in registers into VE K-contiguous chunks.  Needs rows % VE == 0.
template <int DT, int R, int BKE, int NT>
struct LoadMNMajorVec {
  static constexpr int SZ = Ty<DT>::SZ, VE = 16 / SZ, CH = BKE * SZ / 16;
  static constexpr int BLOCKS = (BKE / VE) * (R / VE);
  static constexpr int N = (BLOCKS + NT - 1) / NT;  // threads past BLOCKS idle (whole waves)
  static_assert(BLOCKS % NT == 0 || (BLOCKS < NT && BLOCKS % 64 == 0),
                "transpose blocks must cover whole waves");
  static_assert(SZ == 2 || SZ == 4, "register transpose supports 2- and 4-byte elements");
  typedef typename Ty<DT>::T T;
  u32x4 r[N][VE];
  const T* src;
  int64_t ld, row0, rows, K;
  int tid;
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0_,
                                       int64_t rows_, int64_t K_, int tid_) {
    src = (const T*)base;
    ld = ld_; row0 = row0_; rows = rows_; K = K_; tid = tid_;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, rb = q % (R / VE), kb = q / (R / VE);
      if (BLOCKS % NT != 0 && q >= BLOCKS) continue;
      const int64_t gr = min(row0 + (int64_t)rb * VE, rows - VE);
#pragma unroll
      for (int kk = 0; kk < VE; ++kk) {
        const int64_t k = k0 + (int64_t)kb * VE + kk;
        if (!PRED || k < K)
          r[i][kk] = *(const u32x4*)(src + k * ld + gr);
        else
          r[i][kk] = u32x4{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, rb = q % (R / VE), kb = q / (R / VE);
      if (BLOCKS % NT != 0 && q >= BLOCKS) continue;
#pragma unroll
      for (int rr = 0; rr < VE; ++rr) {
        u32x4 o;
        if constexpr (SZ == 4) {
          o = u32x4{r[i][0][rr], r[i][1][rr], r[i][2][rr], r[i][3][rr]};
        } else {
          const int w = rr >> 1, sh = (rr & 1) * 16;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32 lo = (r[i][2 * d][w] >> sh) & 0xffffu;
            const u32 hi = (r[i][2 * d + 1][w] >> sh) & 0xffffu;
            o[d] = lo | (hi << 16);
          }
        }
        lds[lds_slot<CH>(rb * VE + rr, kb)] = o;
      }
    }
  }
};

// Any alignment: element loads with full predication.  KMAJ selects which index is contiguous;
// threads walk the contiguous direction so neighbouring lanes read neighbouring elements.
template <int DT, bool KMAJ, int R, int BKE, int NT>
struct LoadNarrow {
  typedef typename Ty<DT>::T T;
  static constexpr int SZ = Ty<DT>::SZ, VE = 16 / SZ, CH = BKE * SZ / 16;
  static constexpr int N = R * CH / NT;
  static_assert(R * CH % NT == 0, "tile chunks must divide over the threads");
  T e[N][VE];
  const T* src;
  int64_t ld, row0, rows, K;
  int tid;
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0_,
                                       int64_t rows_, int64_t K_, int tid_) {
    src = (const T*)base;
    ld = ld_; row0 = row0_; rows = rows_; K = K_; tid = tid_;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT;
      const int row = KMAJ ? q / CH : q % R;
      const int c = KMAJ ? q % CH : q / R;
      const int64_t gr = row0 + row;
#pragma unroll
      for (int j = 0; j < VE; ++j) {
        const int64_t k = k0 + (int64_t)c * VE + j;
        const bool ok = gr < rows && k < K;
        const int64_t off = KMAJ ? gr * ld + k : k * ld + gr;
        e[i][j] = ok ? src[off] : T(0);
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT;
      const int row = KMAJ ? q / CH : q % R;
      const int c = KMAJ ? q % CH : q / R;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32 w = 0;
#pragma unroll
        for (int b = 0; b < 4 / SZ; ++b) w |= u32(e[i][d * (4 / SZ) + b]) << (8 * SZ * b);
        o[d] = w;
      }
      lds[lds_slot<CH>(row, c)] = o;
    }
  }
};

// ------------------------------------------------------------------------------------------
// 2-byte operands whose rows are only 2-byte aligned (odd leading dimension or base).  Each
// 16-byte chunk is fetched as the 16 dword-aligned bytes at or below its first element plus the
// dword after them, and realigned with v_alignbyte only when it is written to LDS: nothing
// consumes the loads before then, so they overlap the current k-tile's MFMAs as the other
// loaders' do.  Offsets are 32-bit VGPR offsets from the tile's first byte rounded down to 4
// bytes.  The descriptor's extent is the operand's end rounded up to a whole dword; a raw buffer
// load checks each of its dwords against the extent on its own (a 16-byte load that straddles it
// returns the dwords inside and zeros), and the dword that holds the operand's last element lies
// in that element's page, so no unmapped byte is read.  Chunks wholly past K or past the last
// row take an out-of-range offset (zeros); elements of a partial chunk past K, past the last
// row or column, or past the operand's end are cleared by the element mask.
// ------------------------------------------------------------------------------------------
struct Raw16 {
  u32x4 q;  // the 16 bytes at the dword-aligned address at or below the chunk
  u32 x;    // the dword after them
};
__device__ __forceinline__ Raw16 raw16(__amdgpu_buffer_rsrc_t r, uint32_t a) {
  return {__builtin_amdgcn_raw_buffer_load_b128(r, a, 0, 0),
          __builtin_amdgcn_raw_buffer_load_b32(r, a + 16, 0, 0)};
}
// the 8 elements that start `sh` bytes into a fetched chunk; element e kept where bit e of emask
// is set
__device__ __forceinline__ u32x4 realign16(const Raw16& w, uint32_t sh, uint32_t emask) {
  u32x4 v;
  v[0] = __builtin_amdgcn_alignbyte(w.q[1], w.q[0], sh);
  v[1] = __builtin_amdgcn_alignbyte(w.q[2], w.q[1], sh);
  v[2] = __builtin_amdgcn_alignbyte(w.q[3], w.q[2], sh);
  v[3] = __builtin_amdgcn_alignbyte(w.x, w.q[3], sh);
  if (emask != 0xffu) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t m2 = (emask >> (2 * d)) & 3u;
      v[d] &= (m2 & 1u ? 0xffffu : 0u) | (m2 & 2u ? 0xffff0000u : 0u);
    }
  }
  return v;
}
constexpr uint32_t kOobOffset = 0x80000000u;  // past any extent (extents are below 2^31)

// K-contiguous 2-byte operand, any element alignment.  Same thread -> chunk map and LDS layout as
// LoadKMajorVec.
template <int DT, int R, int BKE, int NT>
struct LoadKMajorMis {
  static_assert(Ty<DT>::SZ == 2, "2-byte elements");
  static constexpr int SZ = 2, VE = 8, CH = BKE * SZ / 16;
  static constexpr int N = R * CH / NT;
  static_assert(R * CH % NT == 0 && NT % CH == 0, "tile chunks must divide over the threads");
  static_assert(N <= 24, "one shift bit per chunk");
  Raw16 w[N];
  uint32_t emask;     // element mask of this thread's chunk in the current k-tile
  uint32_t shifts;    // bit i: chunk i starts 2 bytes past a dword (fixed: k-tiles are 128 bytes)
  const char* rb;     // the tile's first byte rounded down to 4 bytes (uniform)
  int64_t ext, K;     // descriptor extent in bytes; K
  int64_t rows_left;  // rows of the operand from the tile's first row on
  uint32_t voff, row_step;
  int row, kc;        // this thread's first row within the tile; its chunk's first k
  __device__ __forceinline__ void init(const void* base, int64_t ld, int64_t row0, int64_t rows,
                                       int64_t K_, int tid) {
    const char* tile = (const char*)base + row0 * ld * SZ;
    rb = (const char*)((uintptr_t)tile & ~uintptr_t(3));
    const uint32_t delta = (uint32_t)(tile - rb);
    K = K_;
    rows_left = rows - row0;
    ext = (delta + ((rows_left - 1) * ld + K_) * SZ + 3) & ~int64_t(3);
    row = tid / CH;
    kc = (tid % CH) * VE;
    voff = delta + (uint32_t)((row * ld + kc) * SZ);
    row_step = (uint32_t)((NT / CH) * ld * SZ);
    shifts = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) shifts |= ((voff + i * row_step) & 2u) >> 1 << i;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, ext);
    const int64_t k = k0 + kc;
    emask = 0xffu;
    if (PRED) emask = k >= K ? 0u : (k + VE <= K ? 0xffu : ((1u << (K - k)) - 1u));
    const uint32_t kb = (uint32_t)(k0 * SZ);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool live = row + i * (NT / CH) < rows_left && emask != 0;
      w[i] = raw16(rsrc, live ? ((voff + i * row_step + kb) & ~3u) : kOobOffset);
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, rr = q / CH, cc = q % CH;
      lds[lds_slot<CH>(rr, cc)] = realign16(w[i], ((shifts >> i) & 1u) * 2u, emask);
    }
  }
};

// Row-contiguous (M- or N-contiguous) 2-byte operand, any element alignment: chunks of VE rows at
// one k, realigned and then transposed in registers into K-contiguous chunks as in
// LoadMNMajorVec; rows past the operand's last row and k past K are zero.
template <int DT, int R, int BKE, int NT>
struct LoadMNMajorMis {
  static_assert(Ty<DT>::SZ == 2, "2-byte elements");
  static constexpr int SZ = 2, VE = 8, CH = BKE * SZ / 16;
  static constexpr int BLOCKS = (BKE / VE) * (R / VE);
  static constexpr int N = (BLOCKS + NT - 1) / NT;
  static_assert(BLOCKS % NT == 0 || (BLOCKS < NT && BLOCKS % 64 == 0),
                "transpose blocks must cover whole waves");
  static_assert(N <= 3, "mask bytes of the blocks fit one register");
  Raw16 w[N][VE];
  uint32_t nmasks;    // byte i: row mask of block i (fixed per tile)
  uint32_t shifts;    // bit kk: the chunk at k offset kk starts 2 bytes past a dword
  const char* rb;
  int64_t ext, K, ld;
  uint32_t boff[N];   // byte offset of block i at k = 0
  int tid;
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0, int64_t rows,
                                       int64_t K_, int tid_) {
    const char* tile = (const char*)base + row0 * SZ;
    rb = (const char*)((uintptr_t)tile & ~uintptr_t(3));
    const uint32_t delta = (uint32_t)(tile - rb);
    ld = ld_;
    K = K_;
    tid = tid_;
    const int64_t rows_left = rows - row0;
    ext = (delta + ((K_ - 1) * ld_ + rows_left) * SZ + 3) & ~int64_t(3);
    nmasks = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, rbk = q % (R / VE), kb = q / (R / VE);
      const int64_t n = (int64_t)rbk * VE;
      const uint32_t m = n >= rows_left ? 0u : (n + VE <= rows_left ? 0xffu : ((1u << (rows_left - n)) - 1u));
      nmasks |= m << (8 * i);
      boff[i] = delta + (uint32_t)((kb * VE * ld_ + n) * SZ);
    }
    // every block's offset has the same parity in 2-byte units (n and kb * VE * ld are even), so
    // the shift depends only on kk
    shifts = 0;
#pragma unroll
    for (int kk = 0; kk < VE; ++kk) shifts |= ((boff[0] + (uint32_t)(kk * ld_ * SZ)) & 2u) >> 1 << kk;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, ext);
    const uint32_t kb0 = (uint32_t)(k0 * ld * SZ);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, kb = q / (R / VE);
      if (BLOCKS % NT != 0 && q >= BLOCKS) continue;
      const bool any = ((nmasks >> (8 * i)) & 0xffu) != 0;
#pragma unroll
      for (int kk = 0; kk < VE; ++kk) {
        const bool live = any && (!PRED || k0 + (int64_t)kb * VE + kk < K);
        const uint32_t o = boff[i] + kb0 + (uint32_t)(kk * ld * SZ);
        w[i][kk] = raw16(rsrc, live ? (o & ~3u) : kOobOffset);
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = tid + i * NT, rbk = q % (R / VE), kb = q / (R / VE);
      if (BLOCKS % NT != 0 && q >= BLOCKS) continue;
      const uint32_t m = (nmasks >> (8 * i)) & 0xffu;
      u32x4 c[VE];
#pragma unroll
      for (int kk = 0; kk < VE; ++kk) c[kk] = realign16(w[i][kk], ((shifts >> kk) & 1u) * 2u, m);
#pragma unroll
      for (int rr = 0; rr < VE; ++rr) {
        u32x4 o;
        const int wd = rr >> 1, sh = (rr & 1) * 16;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32 lo = (c[2 * d][wd] >> sh) & 0xffffu;
          const u32 hi = (c[2 * d + 1][wd] >> sh) & 0xffffu;
          o[d] = lo | (hi << 16);
        }
        lds[lds_slot<CH>(rbk * VE + rr, kb)] = o;
      }
    }
  }
};

// ------------------------------------------------------------------------------------------
// MN-major 2-byte operands kept as rows of k.  The tile's BKE rows (one per k) of R >= 128
// elements are copied untransposed into LDS (slot mn_slot, atom_maps.h) and the MFMA fragments
// are assembled by transposing LDS reads (read_rows_frag), so no VALU transpose is needed.
// Thread q of a copy owns chunks (k, c) = (q / CHR, q % CHR) + (NT / CHR) rows per step: 16
// consecutive lanes read 256 contiguous bytes of one row and write 16 distinct bank slots.
// Columns past the operand's last one are not cleared: they only reach outputs past N (or M),
// which are never stored; reads past the operand's end return zero (buffer range check).
// ------------------------------------------------------------------------------------------
template <int DT, int R, int BKE, int NT>
struct LoadMNRowsVec {
  static_assert(Ty<DT>::SZ == 2, "2-byte elements");
  static constexpr int SZ = 2, VE = 8, CHR = R * SZ / 16, STEP = NT / CHR;
  static constexpr int N = BKE * CHR / NT;
  static_assert(BKE * CHR % NT == 0 && NT % CHR == 0, "tile chunks must divide over the threads");
  u32x4 r[N];
  const char* tile;
  int64_t ld, span, K;
  uint32_t voff;  // this thread's first chunk: row tid / CHR, chunk tid % CHR
  int k1;         // its first row
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0, int64_t rows,
                                       int64_t K_, int tid) {
    tile = (const char*)base + row0 * SZ;
    ld = ld_;
    K = K_;
    span = ((K_ - 1) * ld_ + (rows - row0)) * SZ;  // bytes from the tile start to the last element
    k1 = tid / CHR;
    voff = (uint32_t)((k1 * ld_ + (tid % CHR) * VE) * SZ);
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(tile, span);
    const uint32_t row_step = (uint32_t)(STEP * ld * SZ);
    const uint32_t kb = (uint32_t)(k0 * ld * SZ);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool ok = !PRED || k0 + k1 + i * STEP < K;
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? voff + kb + i * row_step : kOobOffset, 0, 0);
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[mn_slot<CHR>(tid / CHR + i * STEP, tid % CHR)] = r[i];
  }
};

template <int DT, int R, int BKE, int NT>
struct LoadMNRowsMis {
  static_assert(Ty<DT>::SZ == 2, "2-byte elements");
  static constexpr int SZ = 2, VE = 8, CHR = R * SZ / 16, STEP = NT / CHR;
  static constexpr int N = BKE * CHR / NT;
  static_assert(BKE * CHR % NT == 0 && NT % CHR == 0, "tile chunks must divide over the threads");
  Raw16 w[N];
  const char* rb;      // the tile's first byte rounded down to 4 bytes (uniform)
  int64_t ext, K, ld;
  uint32_t voff;       // this thread's first chunk, from rb
  uint32_t shift;      // 2 when its chunks start 2 bytes past a dword (the same for all of them:
                       // STEP rows apart is a whole number of dwords, STEP being even)
  int k1;
  __device__ __forceinline__ void init(const void* base, int64_t ld_, int64_t row0, int64_t rows,
                                       int64_t K_, int tid) {
    static_assert(STEP % 2 == 0, "even row steps keep the dword phase");
    const char* tile = (const char*)base + row0 * SZ;
    rb = (const char*)((uintptr_t)tile & ~uintptr_t(3));
    const uint32_t delta = (uint32_t)(tile - rb);
    ld = ld_;
    K = K_;
    ext = (delta + ((K_ - 1) * ld_ + (rows - row0)) * SZ + 3) & ~int64_t(3);
    k1 = tid / CHR;
    voff = delta + (uint32_t)((k1 * ld_ + (tid % CHR) * VE) * SZ);
    shift = voff & 2u;
  }
  template <bool PRED>
  __device__ __forceinline__ void load(int64_t k0) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, ext);
    const uint32_t row_step = (uint32_t)(STEP * ld * SZ);
    const uint32_t kb = (uint32_t)(k0 * ld * SZ);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool ok = !PRED || k0 + k1 + i * STEP < K;
      w[i] = raw16(rsrc, ok ? ((voff + kb + i * row_step) & ~3u) : kOobOffset);
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      lds[mn_slot<CHR>(tid / CHR + i * STEP, tid % CHR)] = realign16(w[i], shift, 0xffu);
  }
};

// One MFMA operand fragment from a rows-of-k tile: lane l receives k = kb .. kb + 7 of column
// col0 + frow, frow being its row / column in the atom's operand layout (frag_row), through two
// transposing 8-byte reads.  Each read gives every 16-lane group a 4 (k) x 16 (column) block: the
// lane at place s of its group addresses row kb + 4h + s / 4 at column (the group's first
// column) + 4 (s % 4), and receives that block's column s; the layouts put the lanes of a group
// on 16 consecutive columns, frow = (frow & ~15) + s.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef __attribute__((address_space(3))) char lds_char_t;
template <int CHR>
__device__ __forceinline__ u32x4 read_rows_frag(const u32x4* tile, int kb, int col0, int frow, int lane) {
  const int s = lane & 15;
  const int col = col0 + (frow & ~15) + 4 * (s & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = kb + 4 * h + (s >> 2);
    const int byte = mn_slot<CHR>(k, col >> 3) * 16 + (col & 4) * 2;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)((lds_char_t*)(tile) + byte));
    const u32x4 w = __builtin_bit_cast(u32x4, __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3));
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

// VEC: 0 element loads (any alignment), 1 16-byte loads (aligned rows), 2 realigned 16-byte
// loads (2-byte types, any element alignment)
template <int DT, bool KMAJ, int VEC, int R, int BKE, int NT>
struct PickLoader {
  typedef LoadNarrow<DT, KMAJ, R, BKE, NT> type;
};
template <int DT, int R, int BKE, int NT>
struct PickLoader<DT, true, 1, R, BKE, NT> {
  typedef LoadKMajorVec<DT, R, BKE, NT> type;
};
// MN-major 2-byte operands of at least 128 rows are kept as rows of k (transposing reads)
template <int DT, bool KMAJ, int VEC, int R> struct RowsLayout {
  static constexpr bool value = !KMAJ && VEC != 0 && Ty<DT>::SZ == 2 && R >= 128;
};
template <int DT, int R, int BKE, int NT>
struct PickLoader<DT, false, 1, R, BKE, NT> {
  typedef typename std::conditional<RowsLayout<DT, false, 1, R>::value, LoadMNRowsVec<DT, R, BKE, NT>,
                                    LoadMNMajorVec<DT, R, BKE, NT>>::type type;
};
template <int DT, int R, int BKE, int NT>
struct PickLoader<DT, true, 2, R, BKE, NT> {
  typedef LoadKMajorMis<DT, R, BKE, NT> type;
};
template <int DT, int R, int BKE, int NT>
struct PickLoader<DT, false, 2, R, BKE, NT> {
  typedef typename std::conditional<RowsLayout<DT, false, 2, R>::value, LoadMNRowsMis<DT, R, BKE, NT>,
                                    LoadMNMajorMis<DT, R, BKE, NT>>::type type;
};

// One element of C through a range-checked buffer load: `off` is its byte offset from C's base,
// or kOobOffset for an element outside the problem (the load then returns zero bits).  Unlike a
// predicated pointer load it needs no branch, so the loads of a whole row block issue back to
// back and are waited for once.
template <int ODT>
__device__ __forceinline__ float load_c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ODT == DT_F32)
    return Out<ODT>::from_bits(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  else
    return Out<ODT>::from_bits((u32)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// ------------------------------------------------------------------------------------------
// Epilogue ("CUTLASS", Part IV Stages 5 and 6).
// Phase 1, in registers: y = act(alpha * acc + beta * C + bias[n]) in fp32, rounded once to the
// output type.  Phase 2: the rounded tile goes through LDS so the store to D is 16-byte
// row-contiguous chunks instead of the MFMA's column-wise lane layout.  The caller guarantees
// that no wave still reads the LDS operand stages and no DMA into them is in flight.
//
// Rows of a row-major D whose 16-byte grid does not start at the tile's first column (a leading
// dimension or base off 16 bytes) are placed in LDS shifted by that misalignment, so that chunk
// j of an LDS row holds the outputs of D's aligned chunk j: the store is still one 16-byte store
// per chunk, with element stores only for the partial chunks at the two ends of a row.  A
// row-major C is staged the same way before phase 1 -- 16-byte chunks in D's grid, through
// realigned loads where C's own alignment differs -- and each lane reads its C values from the
// LDS position its result then overwrites.
//
// FORM selects a copy of the epilogue compiled for one class of launch (epilogue_form): 1 = no
// C, no scale vectors, no fused reductions, D row-major in whole 16-byte rows; 0 = every case.
// The epilogue runs once per tile and is unrolled over the wave tile: with every case compiled
// in, its executed path is scattered over a long stretch of code that each tile fetches again,
// and the specialised copy keeps it short and straight.  (A copy for a row-major C staged
// through LDS ran out of registers in the ping-pong kernel.)
// ------------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ int epilogue_form(const KParams& p) {
  constexpr int OSZ = (int)sizeof(typename OutBits<out_dtype(DT)>::T);
  return !p.has_c && !p.has_row_scale && !p.has_col_scale && !p.rsq_ws && !p.csum_ws &&
                 p.d_sn == 1 && (p.d_sm * OSZ) % 16 == 0 &&
                 (reinterpret_cast<uintptr_t>(p.D) % 16) == 0
             ? 1
             : 0;
}

template <int DT, int MI, int BM, int BN, int WTM, int WTN, int RM, int RN, int NT,
          size_t LDS_BYTES, int FORM = 0, class AccT>
__device__ __forceinline__ void epilogue(const KParams& p, AccT (&acc)[RM][RN], u32x4* lds,
                                              int64_t m0, int64_t n0, int wm, int wn, int lane,
                                              int tid, bool no_mainloop) {
  typedef Atom<DT, MI> At;
  constexpr int ODT = out_dtype(DT);
  typedef Out<ODT> O;
  typedef typename OutBits<ODT>::T OT;
  constexpr int OSZ = (int)sizeof(OT);
  // Rows of the LDS tile are PITCH outputs apart.  One store instruction writes rows r and r + 4
  // (16x16 atom: the two quarter-waves of each half-wave; 32x32: the two half-waves); 16 bytes
  // of padding per row put those rows on different banks (with BN * OSZ a multiple of 256 bytes
  // they would share them) and leave room for a row shifted by up to one chunk (below).  The
  // padding is used only where the padded tile still fits.
  constexpr int PAD = 16 / OSZ;
  constexpr bool SHIFT = (size_t)BM * (BN + PAD) * OSZ <= LDS_BYTES;  // room for shifted rows
  constexpr int PITCH = SHIFT ? BN + PAD : BN;
  constexpr bool REPACK = (size_t)BM * PITCH * OSZ <= LDS_BYTES;
  constexpr int VO = 16 / OSZ;            // outputs per 16-byte chunk
  constexpr int CPR = BN / VO;            // chunks per tile row (aligned rows)
  const bool has_c = FORM == 0 && p.has_c != 0, has_bias = p.has_bias != 0;
  const bool has_rs = FORM == 0 && p.has_row_scale != 0, has_cs = FORM == 0 && p.has_col_scale != 0;
  const int act = p.act;
  const float alpha = p.alpha, beta = p.beta;
  OT* tile = reinterpret_cast<OT*>(lds);  // BM x BN, row-major, rows PITCH apart (REPACK only)
  if (REPACK && no_mainloop) __syncthreads();
  // Shifted rows: output (row, n0 + c) at LDS position c + mis(row), mis(row) = the element
  // offset of D(row, n0) past a 16-byte boundary (0 for aligned rows).  Not with the fused
  // reductions, which read the tile unshifted.
  const bool d_rows = FORM == 0 && SHIFT && REPACK && p.d_sn == 1 && !p.rsq_ws && !p.csum_ws;
  const bool vec_ok = FORM == 1 || (p.d_sn == 1 && (p.d_sm * OSZ) % 16 == 0 &&
                                    (reinterpret_cast<uintptr_t>(p.D) % 16) == 0);
  const bool shifted = d_rows && !vec_ok;  // aligned rows have mis = 0 throughout
  const uint32_t d_el0 = (uint32_t)(reinterpret_cast<uintptr_t>(p.D) / OSZ) + (uint32_t)n0;
  auto mis_raw = [&](int64_t row) -> int {
    return (int)((d_el0 + (uint32_t)row * (uint32_t)p.d_sm) & (uint32_t)(VO - 1));
  };
  auto mis_of = [&](int64_t row) -> int { return shifted ? mis_raw(row) : 0; };
  // The chunks of D's 16-byte grid that a tile row touches: chunk j covers columns
  // col0 = n0 - mis + j * VO onward, of which [lo, hi) belong to the tile and the problem.
  constexpr int CPRS = CPR + 1;
  auto chunk_of = [&](int lr, int j, int64_t& col0, int64_t& lo, int64_t& hi) {
    col0 = n0 - mis_of(m0 + lr) + (int64_t)j * VO;
    lo = max(col0, n0);
    hi = min(col0 + VO, min(n0 + BN, p.N));
  };
  // Row-major C staged into the LDS tile at the output positions (buffer loads: C below 2^31
  // bytes).  The descriptor starts at C rounded down to 4 bytes; `cdelta` is the difference.
  const bool c_lds = d_rows && has_c && p.c_sn == 1 && p.c_span > 0;
  if (c_lds) {
    const char* cb = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(p.C) & ~uintptr_t(3));
    const uint32_t cdelta = (uint32_t)(reinterpret_cast<const char*>(p.C) - cb);
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(cb, (cdelta + p.c_span + 3) & ~int64_t(3));
    // Whole chunks: branch-free loads (out-of-range offsets read zero), a batch of them issued
    // back to back before their LDS writes, so a batch waits for memory once.
    constexpr int ITER = (BM * CPRS + NT - 1) / NT;
    constexpr int BATCH = ITER < 9 ? ITER : 9;
#pragma unroll
    for (int it0 = 0; it0 < ITER; it0 += BATCH) {
      Raw16 w[BATCH];
      uint32_t sh[BATCH];
      int pos[BATCH];
      static_for<BATCH>([&](auto b) {
        const int q = tid + (it0 + b) * NT;
        const int lr = q / CPRS, j = q - lr * CPRS;
        int64_t col0, lo, hi;
        chunk_of(lr, j, col0, lo, hi);
        const bool whole = q < BM * CPRS && m0 + lr < p.M && lo == col0 && hi == col0 + VO;
        const uint32_t off = cdelta + (uint32_t)(((m0 + lr) * p.c_sm + col0) * OSZ);
        if constexpr (OSZ == 2) {
          w[b] = raw16(cr, whole ? (off & ~3u) : kOobOffset);
        } else {
          w[b].q = __builtin_amdgcn_raw_buffer_load_b128(cr, whole ? off : kOobOffset, 0, 0);
          w[b].x = 0;
        }
        sh[b] = off & 2u;
        pos[b] = whole ? lr * PITCH + j * VO : -1;
      });
      static_for<BATCH>([&](auto b) {
        if (pos[b] >= 0)
          *reinterpret_cast<u32x4*>(&tile[pos[b]]) = OSZ == 2 ? realign16(w[b], sh[b], 0xffu) : w[b].q;
      });
    }
    // The partial chunks at the two ends of a row (the first when the row is shifted, the one
    // holding the row's last column when it does not end a chunk): element loads.
    for (int q = tid; q < BM * 2; q += NT) {
      const int lr = q >> 1;
      const int64_t row = m0 + lr;
      const int64_t end = min(n0 + BN, p.N);
      if (row >= p.M || end <= n0) continue;
      const int jl = (int)((end - 1 - (n0 - mis_of(row))) / VO);
      if ((q & 1) && jl == 0) continue;  // a single chunk: the even thread takes it
      const int j = (q & 1) ? jl : 0;
      int64_t col0, lo, hi;
      chunk_of(lr, j, col0, lo, hi);
      if (lo >= hi || (lo == col0 && hi == col0 + VO)) continue;
      OT e[VO];
#pragma unroll
      for (int x = 0; x < VO; ++x) {
        const int64_t col = col0 + x;
        const uint32_t off = col >= lo && col < hi ? cdelta + (uint32_t)((row * p.c_sm + col) * OSZ)
                                                   : kOobOffset;
        if constexpr (OSZ == 2) e[x] = (OT)__builtin_amdgcn_raw_buffer_load_b16(cr, off, 0, 0);
        else e[x] = (OT)__builtin_amdgcn_raw_buffer_load_b32(cr, off, 0, 0);
      }
      *reinterpret_cast<u32x4*>(&tile[lr * PITCH + j * VO]) = *reinterpret_cast<const u32x4*>(e);
    }
    __syncthreads();
  }
  // The stages run one row block of atoms (acc[i][*]) at a time, so only that block's values
  // are live in VGPRs; within a block each stage is one straight-line pass entered on a uniform
  // condition, so the common case (no C) carries no per-element branches:
  // y = act((alpha * acc + beta * C) + bias[n]).
  float bias_v[RN], cs_v[RN];
  const int acol = acc_col<DT, MI>(lane, std::integral_constant<int, 0>{});  // the same for every register of the lane
  static_for<RN>([&](auto j) {
    const int64_t col = n0 + wn * WTN + j * MI + acol;
    bias_v[j] = has_bias && col < p.N ? O::load(p.bias, col) : 0.f;
    cs_v[j] = has_cs && col < p.N ? p.col_scale[col] : 1.f;
  });
  static_for<RM>([&](auto i) {
    auto each = [&](auto&& f) {
      static_for<RN>([&](auto j) { static_for<At::NACC>([&](auto r) { f(j, r); }); });
    };
    if (alpha != 1.f) each([&](auto j, auto r) { acc[i][j][(int)r] *= alpha; });  // x1 is exact
    if (has_rs) {
      each([&](auto j, auto r) {
        const int64_t row = m0 + wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
        acc[i][j][(int)r] *= row < p.M ? p.row_scale[row] : 1.f;
      });
    }
    if (has_cs) each([&](auto j, auto r) { acc[i][j][(int)r] *= cs_v[j]; });
    if (c_lds) {
      // (two forms, so that aligned rows carry no per-element shift arithmetic)
      auto get_c = [&](auto SH) {
        each([&](auto j, auto r) {
          const int lc = wn * WTN + j * MI + acol;
          const int lr = wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
          const int pos = lr * PITCH + lc + (SH ? mis_raw(m0 + lr) : 0);
          acc[i][j][(int)r] += beta * O::from_bits((u32)tile[pos]);
        });
      };
      if (shifted) get_c(std::true_type{}); else get_c(std::false_type{});
    } else if (has_c && p.c_span > 0) {
      const __amdgpu_buffer_rsrc_t cr = make_rsrc((const char*)p.C, p.c_span);
      each([&](auto j, auto r) {
        const int64_t col = n0 + wn * WTN + j * MI + acol;
        const int64_t row = m0 + wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
        const uint32_t off = col < p.N && row < p.M
                                 ? (uint32_t)((row * p.c_sm + col * p.c_sn) * (int64_t)sizeof(OT))
                                 : kOobOffset;
        acc[i][j][(int)r] += beta * load_c<ODT>(cr, off);
      });
    } else if (has_c) {  // C spans 2^31 bytes or more: predicated pointer loads
      each([&](auto j, auto r) {
        const int64_t col = n0 + wn * WTN + j * MI + acol;
        const int64_t row = m0 + wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
        if (col < p.N && row < p.M) acc[i][j][(int)r] += beta * O::load(p.C, row * p.c_sm + col * p.c_sn);
      });
    }
    if (has_bias) each([&](auto j, auto r) { acc[i][j][(int)r] += bias_v[j]; });
    if (act == 2) each([&](auto j, auto r) { acc[i][j][(int)r] = gelu(acc[i][j][(int)r]); });
    else if (act == 1) each([&](auto j, auto r) { acc[i][j][(int)r] = relu(acc[i][j][(int)r]); });
    else if (act == 3) each([&](auto j, auto r) { acc[i][j][(int)r] = silu(acc[i][j][(int)r]); });
    auto put = [&](auto SH) {
      static_for<RN>([&](auto j) {
        const int lc = wn * WTN + j * MI + acol;
        const int64_t col = n0 + lc;
        static_for<At::NACC>([&](auto r) {
          const int lr = wm * WTM + i * MI + acc_row<DT, MI>(lane, r);
          const float v = acc[i][j][(int)r];
          if constexpr (REPACK) {
            const int pos = lr * PITCH + lc + (SH ? mis_raw(m0 + lr) : 0);
            tile[pos] = to_bits(v, std::integral_constant<int, ODT>{});
          } else {
            const int64_t row = m0 + lr;
            if (col < p.N && row < p.M) O::store(p.D, row * p.d_sm + col * p.d_sn, v);
          }
        });
      });
    };
    if (shifted) put(std::true_type{}); else put(std::false_type{});
  });
  if constexpr (REPACK) {
    __syncthreads();
    constexpr int NCH = BM * CPR;
    static_assert(NCH % NT == 0, "output chunks must divide over the threads");
    OT* dst = reinterpret_cast<OT*>(p.D);
    if (shifted) {
      // shifted rows: one aligned 16-byte store per whole chunk of D's grid
      constexpr int ITER = (BM * CPRS + NT - 1) / NT;
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int q = tid + it * NT;
        const int lr = q / CPRS, j = q - lr * CPRS;
        const int64_t row = m0 + lr;
        int64_t col0, lo, hi;
        chunk_of(lr, j, col0, lo, hi);
        if (q >= BM * CPRS || row >= p.M || lo >= hi) continue;
        const u32x4 val = *reinterpret_cast<const u32x4*>(&tile[lr * PITCH + j * VO]);
        if (lo == col0 && hi == col0 + VO) {
          *reinterpret_cast<u32x4*>(dst + row * p.d_sm + col0) = val;
        } else {
          const OT* e = reinterpret_cast<const OT*>(&val);
#pragma unroll
          for (int x = 0; x < VO; ++x)
            if (col0 + x >= lo && col0 + x < hi) dst[row * p.d_sm + col0 + x] = e[x];
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < NCH / NT; ++it) {
        const int q = tid + it * NT;
        const int lr = q / CPR, lc = (q % CPR) * VO;
        const int64_t row = m0 + lr, col = n0 + lc;
        if (row >= p.M) continue;
        const u32x4 val = *reinterpret_cast<const u32x4*>(&tile[lr * PITCH + lc]);
        if (vec_ok && col + VO <= p.N) {
          *reinterpret_cast<u32x4*>(dst + row * p.d_sm + col) = val;
        } else {
          const OT* e = reinterpret_cast<const OT*>(&val);
#pragma unroll
          for (int x = 0; x < VO; ++x)
            if (col + x < p.N) dst[row * p.d_sm + (col + x) * p.d_sn] = e[x];
        }
      }
    }
    if (FORM == 0 && p.rsq_ws) {
      // Row reduction for the next layer's norm ("CUTLASS", Part IV Stage 5: an epilogue visitor
      // tree can fuse a reduction): the sum of squares of this tile's stored values of each row,
      // one wave per row, lanes striding the columns, then a fixed-order butterfly.  The
      // partial goes to plane (tile column) of the workspace; a second kernel adds the planes.
      constexpr int NW = NT / 64;
      const int wave = tid >> 6;
      for (int lr = wave; lr < BM && m0 + lr < p.M; lr += NW) {
        float sq = 0.f;
#pragma unroll
        for (int c = lane; c < BN; c += 64) {
          const float v = n0 + c < p.N ? O::from_bits((u32)tile[lr * PITCH + c]) : 0.f;
          sq += v * v;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
        if (lane == 0) p.rsq_ws[(n0 / BN) * p.M + m0 + lr] = sq;
      }
    }
    if (FORM == 0 && p.csum_ws) {
      // Column sums of the stored tile: a wave takes 64 consecutive columns (one per lane, no
      // bank conflicts) and a group of rows; RG row groups give RG partials per column, written
      // to plane (tile row) * RG + (row group).
      constexpr int NW = NT / 64, CG = BN / 64, RG = NW >= CG ? NW / CG : 1;
      static_assert(BN % 64 == 0 && (NW % CG == 0 || NW < CG), "column groups over the waves");
      const int wave = tid >> 6;
      for (int cg = wave % CG; cg < CG; cg += NW >= CG ? CG : NW) {
        const int rg = NW >= CG ? wave / CG : 0;
        const int c = cg * 64 + lane;
        constexpr int RPG = BM / RG;  // rows per group
        float cs = 0.f;
        for (int r = rg * RPG; r < (rg + 1) * RPG && m0 + r < p.M; ++r)
          cs += O::from_bits((u32)tile[r * PITCH + c]);
        if (n0 + c < p.N) p.csum_ws[((m0 / BM) * RG + rg) * p.N + n0 + c] = cs;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// The tiled kernel.
// ------------------------------------------------------------------------------------------
template <int DT, bool AK, bool BKM, int VEC, int BM, int BN, int BKE, int WM, int WN, int MI>
__global__ __launch_bounds__(WM * WN * 64, BM * BN <= 128 * 128 && (AK || BKM) ? 2 : 1) void gemm_tiled(const KParams p_) {
  KParams p;
  int pid, nwg;
  if (!problem_view<BM>(p_, p, pid, nwg)) return;
  typedef Atom<DT, MI> At;
  typedef typename At::acc_t acc_t;
  constexpr int NT = WM * WN * 64;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int CH = BKE * SZ / 16;          // 16-byte chunks per LDS row
  constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
  constexpr int RM = WTM / MI, RN = WTN / MI; // atoms per wave tile
  constexpr int UPL = CH / At::G;             // chunks per lane per row per k-tile
  constexpr int S = UPL / At::UNITS;          // fragment substeps per k-tile
  static_assert(UPL % At::UNITS == 0, "k-tile must hold whole atoms");
  static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must hold whole atoms");
  static_assert(S == 1 || S % 2 == 0, "fragment double buffering needs an even substep count");
  // The next tile's staging registers are written to LDS (and the tile after it is requested)
  // two substeps before the end of the current one, leaving the loads a whole k-tile of MFMA
  // work to arrive.
  constexpr int SW = S >= 2 ? S - 2 : 0;

  __shared__ u32x4 lds[2][(BM + BN) * CH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  tile_of(p, pid, nwg, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm = wave % WM, wn = wave / WM;

  acc_t acc[RM][RN];
  static_for<RM>([&](auto i) { static_for<RN>([&](auto j) { acc[i][j] = acc_t{}; }); });

  typename PickLoader<DT, AK, VEC, BM, BKE, NT>::type la;
  typename PickLoader<DT, BKM, VEC, BN, BKE, NT>::type lb;
  const KRange kr = k_range(p);
  la.init(advance_k<DT, AK>(p.A, p.lda, kr.begin), p.lda, m0, p.M, kr.len, tid);
  lb.init(advance_k<DT, BKM>(p.B, p.ldb, kr.begin), p.ldb, n0, p.N, kr.len, tid);

  const int nk = (int)((kr.len + BKE - 1) / BKE);
  const int nfull = (int)(kr.len / BKE);

  // fragment addressing: lane row within an atom, and lane group along k
  const int frow = frag_row<DT, MI>(lane), fgrp = frag_chunk<DT, MI>(lane);
  u32x4 fa[2][RM][At::UNITS], fb[2][RN][At::UNITS];
  // an MN-major operand tile kept as rows of k is read with transposing reads (the chunk c of
  // the K-major layout is the k run 8c .. 8c + 7)
  constexpr bool ROWS_A = RowsLayout<DT, AK, VEC, BM>::value, ROWS_B = RowsLayout<DT, BKM, VEC, BN>::value;
  auto read_frags = [&](auto buf, const u32x4* stage, auto sub) {
    const u32x4* As = stage;
    const u32x4* Bs = stage + BM * CH;
    static_for<At::UNITS>([&](auto x) {
      const int c = fgrp + At::G * (sub * At::UNITS + x);
      static_for<RM>([&](auto i) {
        if constexpr (ROWS_A)
          fa[buf][i][x] = read_rows_frag<BM * SZ / 16>(As, c * (16 / SZ), wm * WTM + i * MI, frow, lane);
        else
          fa[buf][i][x] = As[lds_slot<CH>(wm * WTM + i * MI + frow, c)];
      });
      static_for<RN>([&](auto j) {
        if constexpr (ROWS_B)
          fb[buf][j][x] = read_rows_frag<BN * SZ / 16>(Bs, c * (16 / SZ), wn * WTN + j * MI, frow, lane);
        else
          fb[buf][j][x] = Bs[lds_slot<CH>(wn * WTN + j * MI + frow, c)];
      });
    });
  };
  auto load_tile = [&](int t) {
    const int64_t k0 = (int64_t)t * BKE;
    if (t < nfull) {
      la.template load<false>(k0);
      lb.template load<false>(k0);
    } else {
      la.template load<true>(k0);
      lb.template load<true>(k0);
    }
  };

  if (nk > 0) {
    load_tile(0);
    la.store(lds[0], tid);
    lb.store(lds[0] + BM * CH, tid);
    if (nk > 1) load_tile(1);
    __syncthreads();
    read_frags(std::integral_constant<int, 0>{}, lds[0], std::integral_constant<int, 0>{});

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      static_for<S>([&](auto s) {
        constexpr int bf = (S == 1) ? 0 : (s & 1);
        if constexpr (s + 1 < S)
          read_frags(std::integral_constant<int, (s + 1) & 1>{}, lds[cur],
                     std::integral_constant<int, s + 1>{});
        if constexpr (s == SW) {
          if (kt + 1 < nk) {
            la.store(lds[cur ^ 1], tid);
            lb.store(lds[cur ^ 1] + BM * CH, tid);
            if (kt + 2 < nk) load_tile(kt + 2);
          }
        }
        static_for<At::PER_UNIT>([&](auto u) {
          static_for<RM>([&](auto i) {
            static_for<RN>([&](auto j) { At::mma(acc[i][j], fa[bf][i], fb[bf][j], u); });
          });
        });
      });
      __syncthreads();
      if (kt + 1 < nk)
        read_frags(std::integral_constant<int, 0>{}, lds[cur ^ 1], std::integral_constant<int, 0>{});
    }
  }

  KParams pe;
  problem_view<BM>(reload_args(), pe, pid, nwg);
  if (pe.split_k > 1) {
    store_partial<DT, MI, BM, BN, WTM, WTN>(pe, acc, m0, n0, wm, wn, lane);
  } else {
    epilogue<DT, MI, BM, BN, WTM, WTN, RM, RN, NT, sizeof(lds)>(pe, acc, &lds[0][0], m0, n0, wm, wn,
                                                                lane, tid, nk == 0);
  }
}

// ------------------------------------------------------------------------------------------
// The streaming kernel: global -> LDS by DMA (buffer_load ... lds), a ring of LDS stages.
//
// Each LDS stage holds the A and B tiles of one k-tile as 64-byte rows (BK = 64 / esize
// elements).  A wave-wide buffer_load_dwordx4 with the lds modifier writes 64 lanes x 16 bytes
// to one contiguous kilobyte of LDS (16 rows) without passing through registers, so the tiles
// of the next STAGES-1 k-tiles can be in flight at once: the loads get about STAGES-1 k-tiles of
// MFMA work to arrive instead of one ("CuTe DSL / CUDA Tile" post, "Pipelining hides a wait":
// buffering lets the slower stage set the pace; "CUTLASS", Part IV Stage 4: the multistage ring
// of shared-memory buffers).  Swizzle: chunk c of row r lives at slot c ^ ((r >> 2) & 3), so the
// 16 consecutive rows one ds_read_b128 phase reads at one logical chunk hit 16 different
// 16-byte bank groups; the DMA lane that owns a slot fetches the logical chunk that belongs
// there.  Rows past M or N and chunks past K are out of the buffer's range and land as zeros.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// XOR key of a row: 16 consecutive rows (one ds_read_b128 phase) must cover all 16 16-byte
// positions of a 256-byte bank window.  With 64-byte rows four rows share a window, so rows
// r, r+4, r+8, r+12 need different keys: (r >> 2) & 3, Swizzle<2,0,4> on the chunk offset.
// With 128-byte rows two rows share a window: (r >> 1) & 7, Swizzle<3,0,4>, as in the
// register-staged kernel (atom_maps.h).
template <int CH> __device__ __forceinline__ int row_key(int row) {
  static_assert(CH == 4 || CH == 8, "64- or 128-byte rows");
  return swizzled_slot<CH>(row, 0) - row * CH;
}
template <int CH> __device__ __forceinline__ int dslot(int row, int chunk) {
  return swizzled_slot<CH>(row, chunk);
}

// s_waitcnt with vmcnt = V (and lgkmcnt = 0 when LGKM0), other counters left free.
template <int V, bool LGKM0>
__device__ __forceinline__ void wait_counts() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  constexpr int imm = (V & 15) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8) | ((V >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier without a hardware memory fence (the waits above are explicit); the
// single-thread signal fences only keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Values that are the same in every lane, passed through readfirstlane so the compiler keeps
// them in scalar registers (buffer descriptors must be scalar; a value it cannot prove uniform
// gets a readfirstlane loop around every use).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  return (const char*)(uintptr_t)uniform_i64((int64_t)(uintptr_t)p);
}

template <int DT, int BM, int BN, int WM, int WN, int MI, int STAGES, int OCC, int CH>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_dma(const KParams p_) {
  KParams p;
  int pid, nwg;
  if (!problem_view<BM>(p_, p, pid, nwg)) return;
  typedef Atom<DT, MI> At;
  typedef typename At::acc_t acc_t;
  constexpr int NW = WM * WN, NT = NW * 64;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int BKE = CH * 16 / SZ;           // elements per k-tile (64- or 128-byte rows)
  constexpr int VE = 16 / SZ;
  constexpr int RPB = 64 / CH;                // rows per 1-KiB DMA block
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int RM = WTM / MI, RN = WTN / MI;
  constexpr int UPL = CH / At::G;             // chunks per lane per row per k-tile
  constexpr int S = UPL / At::UNITS;          // fragment substeps per k-tile
  constexpr int DA = BM / RPB / NW, DB = BN / RPB / NW;  // DMA instructions per wave per k-tile
  constexpr int DPT = DA + DB;
  constexpr int STAGE = (BM + BN) * CH;       // chunks per stage
  static_assert(UPL % At::UNITS == 0 && S >= 1, "k-tile must hold whole atoms");
  static_assert(BM % (RPB * NW) == 0 && BN % (RPB * NW) == 0, "whole DMA blocks per wave");
  static_assert(STAGES >= 2 && (STAGES - 2) * DPT < 64, "stage count");
  static_assert(RM % 2 == 0, "the last substep is issued in two halves");

  __shared__ u32x4 lds[STAGES * STAGE];

  // the wave index is uniform across a wave; saying so keeps M0 (the DMA's LDS address) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_of(p, pid, nwg, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm = wave % WM, wn = wave / WM;

  acc_t acc[RM][RN];
  static_for<RM>([&](auto i) { static_for<RN>([&](auto j) { acc[i][j] = acc_t{}; }); });

  // DMA addressing: lane l of a block fills slot l of a kilobyte, i.e. row l/CH, slot l%CH of
  // the block, which holds logical chunk (l%CH) ^ key(row).
  const char* a_tile = uniform_ptr((const char*)p.A + m0 * p.lda * SZ);
  const char* b_tile = uniform_ptr((const char*)p.B + n0 * p.ldb * SZ);
  const int64_t a_span = uniform_i64(((p.M - m0 - 1) * p.lda + p.K) * SZ);
  const int64_t b_span = uniform_i64(((min((int64_t)BN, p.N - n0) - 1) * p.ldb + p.K) * SZ);
  // per-lane source of DMA instruction i (rows blk*RPB + lane/CH of the tile)
  auto src_off = [&](int blk, int64_t ld, int& kc) -> uint32_t {
    const int row = blk * RPB + lane / CH;
    const int c = (lane % CH) ^ row_key<CH>(row);
    kc = c * VE;
    return (uint32_t)(row * ld * SZ + c * 16);
  };

  const int nk = (int)((p.K + BKE - 1) / BKE);

  // Tile t into stage t % STAGES.  Tiles past the end of K are all out of range (zeros) and are
  // issued anyway so every wave always has the same number of DMA operations in flight.
  auto dma = [&](int t) {
    const int64_t k0 = (int64_t)t * BKE;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile, a_span);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_tile, b_span);
    u32x4* st = lds + (t % STAGES) * STAGE;
    static_for<DA>([&](auto i) {
      const int blk = wave + NW * i;
      int kc;
      const uint32_t off = src_off(blk, p.lda, kc);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(st + blk * 64), 16,
                                               k0 + kc < p.K ? off : 0x80000000u,
                                               (int)(k0 * SZ), 0, 0);
    });
    static_for<DB>([&](auto i) {
      const int blk = wave + NW * i;
      int kc;
      const uint32_t off = src_off(blk, p.ldb, kc);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(st + BM * CH + blk * 64), 16,
                                               k0 + kc < p.K ? off : 0x80000000u,
                                               (int)(k0 * SZ), 0, 0);
    });
  };

  const int frow = frag_row<DT, MI>(lane), fgrp = frag_chunk<DT, MI>(lane);
  u32x4 fa[2][RM][At::UNITS], fb[2][RN][At::UNITS];
  auto read_frags = [&](auto buf, const u32x4* st, auto sub) {
    static_for<At::UNITS>([&](auto x) {
      const int c = fgrp + At::G * (sub * At::UNITS + x);
      static_for<RM>([&](auto i) { fa[buf][i][x] = st[dslot<CH>(wm * WTM + i * MI + frow, c)]; });
      static_for<RN>([&](auto j) { fb[buf][j][x] = st[BM * CH + dslot<CH>(wn * WTN + j * MI + frow, c)]; });
    });
  };
  auto mma_rows = [&](auto buf, auto i0, auto i1) {
    static_for<At::PER_UNIT>([&](auto u) {
      static_for<i1 - i0>([&](auto ii) {
        static_for<RN>([&](auto j) { At::mma(acc[i0 + ii][j], fa[buf][i0 + ii], fb[buf][j], u); });
      });
    });
  };

  if (nk > 0) {
    static_for<STAGES - 1>([&](auto t) { dma(t); });
    wait_counts<(STAGES - 2) * DPT, true>();
    barrier_nofence();
    read_frags(std::integral_constant<int, 0>{}, lds, std::integral_constant<int, 0>{});

    // One k-tile: DMA of tile t+STAGES-1, fragment substeps of tile t, and before its last half
    // of MFMAs the barrier that makes tile t+1 readable.  KK is the parity of t when the
    // fragment buffers alternate between tiles (an odd substep count).
    auto tile_step = [&](int t, auto KK) {
      // stage (t-1) % STAGES was released by the barrier that ended tile t-1
      dma(t + STAGES - 1);
      const u32x4* st = lds + (t % STAGES) * STAGE;
      static_for<S>([&](auto s) {
        constexpr int buf = (KK * S + s) & 1;
        if constexpr (s + 1 < S) {
          read_frags(std::integral_constant<int, buf ^ 1>{}, st, std::integral_constant<int, s + 1>{});
          mma_rows(std::integral_constant<int, buf>{}, std::integral_constant<int, 0>{},
                   std::integral_constant<int, RM>{});
        } else {
          mma_rows(std::integral_constant<int, buf>{}, std::integral_constant<int, 0>{},
                   std::integral_constant<int, RM / 2>{});
          // tile t+1 has landed once at most STAGES-2 tiles of DMA are still in flight
          wait_counts<(STAGES - 2) * DPT, true>();
          barrier_nofence();
          // (after the last tile this reads a stale stage; the values are never used)
          read_frags(std::integral_constant<int, buf ^ 1>{}, lds + ((t + 1) % STAGES) * STAGE,
                     std::integral_constant<int, 0>{});
          mma_rows(std::integral_constant<int, buf>{}, std::integral_constant<int, RM / 2>{},
                   std::integral_constant<int, RM>{});
        }
      });
    };
    if constexpr (S % 2 == 0) {
      for (int kt = 0; kt < nk; ++kt) tile_step(kt, std::integral_constant<int, 0>{});
    } else {
      // Fragment buffers alternate between tiles: walk tiles in pairs.  An odd tile count runs
      // one extra tile past K, which the DMA fills with zeros, so it adds exact zeros.
      for (int kt = 0; kt < nk; kt += 2) {
        tile_step(kt, std::integral_constant<int, 0>{});
        tile_step(kt + 1, std::integral_constant<int, 1>{});
      }
    }
    wait_counts<0, true>();  // the zero-filled tiles issued past the end are still in flight
    barrier_nofence();
  }
  KParams pe;
  problem_view<BM>(reload_args(), pe, pid, nwg);
  epilogue<DT, MI, BM, BN, WTM, WTN, RM, RN, NT, sizeof(lds)>(pe, acc, lds, m0, n0, wm, wn, lane,
                                                              tid, nk == 0);
}

template <int DT, int BM, int BN, int WM, int WN, int MI, int STAGES, int OCC, int CH>
static hipError_t launch_dma(const KParams& p, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((gemm_dma<DT, BM, BN, WM, WN, MI, STAGES, OCC, CH>), grid,
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The split-ring kernel: a 256 x 256 workgroup tile whose A and B k-tiles travel in separate
// LDS rings, so the loads of a k-tile get more than one k-tile of MFMA work to arrive within
// the 160 KiB of LDS.
//
// A stage of a 256 x 256 tile with 128-byte rows (one cache line per row per k-tile, the
// cheapest DMA pattern) holds 64 KiB, so only two whole stages fit and each k-tile's loads
// would get exactly one k-tile of compute to land ("CuTe DSL / CUDA Tile" post, "Pipelining
// hides a wait": the slower of load and compute sets the interval; "CUTLASS", Part IV Stage 4:
// the multistage ring).  Here the unit of buffering is half a stage (32 KiB, the A or the B
// tile of one k-tile) and the 5 units of LDS are split into two rings:
//   * A: 3 slots.  A(t+2) is issued during the first substep of k-tile t, into the slot A(t-1)
//     released, and is read at the start of k-tile t+2: two k-tiles of lead.
//   * B: 2 slots.  Every wave reads all of its B fragments of k-tile t at the start of the
//     k-tile; after half of the MFMA substeps a barrier confirms that no wave still reads B(t),
//     and B(t+2) is issued into that slot during the next substep: one and a half k-tiles of
//     lead.
// The end-of-tile wait leaves A(t+2) and B(t+2) in flight and needs only A(t+1), B(t+1).
// With NB = 1 there is no mid-tile barrier: B(t+2) and A(t+3) are issued after the end-of-tile
// barrier of k-tile t (one and two k-tiles of lead).  The DMA instructions are spread among the
// MFMAs of the substep that issues them (see `interleave`).
// Summation order per output is the same as the two-stage DMA kernel's (k-tiles in order,
// substeps in order), so both produce the same bits.
// ------------------------------------------------------------------------------------------
template <int DT, int WM, int WN, int MI, int NB, bool BKM, bool SK>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_ring(const KParams p_) {
  KParams p;
  int pid, nwg;
  if (!problem_view<256>(p_, p, pid, nwg)) return;
  typedef Atom<DT, MI> At;
  typedef typename At::acc_t acc_t;
  constexpr int BM = 256, BN = 256, CH = 8;   // 128-byte LDS rows
  constexpr int NW = WM * WN, NT = NW * 64;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int BKE = CH * 16 / SZ;           // elements per k-tile
  constexpr int VE = 16 / SZ;
  constexpr int RPB = 64 / CH;                // rows per 1-KiB DMA block
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int RM = WTM / MI, RN = WTN / MI;
  constexpr int UPL = CH / At::G;             // chunks per lane per row per k-tile
  constexpr int S = UPL / At::UNITS;          // fragment substeps per k-tile
  constexpr int DU = BM / RPB / NW;           // DMA instructions per wave per unit
  constexpr int SLOT = BM * CH;               // 16-byte chunks per unit (32 KiB)
  constexpr int MID = S / 2;                  // substeps before B's slot is released
  static_assert(BM == BN, "A and B units share one slot size");
  static_assert(UPL % At::UNITS == 0 && S % 2 == 0, "whole, evenly many substeps");
  static_assert(RM % 2 == 0, "the last substep is issued in two halves");
  static_assert(BM % (RPB * NW) == 0, "whole DMA blocks per wave");

  __shared__ u32x4 lds[5 * SLOT];  // slots 0..2: A ring; 3..4: B ring

  // Output tile (tm, tn) over the K range kr: the whole product's K, this workgroup's slice of
  // a split, or (slot >= 0) a Stream-K piece of the tile, stored raw to that workspace slot.
  auto run_tile = [&](int tm, int tn, const KRange kr, int slot) {
    // The thread index passes through an empty asm here, so that nothing derived from it is
    // hoisted out of a Stream-K workgroup's loop over tiles and held in registers across every
    // tile's main loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    acc_t acc[RM][RN];
    static_for<RM>([&](auto i) { static_for<RN>([&](auto j) { acc[i][j] = acc_t{}; }); });

    const int64_t K = uniform_i64(kr.len);
    const char* a_tile = uniform_ptr((const char*)p.A + (m0 * p.lda + kr.begin) * SZ);
    // B K-major: the tile's first column at its first k; B N-major (row-major): its first k row
    // at its first column
    const char* b_tile = uniform_ptr((const char*)p.B + (BKM ? n0 * p.ldb + kr.begin : kr.begin * p.ldb + n0) * SZ);
    const int64_t a_span = uniform_i64(((p.M - m0 - 1) * p.lda + K) * SZ);
    const int64_t b_span = uniform_i64(BKM ? ((min((int64_t)BN, p.N - n0) - 1) * p.ldb + K) * SZ
                                           : ((K - 1) * p.ldb + (p.N - n0)) * SZ);
    // Lane l of DMA block blk fills slot l of a kilobyte: row blk * RPB + l / CH, slot l % CH,
    // which holds logical chunk (l % CH) ^ key(row).  A wave's blocks are NW apart, so its rows
    // differ by multiples of RPB * NW; the key takes row bits 1..3 (2..3 for 64-byte rows), so
    // with RPB * NW a multiple of 16 every block of the wave has the same chunk per lane, and the
    // source offsets differ only by a uniform row stride.
    static_assert((RPB * NW) % 16 == 0, "one chunk per lane across a wave's DMA blocks");
    const int row0 = wave * RPB + lane / CH;
    const int kc = ((lane % CH) ^ row_key<CH>(row0)) * VE;  // this lane's first k of its chunk
    const uint32_t a_off0 = (uint32_t)(row0 * p.lda * SZ + kc * SZ);
    // B N-major: a k-tile is BKE rows of BN elements (CHR chunks, slot mn_slot); lane l of DMA
    // block blk fills row blk * 2 + l / CHR, slot l % CHR, which holds logical chunk
    // (l % CHR) ^ mn_key(row).  A wave's blocks are NW apart, i.e. rows 2 NW apart, and mn_key
    // takes row bits 0..3, so with 2 NW a multiple of 16 every block has the same chunk per lane.
    constexpr int CHR = BN * SZ / 16, RPBR = 64 / CHR;
    static_assert(BKM || (RPBR * NW) % 16 == 0, "one chunk per lane across a wave's B blocks");
    static_assert(BKM || BKE / RPBR == BN / RPB, "a B unit takes as many DMA blocks either way");
    const int brow0 = wave * RPBR + lane / CHR;
    const uint32_t b_off0 = BKM ? (uint32_t)(row0 * p.ldb * SZ + kc * SZ)
                                : (uint32_t)((brow0 * p.ldb + ((lane % CHR) ^ mn_key(brow0)) * VE) * SZ);
    const int nk = (int)((K + BKE - 1) / BKE);

    // Unit OP (0: A, 1: B) of k-tile t into `slot`.  Units past the end of K are all out of range
    // (zeros) and are issued anyway, so the wait counts stay the same on every k-tile.
    auto dma = [&](auto OP, int t, int slot) {
      const int64_t k0 = (int64_t)t * BKE;
      // elements of this k-tile inside K (at most BKE; zero or less past the end): the per-lane
      // tail check is one 32-bit compare against this uniform value
      const int rem = (int)min(K - k0, (int64_t)BKE);
      u32x4* st = lds + slot * SLOT;
      if constexpr (OP == 1 && !BKM) {
        // rows of k: the k advance moves the descriptor's base, so the range check (on the VGPR
        // offset) covers every row and column read; rows past K read zero
        const int64_t adv = k0 * p.ldb * SZ;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(b_tile + adv, b_span - adv);
        const uint32_t step = (uint32_t)(p.ldb * (RPBR * NW * SZ));
        uint32_t off0 = b_off0;
        asm volatile("" : "+v"(off0));
        static_for<DU>([&](auto i) {
          const int blk = wave + NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(st + blk * 64), 16,
                                                   brow0 + RPBR * NW * i < rem ? off0 + (uint32_t)i * step : kOobOffset,
                                                   0, 0, 0);
        });
      } else {
        const __amdgpu_buffer_rsrc_t r = OP == 0 ? make_rsrc(a_tile, a_span) : make_rsrc(b_tile, b_span);
        const uint32_t step = (uint32_t)((OP == 0 ? p.lda : p.ldb) * (RPB * NW * SZ));
        // The base passes through an empty asm so that the per-block sums are formed here, at the
        // issue, and not hoisted out of the k-loop as DU more live registers per operand.
        uint32_t off0 = OP == 0 ? a_off0 : b_off0;
        asm volatile("" : "+v"(off0));
        const bool in_k = kc < rem;
        static_for<DU>([&](auto i) {
          const int blk = wave + NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(st + blk * 64), 16,
                                                   in_k ? off0 + (uint32_t)i * step : kOobOffset,
                                                   (int)(k0 * SZ), 0, 0);
        });
      }
    };

    const int frow = frag_row<DT, MI>(lane), fgrp = frag_chunk<DT, MI>(lane);
    u32x4 fa[2][RM][At::UNITS], fb[S][RN][At::UNITS];
    auto read_a = [&](auto buf, const u32x4* sa, auto sub) {
      static_for<At::UNITS>([&](auto x) {
        const int c = fgrp + At::G * (sub * At::UNITS + x);
        static_for<RM>([&](auto i) { fa[buf][i][x] = sa[dslot<CH>(wm * WTM + i * MI + frow, c)]; });
      });
    };
    auto read_b = [&](const u32x4* sb, auto sub) {
      static_for<At::UNITS>([&](auto x) {
        const int c = fgrp + At::G * (sub * At::UNITS + x);
        static_for<RN>([&](auto j) {
          if constexpr (BKM)
            fb[sub][j][x] = sb[dslot<CH>(wn * WTN + j * MI + frow, c)];
          else
            fb[sub][j][x] = read_rows_frag<CHR>(sb, c * VE, wn * WTN + j * MI, frow, lane);
        });
      });
    };
    // LDS read instructions per B fragment (two transposing reads from rows of k)
    constexpr int RB = BKM ? 1 : 2;
    auto mma_rows = [&](auto buf, auto sub, auto i0, auto i1) {
      static_for<At::PER_UNIT>([&](auto u) {
        static_for<i1 - i0>([&](auto ii) {
          static_for<RN>([&](auto j) { At::mma(acc[i0 + ii][j], fa[buf][i0 + ii], fb[sub][j], u); });
        });
      });
    };
    constexpr std::integral_constant<int, 0> OPA{};
    constexpr std::integral_constant<int, 1> OPB{};
    typedef std::integral_constant<int, 0> I0;
    // Scheduling hint for one region: spread its NVM DMA instructions and NDS LDS reads (the next
    // substep's fragments) evenly among its NMF MFMAs, then fence the region.  Left alone, the
    // scheduler issues each read just before the MFMA that needs it (every MFMA then waits for an
    // LDS round trip), bunches the DMA issue, and moves MFMAs across the barriers, which with one
    // or two waves per SIMD leaves the matrix pipe idle at every barrier.
    auto interleave = [&](auto NVM, auto NDS, auto NMF) {
      constexpr int nvm = NVM, nds = NDS, nmf = NMF;
      constexpr int ng = nvm > nds ? nvm : nds;
      if constexpr (ng > 0) {
        constexpr int per = (nmf + ng - 1) / ng;
        static_for<ng>([&](auto g) {
          if constexpr (g < nvm) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one DMA
          if constexpr (g < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, per, 0);                        // MFMAs
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    typedef std::integral_constant<int, 0> Z;

    if (nk > 0) {
      dma(OPA, 0, 0);
      dma(OPB, 0, 3);
      dma(OPA, 1, 1);
      dma(OPB, 1, 4);
      wait_counts<2 * DU, true>();
      barrier_nofence();
      if constexpr (NB == 1) dma(OPA, 2, 2);  // the third A slot is free from the start
      read_a(I0{}, lds, I0{});
      read_b(lds + 3 * SLOT, I0{});
      // Substep s of k-tile t, whose A unit sits in slot sa_i.
      auto substep = [&](int t, int sa_i, auto s) {
        constexpr int buf = s & 1;
        const int sb_i = 3 + (t & 1);
        const u32x4* sa = lds + sa_i * SLOT;
        // With two barriers per k-tile, A(t+2) is issued in substep 0, into the slot A(t-1)
        // released, and B(t+2) in substep MID, after the barrier that released B(t)'s slot.
        constexpr int nvm = NB == 2 ? (s == 0 ? DU : 0) + (s == MID ? DU : 0) : 0;
        if constexpr (NB == 2 && s == 0) dma(OPA, t + 2, sa_i == 0 ? 2 : sa_i - 1);
        if constexpr (NB == 2 && s == MID) dma(OPB, t + 2, sb_i);
        if constexpr (s + 1 < S) {
          read_a(std::integral_constant<int, buf ^ 1>{}, sa, std::integral_constant<int, s + 1>{});
          mma_rows(std::integral_constant<int, buf>{}, s, I0{}, std::integral_constant<int, RM>{});
          // the first substep also carries the B reads of the rest of the k-tile
          interleave(std::integral_constant<int, nvm>{},
                     std::integral_constant<int, RM * At::UNITS + (s == 0 ? (S - 1) * RN * At::UNITS * RB : 0)>{},
                     std::integral_constant<int, RM * RN * At::PER_UNIT>{});
          if constexpr (s + 1 == MID && NB == 2) {
            // this wave's reads of B(t) are complete (lgkmcnt 0); after the barrier no wave
            // reads B(t), and B(t+2) may take its slot
            wait_counts<63, true>();
            barrier_nofence();
          }
        } else {
          mma_rows(std::integral_constant<int, buf>{}, s, I0{}, std::integral_constant<int, RM / 2>{});
          // these MFMAs stay before the barrier
          interleave(std::integral_constant<int, nvm>{}, Z{},
                     std::integral_constant<int, RM / 2 * RN * At::PER_UNIT>{});
          // A(t+1) and B(t+1) have landed once at most A(t+2), B(t+2) are in flight (one barrier
          // per k-tile: once at most A(t+2), issued after B(t+1), is)
          if constexpr (NB == 2) wait_counts<2 * DU, true>(); else wait_counts<DU, true>();
          barrier_nofence();
          // (after the last k-tile these read zero-filled slots; the values are never used).  B
          // first: the next substep's first MFMAs need A fragment 0 and every B fragment
          const int na = sa_i == 2 ? 0 : sa_i + 1;
          read_b(lds + (3 + ((t + 1) & 1)) * SLOT, I0{});
          read_a(std::integral_constant<int, buf ^ 1>{}, lds + na * SLOT, I0{});
          if constexpr (NB == 1) {
            // every wave is past k-tile t: B(t+2) and A(t+3) take the slots of B(t) and A(t).
            // Issued after the reads above, so the compiler cannot move those reads across the
            // loop's back edge (the DMA may alias them).
            dma(OPB, t + 2, sb_i);
            dma(OPA, t + 3, sa_i);
          }
          mma_rows(std::integral_constant<int, buf>{}, s, std::integral_constant<int, RM / 2>{},
                   std::integral_constant<int, RM>{});
          interleave(std::integral_constant<int, NB == 1 ? 2 * DU : 0>{},
                     std::integral_constant<int, (RM + RN * RB) * At::UNITS>{},
                     std::integral_constant<int, RM / 2 * RN * At::PER_UNIT>{});
        }
      };
      // First half of k-tile t: read the rest of the k-tile's B fragments, substeps 0 .. MID-1
      // (ending with the barrier that releases B(t)).
      auto tile_front = [&](int t, int sa_i) {
        const u32x4* sb = lds + (3 + (t & 1)) * SLOT;
        static_for<S - 1>([&](auto s) { read_b(sb, std::integral_constant<int, s + 1>{}); });
        static_for<MID>([&](auto s) { substep(t, sa_i, s); });
      };
      auto tile_back = [&](int t, int sa_i) {
        static_for<S - MID>([&](auto s) { substep(t, sa_i, std::integral_constant<int, MID + s>{}); });
      };
      // The loop turns at the B-release barrier in the middle of a k-tile.  Turning at the k-tile
      // boundary instead lets the compiler merge the next k-tile's first fragment reads with the
      // prologue's and sink them to the loop head, right before the MFMAs that consume them, so
      // every k-tile would start with an exposed LDS round trip on all waves at once; nothing
      // can be moved across the barrier and DMA that end each half here.
      int sa_i = 0;  // slot of A(t) in the A ring
      if constexpr (NB == 2) {
        tile_front(0, 0);
        for (int t = 0; t + 1 < nk; ++t) {
          tile_back(t, sa_i);
          sa_i = sa_i == 2 ? 0 : sa_i + 1;
          tile_front(t + 1, sa_i);
        }
        tile_back(nk - 1, sa_i);
      } else {
        for (int t = 0; t < nk; ++t) {
          tile_front(t, sa_i);
          tile_back(t, sa_i);
          sa_i = sa_i == 2 ? 0 : sa_i + 1;
        }
      }
      wait_counts<0, true>();  // the zero-filled units issued past the end are still in flight
      barrier_nofence();
    }
    KParams pe;
    int pid_e, nwg_e;
    problem_view<256>(reload_args(), pe, pid_e, nwg_e);
    if (SK && slot >= 0) {
      store_partial<DT, MI, BM, BN, WTM, WTN>(pe, acc, m0, n0, wm, wn, lane, slot);
    } else if (pe.split_k > 1) {
      store_partial<DT, MI, BM, BN, WTM, WTN>(pe, acc, m0, n0, wm, wn, lane);
    } else {
      epilogue<DT, MI, BM, BN, WTM, WTN, RM, RN, NT, sizeof(lds)>(pe, acc, lds, m0, n0, wm, wn, lane,
                                                                  tid, nk == 0);
    }
  };

  if constexpr (!SK) {
    int tm, tn;
    tile_of(p, pid, nwg, tm, tn);
    run_tile(tm, tn, k_range(p), -1);
  } else {
    // Stream-K: this workgroup's contiguous share of the k-tile iterations, tile by tile.  Its
    // place v in the sharing order puts the workgroups of one XCD (dispatch deals consecutive
    // ids to the 8 XCDs in turn) on consecutive shares, so neighbouring tiles, which share A
    // and B panels, are worked on under one L2.
    const int v = (pid & 7) * (p.sk_wgs >> 3) + (pid >> 3);
    const int64_t nkt = p.sk_nkt, I = (int64_t)p.sk_tiles * nkt;
    int64_t it = sk_start(I, p.sk_wgs, v);
    const int64_t end = sk_start(I, p.sk_wgs, v + 1);
    const int64_t first = it / nkt;
    while (it < end) {
      const int64_t t = it / nkt, kb = it - t * nkt, ke = min(nkt, kb + (end - it));
      int tm, tn;
      tile_walk(p, (int)(p.tile_base + t), tm, tn);
      const KRange kr{kb * BKE, min(p.K, ke * BKE) - kb * BKE};
      run_tile(tm, tn, kr, kb == 0 && ke == nkt ? -1 : (int)(2 * v + (t == first ? 0 : 1)));
      it += ke - kb;
      __syncthreads();  // no wave still reads this tile's LDS when the next tile's copies land
    }
  }
}

template <int DT, int WM, int WN, int MI, int NB, bool BKM, bool SK>
static hipError_t launch_ring(const KParams& p, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((gemm_ring<DT, WM, WN, MI, NB, BKM, SK>), grid, dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The skinny kernel: M <= 16 (a decode-like product), bound by streaming B from HBM.
//
// "CUTLASS" (stanleyjacob.dev), Part III: a tall-skinny GEMM has too few output tiles to fill
// the GPU and memory bandwidth, not the matrix units, sets the ceiling; splitting K restores
// occupancy (Part IV Stage 6).  A workgroup owns BN output columns and all M rows.  Its WK x WN
// waves form a grid: wave (wk, wn) reduces the wk-th of WK slices of K for the NBW 16-column
// blocks of column group wn (BN = WN * NBW * 16); the WK partial sums meet in LDS.  Every byte of
// B is used by exactly one MFMA, so B goes straight from HBM into registers (no LDS staging).
// A (M x K, a few hundred KiB) stays in L2; the WN waves that share a K slice read the same A
// lines, so after the first they hit in the CU's vector L1 and A costs the CU's memory pipe
// 1/WN of what it would if every wave read its own.  Atoms: 16x16xKSTEP MFMA (16x16x128 e4m3,
// 16x16x32 bf16/fp16) with the atoms' layouts (atom_maps.h): lane l supplies row (or column)
// l % 16 and the 16-byte chunks l / 16 (+ 4 for the second chunk of an e4m3 lane) of a k-step.
// ------------------------------------------------------------------------------------------
template <int DT, int WK, int WN, int NBW, int U, int OCC>
__global__ __launch_bounds__(WK * WN * 64, OCC) void gemm_skinny(const KParams p_) {
  const KParams p = batch_view(p_);
  typedef Atom<DT, 16> At;
  typedef typename At::acc_t acc_t;  // 4 floats: rows acc_row(l, r), column acc_col(l, r)
  constexpr int NT = WK * WN * 64;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int LB = At::UNITS * 16;          // bytes per lane per operand per MFMA
  constexpr int KSTEP = 4 * LB / SZ;          // elements of K per MFMA
  constexpr int BN = WN * NBW * 16;           // columns per workgroup
  static_assert(At::PER_UNIT == 1, "one MFMA per k-step");

  // partial sums of each K slice; rows padded to 17 floats so that the four 16-lane groups of a
  // store, which write rows 4 apart, fall on different banks
  __shared__ float part[WK][BN / 16][16][17];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave % WK, wn = wave / WK;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int lr = frag_row<DT, 16>(lane), lg = frag_chunk<DT, 16>(lane);

  // K split: wave (wk, .) owns k-steps [wk*per, min((wk+1)*per, nks))
  const int64_t nks = (p.K + KSTEP - 1) / KSTEP;
  const int64_t per = (nks + WK - 1) / WK;
  const int64_t ks0 = wk * per;
  const int64_t ks1 = min(ks0 + per, nks);

  // A rows lr (zero past M); B columns n0 + 16*b + lr (zero past N, or past this workgroup's
  // BN columns).  Offset of chunk x of a lane's k-runs within a k-step: (lg + 4x)*16 bytes.  Both
  // spans stay below 2^31 bytes (checked on the host), so the offset 0x80000000 is outside
  // either descriptor.
  const char* a_base = uniform_ptr((const char*)p.A);
  const char* b_base = uniform_ptr((const char*)p.B + n0 * p.ldb * SZ);
  const int64_t a_span = uniform_i64(((p.M - 1) * p.lda + p.K) * SZ);
  const int64_t b_span = uniform_i64(((min((int64_t)BN, p.N - n0) - 1) * p.ldb + p.K) * SZ);
  const uint32_t a_off = (uint32_t)(lr * p.lda * SZ + lg * 16);
  const uint32_t b_blk = (uint32_t)(16 * p.ldb * SZ);
  const uint32_t b_off = (uint32_t)(lr * p.ldb * SZ + lg * 16) + (uint32_t)(wn * NBW) * b_blk;

  acc_t acc[NBW];
  static_for<NBW>([&](auto b) { acc[b] = acc_t{}; });

  // Two register batches of U k-steps each: batch i+1 is in flight while batch i feeds the
  // MFMAs.  Chunks past K or past this wave's slice get an offset beyond every descriptor's
  // range, so the buffer unit returns zeros without touching memory (no select after the load,
  // no branch around it).
  struct Batch {
    u32x4 a[U][At::UNITS], b[U][NBW][At::UNITS];
  };
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, a_span);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, b_span);
  auto load = [&](Batch& f, int64_t ks) {
    static_for<U>([&](auto u) {
      const int64_t k0 = (ks + u) * KSTEP;
      const bool live = ks + u < ks1;
      static_for<At::UNITS>([&](auto x) {
        const int64_t kc = k0 + (lg + 4 * x) * (16 / SZ);  // first element of this chunk
        const bool ok = live && kc < p.K;
        const uint32_t ko = (uint32_t)(k0 * SZ) + x * 64;
        f.a[u][x] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? a_off + ko : 0x80000000u, 0, 0);
        static_for<NBW>([&](auto b) {
          f.b[u][b][x] = __builtin_amdgcn_raw_buffer_load_b128(
              rb, ok ? b_off + b * b_blk + ko : 0x80000000u, 0, 0);
        });
      });
    });
  };
  auto mma = [&](const Batch& f) {
    static_for<U>([&](auto u) {
      static_for<NBW>([&](auto b) { At::mma(acc[b], f.a[u], f.b[u][b], 0); });
    });
  };
  Batch f0, f1;
  load(f0, ks0);
  for (int64_t ks = ks0; ks < ks1; ks += 2 * U) {
    load(f1, ks + U);
    // loads stay ahead of the MFMAs that wait on the older batch
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    load(f0, ks + 2 * U);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // partial sums -> LDS; reduction over the WK slices; epilogue
  static_for<NBW>([&](auto b) {
    static_for<4>([&](auto r) {
      part[wk][wn * NBW + b][acc_row<DT, 16>(lane, r)][acc_col<DT, 16>(lane, r)] = acc[b][(int)r];
    });
  });
  __syncthreads();
  constexpr int ODT = out_dtype(DT);
  typedef Out<ODT> O;
  for (int q = tid; q < 16 * BN; q += NT) {
    const int row = q / BN, c = q % BN;
    const int64_t col = n0 + c;
    if (row >= p.M || col >= p.N) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WK; ++w) sum += part[w][c / 16][row][c % 16];
    O::store(p.D, row * p.d_sm + col * p.d_sn, finish_elem<ODT>(p, row, col, sum));
  }
}

template <int DT, int WK, int WN, int NBW, int U, int OCC>
static hipError_t launch_skinny(const KParams& p, hipStream_t s, dim3) {
  constexpr int BN = WN * NBW * 16;
  const dim3 grid((unsigned)((p.N + BN - 1) / BN), 1, (unsigned)p.batch);
  hipLaunchKernelGGL((gemm_skinny<DT, WK, WN, NBW, U, OCC>), grid, dim3(WK * WN * 64), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The streaming skinny kernel: M <= 16, B streamed from HBM into LDS by DMA.
//
// Same problem as gemm_skinny (a decode-like product whose cost is reading B once: "CUTLASS",
// Part III, memory bandwidth sets the ceiling), but B travels HBM -> LDS by buffer_load ... lds
// instead of into registers: each DMA instruction moves 8 columns x 128 bytes of K (whole cache
// lines), which streams from HBM markedly faster than 16-byte register loads of half lines.
// A workgroup owns BN = 16 * NBW columns; its WK waves split K into contiguous slices and each
// wave streams its slice through a private ring of R blocks (a block = 128 bytes of K for all BN
// columns of B and the 16 rows of A, which stay L2-resident), so no barrier is needed in the
// loop: a wave only waits for its own DMA, and no load in the loop targets registers.  R = 3
// keeps the workgroup at 72 KiB of LDS, two per CU, which streamed fastest on MI355X.  Within a
// block, chunk c (16 bytes) of LDS row r sits at slot c ^ ((r >> 1) & 7), so the 16 rows one
// ds_read_b128 phase reads fall in 16 different 16-byte bank groups.  The WK partial sums meet in
// LDS at the end.
// ------------------------------------------------------------------------------------------
template <int DT, int WK, int NBW, int R, int OCC>
__global__ __launch_bounds__(WK * 64, OCC) void gemm_skinny_dma(const KParams p_) {
  const KParams p = batch_view(p_);
  typedef Atom<DT, 16> At;
  typedef typename At::acc_t acc_t;               // 4 floats: rows acc_row(l, r), column acc_col(l, r)
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int BN = NBW * 16;                    // columns per workgroup
  constexpr int ROWS = BN + 16;                   // LDS rows per block: BN columns of B, 16 rows of A
  constexpr int BLK = 128;                        // bytes of K per row per block
  constexpr int BKE = BLK / SZ;                   // elements of K per block
  constexpr int MPB = 2 / At::UNITS;              // MFMAs per block (8 chunks / (4 groups * UNITS))
  constexpr int CPB = BN / 8;                     // B DMA instructions per block (8 rows each)
  constexpr int OPS = CPB + 2;                    // DMA instructions per block per wave (B, then A)
  constexpr int NT = WK * 64;
  static_assert(At::PER_UNIT == 1 && MPB * At::UNITS * 4 == 8, "a block is 8 chunks");
  static_assert((R - 2) * OPS < 64, "vmcnt range");

  __shared__ u32x4 ring[WK][R][ROWS * 8];        // [wave][block][row * 8 + slot]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int lr = frag_row<DT, 16>(lane), lg = frag_chunk<DT, 16>(lane);

  // This workgroup's K range: all of K, or with a split along K (too few column blocks to fill
  // the GPU) slice blockIdx.y.  Within it, wave w owns blocks [w*per, min((w+1)*per, nb)).
  const KRange kr = k_range(p);
  const int64_t K = uniform_i64(kr.len);
  const int64_t nb = (K + BKE - 1) / BKE;
  const int64_t per = (nb + WK - 1) / WK;
  const int64_t b0 = wave * per;
  const int nloc = (int)max((int64_t)0, min(b0 + per, nb) - b0);

  const char* a_base = uniform_ptr((const char*)p.A + kr.begin * SZ);
  const char* b_base = uniform_ptr((const char*)p.B + (n0 * p.ldb + kr.begin) * SZ);
  const int64_t a_span = uniform_i64(((p.M - 1) * p.lda + K) * SZ);
  const int64_t b_span = uniform_i64(((min((int64_t)BN, p.N - n0) - 1) * p.ldb + K) * SZ);
  const int64_t kbytes = K * SZ;
  // DMA lane: LDS row 8c + lane/8 of the block, slot lane%8, holding logical chunk slot ^ key(row)
  auto key = [](int row) { return row_key<8>(row); };

  acc_t acc[NBW];
  static_for<NBW>([&](auto b) { acc[b] = acc_t{}; });

  // Block j (local index) into ring slot `slot`.  Blocks past this wave's slice and chunks past K
  // are out of range (zeros) and are issued anyway, so every block costs exactly OPS counter slots.
  auto issue = [&](int j, auto slot) {
    const bool live = j < nloc;
    const int64_t kb = (b0 + j) * BLK;            // byte offset of the block along K
    const int sk = live ? (int)kb : 0;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, b_span);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, a_span);
    static_for<CPB + 2>([&](auto c) {
      constexpr bool IS_A = c >= CPB;
      const int row = 8 * c + (lane >> 3);        // LDS row; A rows are ROWS-16 .. ROWS-1
      const int src = IS_A ? row - BN : row;      // column of B or row of A
      const int ch = (lane & 7) ^ key(row);
      const bool ok = live && kb + ch * 16 < kbytes;
      const uint32_t off = (uint32_t)(src * (IS_A ? p.lda : p.ldb) * SZ + ch * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(IS_A ? ra : rb, (lds_void_t*)(&ring[wave][slot][c * 64]),
                                               16, ok ? off : 0x80000000u, sk, 0, 0);
    });
  };
  auto compute = [&](auto slot) {
    const u32x4* blk = &ring[wave][slot][0];
    static_for<MPB>([&](auto m) {
      u32x4 fa[At::UNITS];
      static_for<At::UNITS>([&](auto x) {
        const int row = BN + lr, chunk = lg + 4 * (m * At::UNITS + x);
        fa[x] = blk[row * 8 + (chunk ^ key(row))];
      });
      static_for<NBW>([&](auto b) {
        u32x4 fb[At::UNITS];
        static_for<At::UNITS>([&](auto x) {
          const int row = 16 * b + lr, chunk = lg + 4 * (m * At::UNITS + x);
          fb[x] = blk[row * 8 + (chunk ^ key(row))];
        });
        At::mma(acc[b], fa, fb, 0);
      });
    });
  };

  // R-1 blocks in flight; each step waits for the oldest, refills the slot computed on one step
  // earlier, then computes.  The trip count is rounded up to whole rings (the extra blocks are
  // zero-filled and add exact zeros) so the loop body has no branches.
  static_for<R - 1>([&](auto q) { issue(q, q); });
  for (int j = 0; j < nloc; j += R) {
    static_for<R>([&](auto q) {
      // block j+q has landed; lgkmcnt(0) also retires the reads of the slot refilled next
      wait_counts<(R - 2) * OPS, true>();
      issue(j + q + R - 1, std::integral_constant<int, (q + R - 1) % R>{});
      compute(q);
    });
  }
  wait_counts<0, true>();

  // partial sums -> LDS (reusing the ring); reduction over the WK slices; epilogue
  __syncthreads();
  // [WK][NBW][16][17]: rows padded to 17 floats so that the four 16-lane groups of a store, which
  // write rows 4 apart, fall on different banks
  float* part = reinterpret_cast<float*>(&ring[0][0][0]);
  static_assert(sizeof(ring) >= sizeof(float) * WK * NBW * 16 * 17, "reduction buffer");
  static_for<NBW>([&](auto b) {
    static_for<4>([&](auto r) {
      part[((wave * NBW + b) * 16 + acc_row<DT, 16>(lane, r)) * 17 + acc_col<DT, 16>(lane, r)] = acc[b][(int)r];
    });
  });
  __syncthreads();
  constexpr int ODT = out_dtype(DT);
  typedef Out<ODT> O;
  for (int q = tid; q < 16 * BN; q += NT) {
    const int row = q / BN, c = q % BN;
    const int64_t col = n0 + c;
    if (row >= p.M || col >= p.N) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WK; ++w) sum += part[((w * NBW + c / 16) * 16 + row) * 17 + c % 16];
    if (p.split_k > 1)  // raw sums of this K slice to its plane; gemm_splitk_reduce finishes
      p.workspace[(int64_t)blockIdx.y * p.M * p.N + row * p.N + col] = sum;
    else
      O::store(p.D, row * p.d_sm + col * p.d_sn, finish_elem<ODT>(p, row, col, sum));
  }
}

template <int DT, int WK, int NBW, int R, int OCC>
static hipError_t launch_skinny_dma(const KParams& p, hipStream_t s, dim3) {
  constexpr int BN = NBW * 16;
  const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)(p.split_k > 1 ? p.split_k : 1),
                  (unsigned)p.batch);
  hipLaunchKernelGGL((gemm_skinny_dma<DT, WK, NBW, R, OCC>), grid, dim3(WK * 64), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Launchers and the tile table.
// ------------------------------------------------------------------------------------------
template <int DT, bool AK, bool BKM, int VEC, int BM, int BN, int BKE, int WM, int WN, int MI>
static hipError_t launch_tiled(const KParams& p, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((gemm_tiled<DT, AK, BKM, VEC, BM, BN, BKE, WM, WN, MI>), grid,
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

// VEC 2 (realigned 2-byte loads) entries need no 16-byte alignment, so they count as element-
// aligned (vec 0) kernels
#define HT_TILED(NAME, DT, AK, BKM, VEC, BM, BN, BKE, WM, WN, MI)                                 \
  {NAME, DT, AK, BKM, (VEC) == 1, 0, BM, BN, BKE, WM * WN, 2, 2 * (BM + BN) * BKE * Ty<DT>::SZ, 64, \
   &launch_tiled<DT, AK, BKM, VEC, BM, BN, BKE, WM, WN, MI>, (VEC) == 2, MI, BKE * Ty<DT>::SZ / 16, \
   RowsLayout<DT, AK, VEC, BM>::value || RowsLayout<DT, BKM, VEC, BN>::value}

#define HT_DMA(NAME, DT, BM, BN, WM, WN, MI, ST, OCC, CH)                                      \
  {NAME, DT, 1, 1, 1, 0, BM, BN, CH * 16 / Ty<DT>::SZ, WM * WN, ST, ST * (BM + BN) * CH * 16, 1, \
   &launch_dma<DT, BM, BN, WM, WN, MI, ST, OCC, CH>, 0, MI, CH, 0}

// Split-ring entries: 256 x 256 tiles, 128-byte rows, 5 units of 32 KiB.  The _BN form takes a
// row-major (N-contiguous) B kept in LDS as rows of k.
#define HT_RING(NAME, DT, WM, WN, MI, NB)                                                          \
  {NAME, DT, 1, 1, 1, 0, 256, 256, 128 / Ty<DT>::SZ, WM * WN, 5, 5 * 256 * 128, 64,               \
   &launch_ring<DT, WM, WN, MI, NB, true, false>, 0, MI, 8, 0, nullptr}
#define HT_RING_BN(NAME, DT, WM, WN, MI, NB)                                                       \
  {NAME, DT, 1, 0, 1, 0, 256, 256, 128 / Ty<DT>::SZ, WM * WN, 5, 5 * 256 * 128, 64,               \
   &launch_ring<DT, WM, WN, MI, NB, false, false>, 0, MI, 8, 1, nullptr}
// The same entries with the Stream-K form of the kernel as well.  (The fp8 ring has none: its
// 256 registers are full, and the form's loop over tiles spilled and ran at half speed.)
#define HT_RING_SK(NAME, DT, WM, WN, MI, NB)                                                       \
  {NAME, DT, 1, 1, 1, 0, 256, 256, 128 / Ty<DT>::SZ, WM * WN, 5, 5 * 256 * 128, 64,               \
   &launch_ring<DT, WM, WN, MI, NB, true, false>, 0, MI, 8, 0,                                    \
   &launch_ring<DT, WM, WN, MI, NB, true, true>}
#define HT_RING_BN_SK(NAME, DT, WM, WN, MI, NB)                                                    \
  {NAME, DT, 1, 0, 1, 0, 256, 256, 128 / Ty<DT>::SZ, WM * WN, 5, 5 * 256 * 128, 64,               \
   &launch_ring<DT, WM, WN, MI, NB, false, false>, 0, MI, 8, 1,                                   \
   &launch_ring<DT, WM, WN, MI, NB, false, true>}

// Streaming skinny entries: bm = 16 rows, bn = 16*NBW columns, bk = one 128-byte block of K;
// K slices of whole blocks when the column blocks do not fill the GPU.
#define HT_SKINNY_DMA(NAME, DT, WK, NBW, R, OCC)                                                  \
  {NAME, DT, 1, 1, 1, 1, 16, NBW * 16, 128 / Ty<DT>::SZ, WK, R, WK * R * (NBW + 1) * 16 * 128, 64, \
   &launch_skinny_dma<DT, WK, NBW, R, OCC>, 0, 16, 8, 0}

// Skinny entries: bm = 16 rows, bn = WN*NBW*16 columns per workgroup, bk = one MFMA k-step (no
// LDS operand tiles).
#define HT_SKINNY(NAME, DT, WK, WN, NBW, U, OCC)                                                 \
  {NAME, DT, 1, 1, 1, 1, 16, WN * NBW * 16, 4 * Atom<DT, 16>::UNITS * 16 / Ty<DT>::SZ, WK * WN, \
   1, WK * WN * NBW * 16 * 16 * 4, 1, &launch_skinny<DT, WK, WN, NBW, U, OCC>, 0, 16, 0, 0}

}  // namespace htk
