// atom_maps.h -- the thread-to-data maps of the MFMA atoms and of the LDS tiles, written as
// shape:stride layout functions ("CUTLASS, CuTe, and CUDA Tile", introduction: a layout maps a
// coordinate to an offset by an inner product with the stride; "A10 - CuTe, CUTLASS & CuTile",
// section 3.3: an MMA atom's A, B and C fragments are layouts from (thread, value) to the
// (row, column) of the instruction's tile, and their sizes must close over the tile).
//
// Shared by the device kernels (which derive their fragment addressing and accumulator
// positions from these tables) and by the host API (which checks, once per atom, that each
// table agrees with the layout helper's evaluation of the same layout written in the pages'
// notation, and that it is a bijection onto the tile).
//
// Conventions.  Index i = lane + 64 * v runs over the 64 lanes of a wave (fastest) and the v
// values each lane holds.  The offset of an operand map is m + MI * k (A) or n + MI * k (B)
// within the MI x KI tile of one instruction; the offset of the accumulator map is m + MI * n.
// The lane modes come first and multiply to 64, so offset(lane + 64 v) = offset(lane) +
// offset(64 v).
//
// What the hardware fixes (CDNA4 MFMA on 64-lane waves, checked on the device by the index
// probe): lane l supplies row l % MI of A and column l % MI of B; the accumulator layouts below.
// The k that a (lane, value) slot carries is this library's labelling: A and B label slots
// identically, so the product sums the same terms whatever order the hardware assigns to k
// inside one instruction (the probe checks that slots with equal labels meet).
#pragma once

#include <stdint.h>

namespace htk {

// A flat layout of up to four modes; leftmost mode fastest.  `text` is the same function in the
// pages' notation, as the layout helper parses it.
struct AtomLayout {
  int n;
  int shape[4];
  int stride[4];
  const char* text;
};

__host__ __device__ constexpr int layout_eval(const AtomLayout& L, int idx) {
  int off = 0;
  for (int i = 0; i < L.n; ++i) {
    off += (idx % L.shape[i]) * L.stride[i];
    idx /= L.shape[i];
  }
  return off;
}
// the lane part and the value part of offset(lane + 64 v)
__host__ __device__ constexpr int lane_offset(const AtomLayout& L, int lane) { return layout_eval(L, lane); }
__host__ __device__ constexpr int value_offset(const AtomLayout& L, int v) { return layout_eval(L, 64 * v); }

// One MFMA atom: operand element type code (0 f32, 1 f16, 2 bf16, 3 e4m3), MI x MI output
// block, KI = k per instruction, VPL = operand values per lane, NACC = accumulators per lane.
// `op` is the A map and also the B map (B's offset is n + MI * k).
struct AtomMaps {
  int dtype, mi, ki, vpl, nacc;
  AtomLayout op, acc;
};

// 32 x 32 accumulator block: register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.  16 x 16: row 4 (l / 16) + r, column l % 16.
#define HT_ACC32 {4, {32, 2, 4, 4}, {32, 4, 1, 8}, "((32,2),(4,4)):((32,4),(1,8))"}
#define HT_ACC16 {3, {16, 4, 4, 0}, {16, 4, 1, 0}, "((16,4),4):((16,4),1)"}

// Operand maps.  16-bit types: lane l = l0 + MI g carries row l0 and k = 8 g + v (one 16-byte
// run).  e4m3: 32 bytes per lane as two 16-byte runs, k = 16 g + v for v < 16 and
// 16 (g + G) + (v - 16) beyond, with G = 64 / MI lane groups (the two runs are the two 16-byte
// chunks g and g + G of a k-step).  f32: one value per lane, k = g.
constexpr AtomMaps kAtomMaps[] = {
    {2, 32, 16, 8, 16, {3, {32, 2, 8, 0}, {1, 256, 32, 0}, "((32,2),8):((1,256),32)"}, HT_ACC32},
    {2, 16, 32, 8, 4, {3, {16, 4, 8, 0}, {1, 128, 16, 0}, "((16,4),8):((1,128),16)"}, HT_ACC16},
    {1, 32, 16, 8, 16, {3, {32, 2, 8, 0}, {1, 256, 32, 0}, "((32,2),8):((1,256),32)"}, HT_ACC32},
    {1, 16, 32, 8, 4, {3, {16, 4, 8, 0}, {1, 128, 16, 0}, "((16,4),8):((1,128),16)"}, HT_ACC16},
    {3, 32, 64, 32, 16, {4, {32, 2, 16, 2}, {1, 512, 32, 1024}, "((32,2),(16,2)):((1,512),(32,1024))"}, HT_ACC32},
    {3, 16, 128, 32, 4, {4, {16, 4, 16, 2}, {1, 256, 16, 1024}, "((16,4),(16,2)):((1,256),(16,1024))"}, HT_ACC16},
    {0, 32, 2, 1, 16, {2, {32, 2, 0, 0}, {1, 32, 0, 0}, "(32,2):(1,32)"}, HT_ACC32},
    {0, 16, 4, 1, 4, {2, {16, 4, 0, 0}, {1, 16, 0, 0}, "(16,4):(1,16)"}, HT_ACC16},
};
#undef HT_ACC32
#undef HT_ACC16
constexpr int kNumAtomMaps = (int)(sizeof(kAtomMaps) / sizeof(kAtomMaps[0]));

__host__ __device__ constexpr int atom_index(int dtype, int mi) {
  for (int i = 0; i < kNumAtomMaps; ++i)
    if (kAtomMaps[i].dtype == dtype && kAtomMaps[i].mi == mi) return i;
  return -1;
}

// The LDS tiles' XOR swizzle ("A10 - CuTe, CUTLASS & CuTile", section 3.4): Swizzle<B, M, S>
// maps an offset o to o ^ ((o & mask) >> S) with mask = (2^B - 1) << (M + S).  Offsets here
// count 16-byte chunks (M = 0) of a tile stored row after row.
__host__ __device__ constexpr int swizzle(int o, int bbits, int mbase, int sshift) {
  return o ^ ((o & (((1 << bbits) - 1) << (mbase + sshift))) >> sshift);
}
// Rows of 8 chunks (128 bytes): Swizzle<3,0,4>, i.e. chunk c of row r at slot c ^ ((r >> 1) & 7).
// Rows of 4 chunks (64 bytes): Swizzle<2,0,4>, i.e. c ^ ((r >> 2) & 3).
template <int CH> struct RowSwizzle;
template <> struct RowSwizzle<8> { static constexpr int B = 3, M = 0, S = 4; };
template <> struct RowSwizzle<4> { static constexpr int B = 2, M = 0, S = 4; };
template <int CH> __host__ __device__ constexpr int swizzled_slot(int row, int chunk) {
  return swizzle(row * CH + chunk, RowSwizzle<CH>::B, RowSwizzle<CH>::M, RowSwizzle<CH>::S);
}

// MN-major operand tiles (A stored M-contiguous, B N-contiguous): one LDS row per k holding the
// tile's R elements as CHR = R * esize / 16 >= 16 chunks, so that rows are copied untransposed
// and the MFMA fragments are assembled by transposing LDS reads (ds_read_b64_tr_b16: within
// each 16-lane group, lane i receives element i % 4 of the 8 bytes read by lanes 4j + i / 4,
// j = 0..3, so 16 lanes that address a 4 (k) x 16 (m or n) block receive 4 consecutive k of one
// column each).  Chunk c of row k sits at slot c ^ mn_key(k).  On the 16-chunk view
// o = 16 (k mod 16) + (c mod 16) this is Swizzle<2,2,2> followed by Swizzle<1,1,6>.  The 32
// lanes that one 8-byte read phase serves then touch 16 different 16-byte bank slots: rows
// k..k+3 (and k+8..k+11 for the 16 x 16 atom) over 2 or 4 neighbouring chunks.
__host__ __device__ constexpr int mn_key(int k) { return 4 * (k & 3) + 2 * ((k >> 3) & 1); }
template <int CHR> __host__ __device__ constexpr int mn_slot(int k, int c) {
  static_assert(CHR >= 16 && CHR % 16 == 0, "rows of at least 256 bytes");
  return k * CHR + (c ^ mn_key(k));
}

}  // namespace htk
