// pingpong.h -- the ping-pong GEMM kernel for gfx950 (MI355X) and its tile-table entry macros.
// Included after kernels.h, whose loaders, swizzles, atoms and epilogue it uses.
#pragma once

#include "kernels.h"

namespace htk {

// ------------------------------------------------------------------------------------------
// The ping-pong kernel: a 256 x 256 workgroup tile whose eight waves form two groups of four,
// one wave of each group on every SIMD.  The groups take turns: while one group issues only the
// MFMAs of a k-tile from fragments already in its registers, the other reads the fragments of
// its next k-tile from LDS and issues its share of the DMA, and every barrier swaps the roles.
// Each SIMD so always holds one wave whose next instruction is an MFMA with no LDS or memory
// wait in front of it, and the LDS round trips and DMA issue of the other wave hide behind that
// MFMA stream ("CuTe DSL / CUDA Tile" post, "Pipelining hides a wait": the slower of load and
// compute sets the interval; "CUTLASS", Part IV Stage 4: the mainloop overlaps the loads of
// later k-tiles with the math of the current one).  Group 1 starts one phase late (one extra
// barrier before its loop); group 0 ends one phase early (one extra barrier after it), so both
// pass the same number of barriers.
//
// Group g computes output rows [128 g, 128 g + 128) of the tile; wave q of the group the 64
// columns [64 q, 64 q + 64), as 8 x 4 atoms of 16 x 16.  In global phase 2v group 0 reads k-tile
// v, in phase 2v + 1 group 1 reads it, so the two halves of the A tile are read by different
// groups at different phases and are kept as separate half units (16 KiB: 128 rows of 128
// bytes), two slots each; B, read by both, in three slots of 32 KiB: 64 + 96 = 160 KiB of LDS.
//   * A half 1 of k-tile v + 1 is issued by group 0 in phase 2v (its slot's previous tile,
//     v - 1, was last read in phase 2v - 1) and is read in phase 2v + 3;
//   * A half 0 of k-tile v + 2 by group 1 in phase 2v + 1 (previous tile v, read in phase 2v),
//     read in phase 2v + 4;
//   * B of k-tile v + 2, one half by each group, group g in phase 2v + g (previous tile v - 1,
//     read in phases 2v - 2 and 2v - 1), read from phase 2v + 4 on.
// A wave issues 8 DMA instructions per read phase and, before the barrier that ends its next
// read phase, waits until at most those 8 are in flight: every unit is complete before the
// barrier in front of its first reader.
//
// B K-major: B's halves are its column halves.  B N-major (row-major, 2-byte types): a B unit is
// 64 rows of k of 512 bytes (slot mn_slot) read by transposing LDS reads, as in the split ring;
// wave w issues its DMA blocks w, w + 8, w + 16, w + 24 (2 rows of k each), so a group's half is
// every other run of 8 rows of k.
// Summation order per output is the split ring's (k-tiles in order, atoms' k runs in order), so
// both produce the same bits.
// ------------------------------------------------------------------------------------------
template <int DT, bool BKM>
__global__ __launch_bounds__(512, 1) void gemm_pp(const KParams p_) {
  KParams p;
  int pid, nwg;
  if (!problem_view<256>(p_, p, pid, nwg)) return;
  // opt-in clock record of this workgroup (a uniform branch on a kernel argument)
  const int64_t rec_id = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const bool rec = p_.clock_rec != nullptr && rec_id < p_.clock_cap;
  unsigned long long clk0 = 0, rt0 = 0;
  if (rec) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  constexpr int MI = 16;
  typedef Atom<DT, MI> At;
  typedef typename At::acc_t acc_t;
  constexpr int BM = 256, BN = 256, CH = 8;   // 128-byte LDS rows
  constexpr int NT = 512;
  constexpr int SZ = Ty<DT>::SZ;
  constexpr int BKE = CH * 16 / SZ;           // elements per k-tile
  constexpr int VE = 16 / SZ;
  constexpr int WTM = 128, WTN = 64;
  constexpr int RM = WTM / MI, RN = WTN / MI;
  constexpr int U = At::UNITS;                // 16-byte chunks per operand per MFMA
  constexpr int S = CH / At::G / U;           // fragment substeps per k-tile
  constexpr int HALF = 128 * CH;              // 16-byte chunks per half unit (16 KiB)
  constexpr int B0 = 4 * HALF;                // B ring after the four A half slots
  constexpr int CHR = BN * SZ / 16;           // chunks per row of k (B N-major)
  static_assert(At::PER_UNIT == 1 && S >= 1, "whole MFMAs per k-tile");
  static_assert(BKM || (SZ == 2 && BKE * CHR == 2 * HALF), "rows of k: 2-byte B, one unit per k-tile");

  __shared__ u32x4 lds[10 * HALF];

  int tm, tn;
  tile_of(p, pid, nwg, tm, tn);
  const KRange kr = k_range(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, wq = wave & 3;     // group, wave within the group
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  acc_t acc[RM][RN];
  static_for<RM>([&](auto i) { static_for<RN>([&](auto j) { acc[i][j] = acc_t{}; }); });

  const int64_t K = uniform_i64(kr.len);
  const char* a_tile = uniform_ptr((const char*)p.A + (m0 * p.lda + kr.begin) * SZ);
  const char* b_tile = uniform_ptr((const char*)p.B + (BKM ? n0 * p.ldb + kr.begin : kr.begin * p.ldb + n0) * SZ);
  const int64_t a_span = uniform_i64(((p.M - m0 - 1) * p.lda + K) * SZ);
  const int64_t b_span = uniform_i64(BKM ? ((min((int64_t)BN, p.N - n0) - 1) * p.ldb + K) * SZ
                                         : ((K - 1) * p.ldb + (p.N - n0)) * SZ);
  // A K-major half unit is 16 DMA blocks of 1 KiB (8 rows each); wave q of a group issues blocks
  // q, q + 4, q + 8, q + 12.  Lane l of block blk fills row blk * 8 + l / 8, slot l % 8, which
  // holds logical chunk (l % 8) ^ key(row); blocks of one wave differ by 32 rows, which the key
  // (row bits 1..3) does not see, so the chunk of a lane is the same in all four.
  const int hrow = wq * 8 + lane / 8;
  const int kc = ((lane % CH) ^ row_key<CH>(hrow)) * VE;
  // this wave's A half (1 - g) and, K-major B, its B half (g)
  const uint32_t a_off0 = (uint32_t)(((1 - g) * 128 + hrow) * p.lda * SZ + kc * SZ);
  const uint32_t a_step = (uint32_t)(32 * p.lda * SZ);
  // B N-major: lane l of block blk (2 rows of k) fills row blk * 2 + l / CHR, slot l % CHR,
  // holding logical chunk (l % CHR) ^ mn_key(row); this wave's blocks are 16 rows apart, which
  // mn_key (row bits 0..3) does not see.
  const int brow0 = wave * 2 + lane / CHR;
  const uint32_t b_off0 = BKM ? (uint32_t)((g * 128 + hrow) * p.ldb * SZ + kc * SZ)
                              : (uint32_t)((brow0 * p.ldb + ((lane % CHR) ^ mn_key(brow0)) * VE) * SZ);
  const uint32_t b_step = BKM ? (uint32_t)(32 * p.ldb * SZ) : (uint32_t)(16 * p.ldb * SZ);
  const int nk = (int)((K + BKE - 1) / BKE);

  // Four DMA blocks of a K-major half unit of k-tile t into LDS chunk base `dst`.  Units past
  // the end of K are all out of range (zeros) and are issued anyway, so the wait counts stay the
  // same on every k-tile.
  auto dma_k = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off0, uint32_t step, int t, u32x4* dst) {
    const int64_t k0 = (int64_t)t * BKE;
    const int rem = (int)min(K - k0, (int64_t)BKE);
    // formed here, at the issue, not hoisted out of the loop as more live registers
    asm volatile("" : "+v"(off0));
    const bool in_k = kc < rem;
    static_for<4>([&](auto i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + (wq + 4 * i) * 64), 16,
                                               in_k ? off0 + (uint32_t)i * step : kOobOffset,
                                               (int)(k0 * SZ), 0, 0);
    });
  };
  auto dma_a = [&](int half, uint32_t off0, int t) {  // half of A(t) into its slot t % 2
    dma_k(make_rsrc(a_tile, a_span), off0, a_step, t, lds + (half * 2 + (t & 1)) * HALF);
  };
  auto dma_b = [&](int t) {  // this wave's share of B(t) into slot t % 3
    u32x4* st = lds + B0 + (t % 3) * 2 * HALF;
    if constexpr (BKM) {
      dma_k(make_rsrc(b_tile, b_span), b_off0, b_step, t, st + g * HALF);
    } else {
      // rows of k: the k advance moves the descriptor's base, so the range check (on the VGPR
      // offset) covers every row and column read; rows past K read zero
      const int64_t k0 = (int64_t)t * BKE;
      const int rem = (int)min(K - k0, (int64_t)BKE);
      const int64_t adv = k0 * p.ldb * SZ;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(b_tile + adv, b_span - adv);
      uint32_t off0 = b_off0;
      asm volatile("" : "+v"(off0));
      static_for<4>([&](auto i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(st + (wave + 8 * i) * 64), 16,
                                                 brow0 + 16 * i < rem ? off0 + (uint32_t)i * b_step : kOobOffset,
                                                 0, 0, 0);
      });
    }
  };

  const int frow = frag_row<DT, MI>(lane), fgrp = frag_chunk<DT, MI>(lane);
  u32x4 fa[S][RM][U], fb[S][RN][U];
  // Fragment addresses.  K-major tiles: the chunk index of (row i * MI + frow, chunk c) is that of
  // (frow, c) plus i * MI * CH, since the XOR key sees row bits 1..3 only, so one per-lane index
  // per k run serves all rows of A and B and the rest is an instruction offset.  Rows of k: the
  // key of the rows a lane reads (row bits 0..1 and 3) does not change with the k runs of the
  // k-tile (multiples of 32 rows) or the second transposing read (4 rows on, within the lane's
  // run of 8), so one byte offset per 16-column block serves every k run and both reads.
  static_assert(MI % 16 == 0, "row blocks keep the XOR key");
  int ka[S * U];
  static_for<S * U>([&](auto su) { ka[su] = dslot<CH>(frow, fgrp + At::G * su); });
  int kb_rows[RN];
  if constexpr (!BKM) {
    const int sl = lane & 15, col = (frow & ~15) + 4 * (sl & 3);
    const int k = fgrp * VE + (sl >> 2);
    static_for<RN>([&](auto j) {
      const int cj = wq * WTN + j * MI + col;
      kb_rows[j] = mn_slot<CHR>(k, cj >> 3) * 16 + (cj & 4) * 2;
    });
  }
  // fragments of k-tile t: this group's A half and this wave's 64 columns of B
  auto read_frags = [&](int t) {
    const int sa = (g * 2 + (t & 1)) * HALF, sb = B0 + (t % 3) * 2 * HALF;
    static_for<S>([&](auto s) {
      static_for<U>([&](auto x) {
        constexpr int su = s * U + x;
        // recomputed per phase from one register, so that no per-row address stays live
        int ia = sa + ka[su];
        asm volatile("" : "+v"(ia));
        static_for<RM>([&](auto i) { fa[s][i][x] = lds[ia + i * MI * CH]; });
        if constexpr (BKM) {
          int ib = sb + ka[su] + wq * WTN * CH;
          asm volatile("" : "+v"(ib));
          static_for<RN>([&](auto j) { fb[s][j][x] = lds[ib + j * MI * CH]; });
        } else {
          // k run su starts At::G * su chunks = At::G * su * VE rows of k further down
          static_for<RN>([&](auto j) {
            int byte = sb * 16 + kb_rows[j];
            asm volatile("" : "+v"(byte));
            const lds_char_t* base = (const lds_char_t*)lds + byte + su * At::G * VE * CHR * 16;
            u32x4 out;
            static_for<2>([&](auto h) {
              const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_v4i16_t*)(base + h * 4 * CHR * 16));
              const u32x4 w = __builtin_bit_cast(u32x4, __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3));
              out[2 * h] = w[0];
              out[2 * h + 1] = w[1];
            });
            fb[s][j][x] = out;
          });
        }
      });
    });
  };
  auto mma_all = [&]() {
    static_for<S>([&](auto s) {
      static_for<RM>([&](auto i) {
        static_for<RN>([&](auto j) { At::mma(acc[i][j], fa[s][i], fb[s][j], 0); });
      });
    });
  };
  // Barrier between phases; the scheduling fences keep each phase's MFMAs and LDS reads on
  // their side of it.
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    barrier_nofence();
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nk > 0) {
    // Prologue: A(0) both halves and A half 0 of k-tile 1, B(0) and B(1) (A half 1 of k-tile 1
    // and B(2) come with group 0's first read phase).
    if (g == 0) {
      dma_a(0, (uint32_t)(hrow * p.lda * SZ + kc * SZ), 0);
      dma_a(1, a_off0, 0);
    } else {
      dma_a(0, a_off0, 1);
    }
    dma_b(0);
    dma_b(1);
    wait_counts<0, true>();
    barrier_nofence();
    if (g == 1) phase_end();  // group 1 starts one phase late
    for (int v = 0; v < nk; ++v) {
      // read phase: fragments of k-tile v; DMA of A half 1 - g of k-tile v + 1 + g, and of B(v + 2)
      read_frags(v);
      dma_a(1 - g, a_off0, v + 1 + g);
      dma_b(v + 2);
      wait_counts<8, true>();
      phase_end();
      // compute phase
      mma_all();
      phase_end();
    }
    if (g == 0) phase_end();  // group 0 ends one phase early
    wait_counts<0, true>();   // the zero-filled units issued past the end are still in flight
    barrier_nofence();
  }
  KParams pe;
  int pid_e, nwg_e;
  problem_view<256>(reload_args(), pe, pid_e, nwg_e);
  if (pe.split_k > 1) {
    store_partial<DT, MI, BM, BN, WTM, WTN>(pe, acc, m0, n0, g, wq, lane);
  } else if (epilogue_form<DT>(pe) == 1) {
    epilogue<DT, MI, BM, BN, WTM, WTN, RM, RN, NT, sizeof(lds), 1>(pe, acc, lds, m0, n0, g, wq,
                                                                   lane, tid, nk == 0);
  } else {
    epilogue<DT, MI, BM, BN, WTM, WTN, RM, RN, NT, sizeof(lds)>(pe, acc, lds, m0, n0, g, wq, lane,
                                                                tid, nk == 0);
  }
  if (rec) {
    const unsigned long long clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
      unsigned long long* r = p_.clock_rec + 4 * rec_id;
      r[0] = clk0;
      r[1] = clk1;
      r[2] = rt0;
      r[3] = rt1;
    }
  }
}

template <int DT, bool BKM>
static hipError_t launch_pp(const KParams& p, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((gemm_pp<DT, BKM>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

// Ping-pong entries: 256 x 256 tiles, K-major A, 128-byte rows, 10 half units of 16 KiB.  The
// _BN form takes a row-major (N-contiguous) 2-byte B kept in LDS as rows of k.
#define HT_PP(NAME, DT)                                                                            \
  {NAME, DT, 1, 1, 1, 0, 256, 256, 128 / Ty<DT>::SZ, 8, 5, 5 * 256 * 128, 64,                     \
   &launch_pp<DT, true>, 0, 16, 8, 0, nullptr}
#define HT_PP_BN(NAME, DT)                                                                         \
  {NAME, DT, 1, 0, 1, 0, 256, 256, 128 / Ty<DT>::SZ, 8, 5, 5 * 256 * 128, 64,                     \
   &launch_pp<DT, false>, 0, 16, 8, 1, nullptr}

}  // namespace htk
