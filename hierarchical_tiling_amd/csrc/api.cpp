// api.cpp -- host side of the C ABI in htgemm.h: validation ("can_implement"), the tile-table
// choice, and the launch on the caller's stream.
//
// The life cycle mirrors the pages' device layer ("CUTLASS", stanleyjacob.dev, Part IV Stage 1:
// get_workspace_size, can_implement, initialize, run; "CUTLASS, CuTe, and CUDA Tile", section
// "Assembling a CUTLASS kernel": a stateful reusable handle; the kernel, not the caller, fixes
// the grid).  The tile table plays the part of the pages' builder that picks a configuration
// from the problem ("CUTLASS", Part IX: the best tile depends on the problem shape, which is why
// the measurement tool ships with the library).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "../../include/htgemm.h"
#include "../../include/htlayout.h"
#include "atom_maps.h"
#include "gemm_internal.h"

using namespace htk;

namespace {

constexpr uint32_t kMagic = 0x47454d4du;   // live handle
constexpr uint32_t kDead = 0xdeadbeefu;    // destroyed handle
constexpr int64_t kLdsBudget = 160 * 1024;  // LDS per CU on gfx950
constexpr int kCUs = 256;                   // compute units of an MI355X: one round of a
                                            // one-workgroup-per-CU kernel, and the Stream-K
                                            // launch's persistent workgroups
static_assert(kCUs % 8 == 0, "Stream-K shares are dealt over the 8 XCDs");

struct Operand {
  bool kmajor;  // unit stride along K
  int64_t ld;   // the other stride
};

}  // namespace

struct gemm_handle_s {
  uint32_t magic;
  gemm_desc d;
  Operand a, b;
  int cfg;       // entry used when A and B are 16-byte aligned
  int fallback;  // narrow-load entry
  int group_m;
  int split_cfg, split_fb;     // K slices of each entry (1: no split)
  int64_t kps_cfg, kps_fb;     // K elements per slice
  int tail_tiles, tail_split;  // split tail of the cfg entry (tail_split 1: none)
  int64_t tail_kps;            // K elements per slice of a tail tile
  int sk_tiles;                // Stream-K tiles of the cfg entry (0: none)
  double predicted_us;         // the cost model's time of one run (0: no measured costs)
  // Repack plan: A and B are read through K-major, 16-byte aligned copies of K padded to kp
  // (zeros past K) at the start of the workspace (A' then B', each rounded to 256 bytes), and
  // cfg is the entry chosen for that aligned problem.  An operand that is already K-major with
  // a 16-byte leading dimension, K == kp and a 16-byte aligned pointer is used in place.
  int repack;
  int64_t kp;
  size_t repack_bytes_a, repack_bytes_b;
  // clock record of the product kernel's launches (gemm_set_clock_record), or nullptr
  unsigned long long* clock_rec;
  int64_t clock_cap;
};

namespace {

bool valid_type(int t) { return t >= GEMM_F32 && t <= GEMM_F8E4M3; }

// Unit-stride analysis of one input operand: rows x K with strides (s_row, s_k).
int classify(int64_t s_row, int64_t s_k, Operand* op) {
  if (s_row < 0 || s_k < 0) return GEMM_ERR_LAYOUT;
  if (s_k == 1) { op->kmajor = true; op->ld = s_row; return GEMM_OK; }
  if (s_row == 1) { op->kmajor = false; op->ld = s_k; return GEMM_OK; }
  return GEMM_ERR_LAYOUT;
}

// Can the 16-byte-load path read this operand (given 16-byte aligned base pointers)?
bool vec_ok(const Operand& op, int64_t rows, int64_t K, int dt) {
  const int sz = dtype_size(dt), ve = 16 / sz;
  if ((op.ld * sz) % 16 != 0) return false;
  // Rows must not overlap: the buffer loaders' range check (on the row offset) then also bounds
  // the k offset they add outside the check.
  if (op.ld < (op.kmajor ? K : rows)) return false;
  if (op.kmajor) return K % ve == 0;
  if (dt == DT_F8) return false;  // no transposing vector loader for 1-byte elements
  return rows % ve == 0;
}

bool entry_fits(const KernelEntry& e, const gemm_handle_s& h, bool vec_a, bool vec_b) {
  const gemm_desc& d = h.d;
  if (e.dtype != d.a_type) return false;
  if ((e.a_kmajor != 0) != h.a.kmajor || (e.b_kmajor != 0) != h.b.kmajor) return false;
  if (e.vec && !(vec_a && vec_b)) return false;
  if (e.skinny && d.M > e.bm) return false;  // the streaming kernel holds all M rows in one tile
  if (e.skinny && (d.ragged_m || d.grouped)) return false;  // grouped launches use tile kernels
  // the row reduction reads the output tile repacked in LDS: tile kernels whose LDS holds it
  if ((d.has_row_sumsq || d.has_col_sum) &&
      (e.skinny || int64_t(e.bm) * e.bn * dtype_size(d.d_type) > e.lds_bytes))
    return false;
  if (e.vec) {
    // the 16-byte K-major loaders address one tile with 31-bit buffer offsets, and so do the
    // MN-major loaders that keep 2-byte tiles as rows of k, over all of K
    const int64_t sz = dtype_size(e.dtype), lim = int64_t(1) << 31;
    if (h.a.kmajor && (int64_t(e.bm) * h.a.ld + d.K) * sz >= lim) return false;
    if (h.b.kmajor && (int64_t(e.bn) * h.b.ld + d.K) * sz >= lim) return false;
    if (e.mn_rows && !h.a.kmajor && (d.K * h.a.ld + e.bm) * sz >= lim - 64) return false;
    if (e.mn_rows && !h.b.kmajor && (d.K * h.b.ld + e.bn) * sz >= lim - 64) return false;
  }
  if (e.realign) {
    // realigned loaders: 31-bit offsets over a tile's rows (K-major) or over all of K (M/N-major)
    const int64_t sz = dtype_size(e.dtype), lim = (int64_t(1) << 31) - 64;
    const int64_t a_span = h.a.kmajor ? int64_t(e.bm) * h.a.ld + d.K : d.K * h.a.ld + e.bm;
    const int64_t b_span = h.b.kmajor ? int64_t(e.bn) * h.b.ld + d.K : d.K * h.b.ld + e.bn;
    if (a_span * sz >= lim || b_span * sz >= lim) return false;
  }
  ht_tile_stats st;
  ht_tile_plan(e.bm, e.bn, e.bk, dtype_size(e.dtype), kLdsBudget, &st);
  if (!st.fits) return false;  // double-buffered A and B tiles must fit the LDS budget
  if (e.lds_bytes > kLdsBudget) return false;
  return true;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row groups per tile of the column-sum partials (the epilogue's wave split of a tile's rows).
int col_sum_row_groups(const KernelEntry& e) {
  const int cg = e.bn / 64;
  return e.waves >= cg ? e.waves / cg : 1;
}

// ---- cost model ----------------------------------------------------------------------------
// The kernel choice and the split plan predict run times from each entry's measured costs
// (EntryCost; "CUTLASS", stanleyjacob.dev, Part IX: the best tile depends on the problem, so the
// library is measured rather than guessed).  launch_us is a launch of wg workgroups of kt k-tiles
// each.  Whole loads n (n workgroups on every CU) take the measured time; a load above 8 adds
// whole groups of 8; a partly filled last round costs the step to the next whole load, scaled as
// a round with that fraction of the CUs busy (piecewise linear over the loads 1/4, 1/2, 3/4, 1).
double launch_us(const EntryCost& c, int64_t wg, int64_t kt) {
  if (wg <= 0 || kt <= 0) return 0.0;
  static constexpr double kPart[kCostLoadOne + 1] = {0.25, 0.5, 0.75, 1.0};
  auto at = [&](int i) { return double(c.f[i]) + double(kt) * double(c.c[i]); };
  auto whole = [&](int64_t n) {
    if (n <= 0) return 0.0;
    const int64_t g = (n - 1) / 8;
    return double(g) * at(kCostLoads - 1) + at(int(n - 8 * g) + kCostLoadOne - 1);
  };
  auto part = [&](double w) {
    double t = at(0);
    if (w > kPart[0]) {
      int i = 1;
      while (kPart[i] < w) ++i;
      t = at(i - 1) + (w - kPart[i - 1]) / (kPart[i] - kPart[i - 1]) * (at(i) - at(i - 1));
    }
    return t / at(kCostLoadOne);
  };
  const int64_t n = cdiv(wg, kCUs);
  const double w = double(wg - (n - 1) * kCUs) / kCUs;
  const double lo = whole(n - 1), hi = whole(n);
  return lo + (hi - lo) * part(w);
}

// The sum kernel of a split: partial_bytes of fp32 partials (written by the first kernel and read
// by the second) and out_bytes of output.
double reduce_us(double partial_bytes, double out_bytes) {
  return kSplitFixedUs + kSplitUsPerByte * (2.0 * partial_bytes + out_bytes);
}

// Output tiles of entry e over d: all problems of a batch, or a grouped launch's tiles (each group
// may start a tile row of its own).
int64_t tiles_of(const KernelEntry& e, const gemm_desc& d) {
  const int64_t groups = d.batch > 1 ? d.batch : 1;
  if (d.ragged_m) return (cdiv(d.M, e.bm) + groups) * cdiv(d.N, e.bn);
  return cdiv(d.M, e.bm) * cdiv(d.N, e.bn) * (d.grouped ? 1 : groups);
}

// An entry whose LDS leaves no room for a second workgroup runs one per CU: 256 make a round.
bool one_per_cu(const KernelEntry& e) { return 2 * int64_t(e.lds_bytes) > kLdsBudget; }

// Split along K for entry e: S slices of whole k-tiles ("CUTLASS", Part III: split-K restores
// occupancy when the output has too few tiles).  req > 1 forces S (at most one slice per
// k-tile); req == 1 never splits; req == 0 (automatic) considers splitting an output of fewer
// than 256 tiles into at most 16 slices and takes the count with the least predicted time: the
// launch of tiles x S workgroups plus the sum kernel.  With the measured costs the choice keeps
// what was found by hand on MI355X: bf16 1536^2 x 8192 runs on the ring in 7 slices (252
// workgroups; 8 would start a second round), and bf16 2048^2 x 4096 unsplit on 128 x 128 tiles
// (0.048 ms, against 0.055 ms in 4 ring slices).  An entry without measured costs is not split
// unless forced.
void plan_split(const KernelEntry& e, const gemm_desc& d, int req, int* S, int64_t* kps) {
  *S = 1;
  *kps = d.K;
  if (req == 1 || e.max_split_k <= 1 || d.K == 0) return;
  const int64_t tiles = cdiv(d.M, e.bm) * cdiv(d.N, e.bn);
  const int64_t nkt = cdiv(d.K, e.bk);
  if (req > 1) {
    const int64_t s = std::min<int64_t>({(int64_t)req, nkt, (int64_t)e.max_split_k});
    if (s <= 1) return;
    const int64_t per = cdiv(nkt, s);  // k-tiles per slice
    *kps = per * e.bk;
    *S = (int)cdiv(nkt, per);           // no empty slice
    return;
  }
  if (e.skinny) {
    // The streaming kernel (no measured costs; chosen by its shape) pulls B from HBM.  A grid of
    // few column blocks with long K leaves most CUs idle, so K is cut into S slices (fp32 planes
    // of 16 x N, summed by the split-K kernel): the largest power of two S <= 8 that keeps at
    // least 32 blocks of K per slice and at most 512 workgroups, and only below 64 column blocks
    // or from 256 blocks of K.  Measured on MI355X (bf16, microseconds, unsplit -> chosen):
    // 16x16x32768 31.8 -> 11.7 (S 8), 16x256x32768 33.1 -> 12.4 (8), 16x1024x8192 11.0 -> 10.1
    // (4), 16x2048x32768 60.5 -> 33.2 (8), 16x4096x16384 38.1 -> 36.0 (4); left unsplit:
    // 16x4096x4096 8.3 (S 2: 11.2), 16x8192x8192 33.8 (S 2: 32.2, S 4: 38.1), e4m3 8x4096x4096
    // 7.1 (S 2: 10.1).
    if (tiles >= 64 && nkt < 256) return;
    int64_t s = 1;
    while (2 * s <= std::min<int64_t>(8, e.max_split_k) && nkt / (2 * s) >= 32 && tiles * 2 * s <= 512)
      s *= 2;
    if (s < 2) return;
    const int64_t per = cdiv(nkt, s);
    *kps = per * e.bk;
    *S = (int)cdiv(nkt, per);
    return;
  }
  if (tiles >= kCUs || !e.cost) return;
  const double out_bytes = double(d.M) * double(d.N) * dtype_size(d.d_type);
  double best = launch_us(*e.cost, tiles, nkt);
  const int64_t smax = std::min<int64_t>({nkt, (int64_t)e.max_split_k, 16});
  for (int64_t s = 2; s <= smax; ++s) {
    const int64_t per = cdiv(nkt, s);
    if (cdiv(nkt, per) != s) continue;  // the same slices as a smaller count
    const double t = launch_us(*e.cost, tiles * s, per) +
                     reduce_us(4.0 * double(s) * double(d.M) * double(d.N), out_bytes);
    if (t < best) {
      best = t;
      *S = (int)s;
      *kps = per * e.bk;
    }
  }
}

// Split tail (the data-parallel plus split-K hybrid of Stream-K scheduling; "CUTLASS", Part III:
// Stream-K evens out work when the tiles do not divide over the processors).  An entry whose LDS
// allows one workgroup per CU runs 256 tiles per round.  When more than one round is needed and
// the last is at most half full, the R = tiles mod 256 tiles of that round are split along K into
// S slices each, about R * S <= 256 workgroups, written as compact fp32 partials and summed in
// fixed order by a second kernel; the other tiles run whole.  Only when the library decides the
// split (split_k = 0, one plain product), no whole-problem split is planned and Stream-K is
// not (it takes this case for the kernels that have a Stream-K form; with decomposition 1 the
// split tail stays).
void plan_tail(const KernelEntry& e, const gemm_desc& d, int split_req, int split_whole, int* R,
               int* S, int64_t* kps) {
  *R = 0;
  *S = 1;
  *kps = d.K;
  if (split_req != 0 || split_whole > 1 || e.max_split_k <= 1 || e.skinny) return;
  if (!one_per_cu(e)) return;
  const int64_t tiles = cdiv(d.M, e.bm) * cdiv(d.N, e.bn);
  const int64_t rem = tiles % 256;
  if (tiles <= 256 || rem == 0 || rem > 128) return;
  // Each slice carries fixed costs (pipeline fill, an fp32 partial tile, its share of the sum
  // kernel).  Measured on MI355X, the split pays from 64 k-tiles per tile with at least 8 per
  // slice (bf16 4352^2 x 4096: -10 %; at 16 or 32 k-tiles it was 3-11 % slower).
  const int64_t nkt = cdiv(d.K, e.bk);
  if (nkt < 64) return;
  const int64_t s = std::min<int64_t>({256 / rem, nkt / 8, (int64_t)e.max_split_k, 16});
  if (s < 2) return;
  const int64_t per = cdiv(nkt, s);  // k-tiles per slice, at least 8
  const int64_t slices = cdiv(nkt, per);
  if (slices < 2) return;
  *R = (int)rem;
  *S = (int)slices;
  *kps = per * e.bk;
}

// Stream-K (the work-centric tile scheduler; "CUTLASS", Part IV Stage 2 and its Stream-K
// reference, Osama et al. 2023): kCUs persistent workgroups share the k-tile iterations of the
// last tiles equally, so no CU idles in a last round that the tiles fill only partly.  As in
// that paper's data-parallel hybrid, only the tiles of the last partial round run Stream-K (each
// workgroup then takes less than one tile of work); the others run whole, a tile per workgroup.
// With at most kCUs tiles all of them run Stream-K (with whole rounds only, forced, the last
// round: whole tiles on persistent workgroups).  decomposition 2 forces the plan.  0 applies it
// where it was measured to pay on MI355X: a last round at most half full after whole rounds,
// with at least 64 k-tiles per tile, where it replaces the split tail (bf16 ring: 6144^2 x 8192
// 495 us against 562 us split tail and 541-554 us data-parallel; 7168^2 x 8192 675 / 746 /
// 732-742; 4352^2 x 8192 297 / 311 / 348-356; 4864 x 4096 x 4096 180 / 185 / 188-197).  With
// a fuller last round, or with every tile in one round, the shares are larger than half a tile
// and Stream-K lost (5376^2 x 4096: 280 us against 199-212 data-parallel; 3840^2 x 8192, 225
// tiles: 336 against 190-209): a workgroup's share starts at a k offset of its own, so the
// workgroups that share A and B panels no longer read them together and most reads miss L2.
void plan_sk(const KernelEntry& e, const gemm_desc& d, int split_req, int split_whole,
             int* sk_tiles) {
  *sk_tiles = 0;
  if (!e.launch_sk || d.decomposition == 1 || split_whole > 1) return;
  if (d.batch > 1 || d.ragged_m || d.grouped || d.has_row_sumsq || d.has_col_sum) return;
  const int64_t tiles = cdiv(d.M, e.bm) * cdiv(d.N, e.bn);
  const int64_t nkt = cdiv(d.K, e.bk);
  if (tiles == 0 || nkt == 0) return;
  const int64_t rem = tiles % kCUs;
  if (d.decomposition == 0) {
    if (split_req != 0 || tiles <= kCUs || rem == 0 || rem > kCUs / 2 || nkt < 64) return;
  }
  *sk_tiles = (int)(tiles <= kCUs ? tiles : (rem == 0 ? kCUs : rem));
}

// An entry's plan for a problem: its split, Stream-K tiles or split tail, and the predicted time
// of a run (infinite for an entry without measured costs).
struct Plan {
  int S = 1;                    // K slices of the whole problem
  int64_t kps = 0;              // K elements per slice
  int sk_tiles = 0;             // tiles run Stream-K
  int tail_R = 0, tail_S = 1;   // split tail: tiles, and slices of each
  int64_t tail_kps = 0;
  double us = 0.0;
};

Plan make_plan(const KernelEntry& e, const gemm_desc& d, int split_req) {
  Plan p;
  plan_split(e, d, split_req, &p.S, &p.kps);
  plan_sk(e, d, split_req, p.S, &p.sk_tiles);
  plan_tail(e, d, p.sk_tiles > 0 ? 1 : split_req, p.S, &p.tail_R, &p.tail_S, &p.tail_kps);
  if (!e.cost) {
    p.us = std::numeric_limits<double>::infinity();
    return p;
  }
  const EntryCost& c = *e.cost;
  const int64_t tiles = tiles_of(e, d);
  const int64_t nkt = cdiv(d.K, e.bk);
  const double tile_out = double(e.bm) * e.bn, osz = dtype_size(d.d_type);
  // edges: a partial last k-tile in every tile, partial last tile rows or columns, and D rows
  // that the epilogue cannot store as whole aligned 16-byte chunks (with a base 16-byte aligned)
  double edges = 0.0;
  if (d.K % e.bk != 0) edges += double(c.edge_k) * double(cdiv(tiles, kCUs));
  if (d.M % e.bm != 0 || d.N % e.bn != 0) edges += c.edge_mn;
  if (d.d_stride_n != 1 || (d.d_stride_m * int64_t(osz)) % 16 != 0)
    edges += double(c.edge_d) * double(cdiv(tiles, kCUs));
  if (p.sk_tiles > 0) {
    // whole tiles, then 256 workgroups sharing the k-tiles of the others, then the fix-up
    p.us = launch_us(c, tiles - p.sk_tiles, nkt) + kSkFixedUs +
           kSkShareFactor * launch_us(c, kCUs, cdiv(int64_t(p.sk_tiles) * nkt, kCUs));
  } else if (p.tail_S > 1) {
    const double parts = double(p.tail_R) * p.tail_S;
    p.us = launch_us(c, tiles - p.tail_R, nkt) +
           launch_us(c, int64_t(p.tail_R) * p.tail_S, cdiv(p.tail_kps, e.bk)) +
           reduce_us(4.0 * parts * tile_out, osz * p.tail_R * tile_out);
  } else {
    p.us = launch_us(c, tiles * p.S, cdiv(p.kps, e.bk));
    if (p.S > 1)
      p.us += reduce_us(4.0 * p.S * double(d.M) * double(d.N), osz * double(d.M) * double(d.N));
  }
  p.us += edges;
  return p;
}

// Sustained cost of an entry: its time per k-tile with four workgroups on every CU, per
// multiply-add of a k-tile (the steadiest of its measurements: long launches at full load).
double sustained_cost(const KernelEntry& e) {
  return double(e.cost->c[kCostLoadOne + 3]) / (double(e.bm) * e.bn * e.bk);
}

// Predictions closer than this fraction count as a tie: on 66 measured shapes, times of the same
// kernel and plan differed by up to ~5 % between runs, and the model's predictions for the leading
// entries were within a few percent of their measured times.
constexpr double kTie = 0.03;

// Kernel choice.  A product with M <= 16 is bound by streaming B and takes the skinny kernel when
// one fits.  Otherwise the choice is the fitting entry of the family (16-byte loaders or not) with
// the least predicted time under the plan it would get (make_plan); among entries predicted within
// kTie of that least time, the one with the least sustained cost (then the earlier entry) wins.
// An entry without measured costs is chosen only when nothing else fits.  A forced split
// (split_req > 1) admits only entries that can split.  *us receives the chosen plan's predicted
// time.
int choose(const gemm_handle_s& h, bool vec_a, bool vec_b, bool want_vec, int split_req,
           double* us = nullptr) {
  const KernelEntry* t = table();
  const bool need_split = split_req > 1;
  if (us) *us = 0.0;
  for (int i = 0; i < table_size() && !h.d.ragged_m && !h.d.grouped && !h.d.has_row_sumsq &&
                  !h.d.has_col_sum; ++i)
    if (t[i].skinny && (t[i].vec != 0) == want_vec && (!need_split || t[i].max_split_k > 1) &&
        entry_fits(t[i], h, vec_a, vec_b))
      return i;
  std::vector<std::pair<int, double>> cand;  // fitting entries and their predicted times
  double least = std::numeric_limits<double>::infinity();
  for (int i = 0; i < table_size(); ++i) {
    const KernelEntry& e = t[i];
    if ((e.vec != 0) != want_vec || e.skinny) continue;
    if (need_split && e.max_split_k <= 1) continue;
    if (!entry_fits(e, h, vec_a, vec_b)) continue;
    const double u = make_plan(e, h.d, split_req).us;
    cand.emplace_back(i, u);
    least = std::min(least, u);
  }
  if (cand.empty()) return -1;
  // Stream-K asked for: the entries that have a Stream-K form, where one fits
  if (h.d.decomposition == 2) {
    std::vector<std::pair<int, double>> sk;
    for (const auto& c : cand)
      if (t[c.first].launch_sk) sk.push_back(c);
    if (!sk.empty()) {
      cand.swap(sk);
      least = std::numeric_limits<double>::infinity();
      for (const auto& c : cand) least = std::min(least, c.second);
    }
  }
  int best = -1;
  double best_us = 0.0;
  if (std::isfinite(least)) {
    for (const auto& c : cand) {
      if (c.second > least * (1.0 + kTie)) continue;
      if (best < 0 || sustained_cost(t[c.first]) < sustained_cost(t[best])) {
        best = c.first;
        best_us = c.second;
      }
    }
  } else {
    best = cand.front().first;  // no fitting entry has measured costs
    best_us = cand.front().second;
  }
  if (us) *us = std::isfinite(best_us) ? best_us : 0.0;
  return best;
}

void set_plan(gemm_handle_s* h, const Plan& p) {
  h->split_cfg = p.S;
  h->kps_cfg = p.kps;
  h->sk_tiles = p.sk_tiles;
  h->tail_tiles = p.tail_R;
  h->tail_split = p.tail_S;
  h->tail_kps = p.tail_kps;
  h->predicted_us = std::isfinite(p.us) ? p.us : 0.0;
}

// ---- lane maps checked with the layout helper ---------------------------------------------
// An MFMA atom's A/B and C fragment maps are layouts from (lane, value) to a place in the
// instruction's tile; a wrong map gives silently wrong results ("A10 - CuTe, CUTLASS & CuTile",
// section 3.3 and section 6 Pitfall 2; "CUTLASS", Part V: the layout algebra is what catches a
// wrong thread layout).  Once per atom the kernels' tables (atom_maps.h) are checked against the
// layout helper's evaluation of the same layouts written in the pages' notation: same function,
// a bijection onto the tile (the fragment closure: 64 lanes x values per lane = the tile), and
// lane l on row / column l % MI as the instruction requires.  The LDS swizzles are checked the
// same way against the helper's Swizzle functor.

// the helper's table of `text`, or empty if it does not parse or has the wrong size
std::vector<int64_t> helper_table(const char* text, int64_t n) {
  int64_t size = 0;
  if (ht_layout_size(text, &size) != HT_OK || size != n) return {};
  std::vector<int64_t> t((size_t)n);
  if (ht_layout_table(text, t.data(), n) != HT_OK) return {};
  return t;
}

bool is_bijection(const std::vector<int64_t>& t, int64_t n) {
  std::vector<char> seen((size_t)n, 0);
  for (int64_t v : t) {
    if (v < 0 || v >= n || seen[(size_t)v]) return false;
    seen[(size_t)v] = 1;
  }
  return (int64_t)t.size() == n;
}

bool check_atom_now(int idx) {
  const AtomMaps& M = kAtomMaps[idx];
  const std::vector<int64_t> op = helper_table(M.op.text, 64 * M.vpl);
  const std::vector<int64_t> acc = helper_table(M.acc.text, 64 * M.nacc);
  if (op.empty() || acc.empty()) return false;
  if (64 * M.vpl != M.mi * M.ki || 64 * M.nacc != M.mi * M.mi) return false;  // closure
  if (!is_bijection(op, (int64_t)M.mi * M.ki) || !is_bijection(acc, (int64_t)M.mi * M.mi)) return false;
  for (int i = 0; i < 64 * M.vpl; ++i)
    if (op[(size_t)i] != layout_eval(M.op, i) || (i < 64 && layout_eval(M.op, i) % M.mi != i % M.mi))
      return false;
  for (int i = 0; i < 64 * M.nacc; ++i)
    if (acc[(size_t)i] != layout_eval(M.acc, i) || layout_eval(M.acc, i) / M.mi != (i % 64) % M.mi)
      return false;
  return true;
}

template <int CH> bool check_swizzle_now() {
  for (int row = 0; row < 256; ++row)
    for (int c = 0; c < CH; ++c) {
      const int slot = swizzled_slot<CH>(row, c);
      if (slot != (int)ht_swizzle(row * CH + c, RowSwizzle<CH>::B, RowSwizzle<CH>::M, RowSwizzle<CH>::S))
        return false;
      if (slot / CH != row) return false;  // the swizzle stays within the row
    }
  return true;
}

// The MN-major tiles' slots against two Swizzle functors of the helper.
template <int CHR> bool check_mn_swizzle_now() {
  for (int k = 0; k < 256; ++k)
    for (int c = 0; c < CHR; ++c) {
      const int o = 16 * (k % 16) + (c % 16);
      const int64_t sw = ht_swizzle(ht_swizzle(o, 2, 2, 2), 1, 1, 6);
      const int slot = mn_slot<CHR>(k, c);
      if (slot != k * CHR + (c & ~15) + (int)(sw % 16)) return false;
      if (slot / CHR != k) return false;
    }
  return true;
}

// 0: not checked yet, 1: agrees, 2: disagrees (the result is the same every time)
std::atomic<int> g_atom_state[kNumAtomMaps];
std::atomic<int> g_swizzle_state[2];
std::atomic<int> g_mn_swizzle_state[2];

bool cached(std::atomic<int>& st, bool (*fn)()) {
  int v = st.load(std::memory_order_acquire);
  if (v == 0) {
    v = fn() ? 1 : 2;
    st.store(v, std::memory_order_release);
  }
  return v == 1;
}

template <int IDX> bool check_atom_fn() { return check_atom_now(IDX); }
template <int... I>
bool check_atom_dispatch(int idx, std::integer_sequence<int, I...>) {
  bool ok = false;
  ((idx == I ? (ok = cached(g_atom_state[I], &check_atom_fn<I>), 0) : 0), ...);
  return ok;
}

bool atom_ok(int dtype, int mi) {
  const int idx = atom_index(dtype, mi);
  return idx >= 0 && check_atom_dispatch(idx, std::make_integer_sequence<int, kNumAtomMaps>{});
}

// The lane maps and LDS swizzle of table entry e agree with the layout helper.
bool entry_maps_ok(const KernelEntry& e) {
  if (!atom_ok(e.dtype, e.mi)) return false;
  if (e.mn_rows) {  // an MN-major operand tile with rows of k (16 or 32 chunks)
    if (!cached(g_mn_swizzle_state[0], &check_mn_swizzle_now<16>) ||
        !cached(g_mn_swizzle_state[1], &check_mn_swizzle_now<32>))
      return false;
  }
  if (e.lds_row_chunks == 8) return cached(g_swizzle_state[1], &check_swizzle_now<8>);
  if (e.lds_row_chunks == 4) return cached(g_swizzle_state[0], &check_swizzle_now<4>);
  return e.lds_row_chunks == 0;
}

// Whether a product whose operands the 16-byte loaders cannot read (a leading dimension or base
// off 16 bytes, or an fp8 operand that is not K-contiguous) may run on aligned K-major copies:
// one extra pass over A and B (HBM-bound) against running every k-tile with realigned or
// element-wise register-staged loads, which keep only one k-tile of loads in flight.  The cost
// model decides between the two (the copies plus the kernel chosen for them against the best
// direct entry).  Measured on MI355X before the model decided: e4m3 3001 x 2999 x 2049 with odd
// leading dimensions, 81 us on copies against 533 us with element loads; f16 4099 x 3071 x 2053,
// 110 us against 129 us on realigned loads.  Batches and groups keep the direct path, and so
// do products too small to be worth a pass.
bool repack_allowed(const gemm_desc& d, bool vec_both) {
  if (vec_both || d.ragged_m || d.grouped || d.batch > 1) return false;
  return d.M >= 128 && d.N >= 128 && d.K >= 64;
}

int check_arch() {
  const char* fake = std::getenv("HTGEMM_FAKE_ARCH");
  if (fake && *fake) return std::strncmp(fake, "gfx950", 6) == 0 ? GEMM_OK : GEMM_ERR_ARCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? GEMM_OK : GEMM_ERR_ARCH;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int gemm_create(const gemm_desc* desc, gemm_t* out) {
  if (!desc || !out) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  const gemm_desc& d = *desc;
  if (d.split_k < 0 || d.split_k > 64) return GEMM_ERR_INVALID_ARG;
  if (d.M < 0 || d.N < 0 || d.K < 0) return GEMM_ERR_INVALID_ARG;
  if (d.M > INT32_MAX / 2 || d.N > INT32_MAX / 2 || d.K > INT32_MAX / 2) return GEMM_ERR_INVALID_ARG;
  if (d.act < GEMM_ACT_NONE || d.act > GEMM_ACT_SILU) return GEMM_ERR_INVALID_ARG;
  if ((d.has_c != 0 && d.has_c != 1) || (d.has_bias != 0 && d.has_bias != 1)) return GEMM_ERR_INVALID_ARG;
  if ((d.has_row_scale != 0 && d.has_row_scale != 1) || (d.has_col_scale != 0 && d.has_col_scale != 1))
    return GEMM_ERR_INVALID_ARG;
  // batch (the problem shape's L mode): up to 65535 problems, one per grid z index
  if (d.batch < 0 || d.batch > 65535) return GEMM_ERR_INVALID_ARG;
  const int64_t L = d.batch > 1 ? d.batch : 1;
  if (d.ragged_m != 0 && d.ragged_m != 1) return GEMM_ERR_INVALID_ARG;
  if (d.grouped != 0 && d.grouped != 1) return GEMM_ERR_INVALID_ARG;
  if (d.decomposition < 0 || d.decomposition > 2) return GEMM_ERR_INVALID_ARG;
  if (d.decomposition == 2 && (d.split_k > 1 || d.batch > 1 || d.ragged_m || d.grouped ||
                               d.has_row_sumsq || d.has_col_sum))
    return GEMM_ERR_INVALID_ARG;
  if (d.has_row_sumsq != 0 && d.has_row_sumsq != 1) return GEMM_ERR_INVALID_ARG;
  if (d.has_col_sum != 0 && d.has_col_sum != 1) return GEMM_ERR_INVALID_ARG;
  // the reductions cover one problem and are not split along K
  if ((d.has_row_sumsq || d.has_col_sum) && (L > 1 || d.ragged_m || d.split_k > 1))
    return GEMM_ERR_INVALID_ARG;
  if (d.ragged_m) {
    // grouped: the groups share A's, C's and D's rows (device offsets at run time); B moves by
    // b_stride_l per group.  Row offsets must keep 16-byte rows aligned: A is K-major.  The
    // batch field is the group count G (offsets holds G + 1 values), so it must be at least 1.
    if (d.batch < 1) return GEMM_ERR_INVALID_ARG;
    if (d.b_stride_l < 0) return GEMM_ERR_LAYOUT;
    if (d.split_k > 1 || d.grouped) return GEMM_ERR_INVALID_ARG;
  } else if (d.grouped) {
    // independent problems: shapes, pointers and leading dimensions come with each run; the
    // descriptor fixes types, layouts and epilogue.  One launch, no split, no per-row or
    // per-column vectors (their lengths would differ per problem).
    if (d.batch < 1 || d.split_k > 1) return GEMM_ERR_INVALID_ARG;
    if (d.has_row_scale || d.has_col_scale || d.has_row_sumsq || d.has_col_sum)
      return GEMM_ERR_INVALID_ARG;
    if (d.d_stride_n != 1 && d.d_stride_m != 1) return GEMM_ERR_LAYOUT;
    if (d.has_c && d.c_stride_n != 1 && d.c_stride_m != 1) return GEMM_ERR_LAYOUT;
  } else if (L > 1) {
    if (d.a_stride_l < 0 || d.b_stride_l < 0 || d.c_stride_l < 0 || d.d_stride_l < 0)
      return GEMM_ERR_LAYOUT;
    // distinct problems must not write the same D; split-K is for single problems
    if (d.d_stride_l == 0 && d.M > 0 && d.N > 0) return GEMM_ERR_INVALID_ARG;
    if (d.split_k > 1) return GEMM_ERR_INVALID_ARG;
  }
  if (!valid_type(d.a_type) || !valid_type(d.b_type) || !valid_type(d.d_type)) return GEMM_ERR_DTYPE_COMBO;
  if (d.a_type != d.b_type || d.d_type != out_dtype(d.a_type)) return GEMM_ERR_DTYPE_COMBO;
  if (d.has_c && d.c_type != d.d_type) return GEMM_ERR_DTYPE_COMBO;
  if (d.has_bias && d.bias_type != d.d_type) return GEMM_ERR_DTYPE_COMBO;
  if (d.d_stride_m < 0 || d.d_stride_n < 0) return GEMM_ERR_LAYOUT;
  if (d.has_c && (d.c_stride_m < 0 || d.c_stride_n < 0)) return GEMM_ERR_LAYOUT;

  gemm_handle_s h;
  std::memset(&h, 0, sizeof(h));
  h.d = d;
  int rc = classify(d.a_stride_m, d.a_stride_k, &h.a);
  if (rc) return rc;
  rc = classify(d.b_stride_n, d.b_stride_k, &h.b);
  if (rc) return rc;
  if (d.ragged_m && !h.a.kmajor) return GEMM_ERR_LAYOUT;
  rc = check_arch();
  if (rc) return rc;

  // the 16-byte loaders need every problem's operand base 16-byte aligned
  const int64_t isz = dtype_size(d.a_type);
  const bool va = vec_ok(h.a, d.M, d.K, d.a_type) &&
                  (L == 1 || d.ragged_m || d.grouped || (d.a_stride_l * isz) % 16 == 0);
  const bool vb = vec_ok(h.b, d.N, d.K, d.b_type) &&
                  (L == 1 || d.grouped || (d.b_stride_l * isz) % 16 == 0);
  const bool need_split = d.split_k > 1;
  // no split of a batch, a group or a product with a row reduction
  // (and Stream-K, when forced, in place of any split)
  const int split_req = L > 1 || d.ragged_m || d.grouped || d.has_row_sumsq || d.has_col_sum ||
                                d.decomposition == 2
                            ? 1 : d.split_k;
  double fallback_us = 0.0;
  h.fallback = choose(h, va, vb, false, split_req, &fallback_us);
  if (h.fallback < 0) return GEMM_ERR_NO_CONFIG;
  if (d.force_config < 0 && repack_allowed(d, va && vb)) {
    // the product runs on aligned K-major copies of A and B: choose for that problem
    gemm_handle_s v = h;
    v.kp = (d.K + 16 / isz - 1) / (16 / isz) * (16 / isz);
    v.d.K = v.kp;
    v.d.a_stride_m = v.kp;
    v.d.a_stride_k = 1;
    v.d.b_stride_k = 1;
    v.d.b_stride_n = v.kp;
    v.a = Operand{true, v.kp};
    v.b = Operand{true, v.kp};
    double inner_us = 0.0;
    const int inner = choose(v, true, true, true, split_req, &inner_us);
    // the copies read and write A and B once
    const double copy_us = kRepackFixedUs + kRepackUsPerByte * 2.0 * double(d.M + d.N) *
                                                double(v.kp) * double(isz);
    if (inner >= 0 && table()[inner].vec && copy_us + inner_us < fallback_us) {
      h.repack = 1;
      h.kp = v.kp;
      h.cfg = h.fallback = inner;
      h.repack_bytes_a = ((size_t)d.M * v.kp * isz + 255) / 256 * 256;
      h.repack_bytes_b = ((size_t)d.N * v.kp * isz + 255) / 256 * 256;
      if (!entry_maps_ok(table()[inner])) return GEMM_ERR_LANE_MAP;
      h.group_m = 4;
      set_plan(&h, make_plan(table()[inner], v.d, split_req));
      h.predicted_us += copy_us;
      h.split_fb = h.split_cfg;
      h.kps_fb = h.kps_cfg;
      gemm_handle_s* p = new (std::nothrow) gemm_handle_s(h);
      if (!p) return GEMM_ERR_INVALID_ARG;
      p->magic = kMagic;
      *out = p;
      return GEMM_OK;
    }
  }
  if (d.force_config >= 0) {
    if (d.force_config >= table_size() || !entry_fits(table()[d.force_config], h, va, vb))
      return GEMM_ERR_NO_CONFIG;
    if (need_split && table()[d.force_config].max_split_k <= 1) return GEMM_ERR_NO_CONFIG;
    h.cfg = d.force_config;
  } else {
    h.cfg = (va && vb) ? choose(h, va, vb, true, split_req) : -1;
    if (h.cfg < 0) h.cfg = h.fallback;
  }
  // the chosen kernels' thread-to-data maps, checked once per atom against the layout helper
  if (!entry_maps_ok(table()[h.cfg]) || !entry_maps_ok(table()[h.fallback])) return GEMM_ERR_LANE_MAP;
  h.group_m = 4;
  // split, Stream-K or split tail, as the plan for the chosen entry has it
  set_plan(&h, make_plan(table()[h.cfg], d, split_req));
  plan_split(table()[h.fallback], d, split_req, &h.split_fb, &h.kps_fb);

  gemm_handle_s* p = new (std::nothrow) gemm_handle_s(h);
  if (!p) return GEMM_ERR_INVALID_ARG;
  p->magic = kMagic;
  *out = p;
  return GEMM_OK;
}

}  // extern "C"

namespace {
// Workspace of the fused reductions, for whichever entry a run uses: the row partials (one per
// tile column and row) first, then the column partials (one per tile row, row group and column);
// *col_off receives the byte offset of the column part.
size_t reduction_bytes(const gemm_handle_s& h, size_t* col_off) {
  const KernelEntry& c = table()[h.cfg];
  const KernelEntry& f = table()[h.fallback];
  size_t rows = 0, cols = 0;
  if (h.d.has_row_sumsq)
    rows = (size_t)std::max(cdiv(h.d.N, c.bn), cdiv(h.d.N, f.bn)) * (size_t)h.d.M * sizeof(float);
  if (h.d.has_col_sum)
    cols = (size_t)std::max(cdiv(h.d.M, c.bm) * col_sum_row_groups(c),
                            cdiv(h.d.M, f.bm) * col_sum_row_groups(f)) * (size_t)h.d.N * sizeof(float);
  rows = (rows + 255) / 256 * 256;
  if (col_off) *col_off = rows;
  return rows + cols;
}
}  // namespace

namespace {
size_t inner_workspace(const gemm_handle_s& h);
// grouped launches: G + 1 effective offsets (int32, padded to 256 bytes), then G + 1 first tiles
size_t group_lo_bytes(int64_t G) { return ((size_t)(G + 1) * 4 + 255) / 256 * 256; }
// independent problems: the problem table (padded to 256 bytes), then their G + 1 first tiles
size_t problem_table_bytes(int64_t G) {
  return ((size_t)G * sizeof(GroupProblem) + 255) / 256 * 256;
}
size_t group_table_bytes(const gemm_handle_s& h) {
  if (h.d.grouped) return problem_table_bytes(h.d.batch) + (size_t)(h.d.batch + 1) * 8;
  return h.d.ragged_m ? group_lo_bytes(h.d.batch) + (size_t)(h.d.batch + 1) * 8 : 0;
}
}  // namespace

extern "C" {

int gemm_workspace_size(gemm_t h, size_t* bytes) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (!bytes) return GEMM_ERR_INVALID_ARG;
  *bytes = h->repack_bytes_a + h->repack_bytes_b + inner_workspace(*h) + group_table_bytes(*h);
  return GEMM_OK;
}

}  // extern "C"

namespace {
// Workspace of the kernels proper (split-K planes, split-tail partials or reduction partials).
size_t inner_workspace(const gemm_handle_s& hh) {
  const gemm_handle_s* h = &hh;
  size_t v = 0;
  size_t* bytes = &v;
  const int s = std::max(h->split_cfg, h->split_fb);
  *bytes = s > 1 ? (size_t)s * (size_t)h->d.M * (size_t)h->d.N * sizeof(float) : 0;
  if (h->tail_split > 1) {
    const KernelEntry& e = table()[h->cfg];
    *bytes = std::max(*bytes, (size_t)h->tail_split * (size_t)h->tail_tiles * (size_t)e.bm *
                                  (size_t)e.bn * sizeof(float));
  }
  if (h->sk_tiles > 0) {
    const KernelEntry& e = table()[h->cfg];
    *bytes = std::max(*bytes, (size_t)2 * kCUs * (size_t)e.bm * (size_t)e.bn * sizeof(float));
  }
  if (h->d.has_row_sumsq || h->d.has_col_sum) *bytes = reduction_bytes(*h, nullptr);
  return v;
}
}  // namespace

extern "C" {

int gemm_get_info(gemm_t h, gemm_info* info) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (!info) return GEMM_ERR_INVALID_ARG;
  const KernelEntry& e = table()[h->cfg];
  std::memset(info, 0, sizeof(*info));
  info->config = h->cfg;
  info->fallback = h->fallback;
  info->bm = e.bm;
  info->bn = e.bn;
  info->bk = e.bk;
  info->waves = e.waves;
  info->stages = e.stages;
  info->lds_bytes = e.lds_bytes;
  info->split_k = h->split_cfg;
  const int64_t groups = h->d.batch > 1 ? h->d.batch : 1;
  info->grid = h->d.ragged_m ? (cdiv(h->d.M, e.bm) + groups) * cdiv(h->d.N, e.bn)
                             : cdiv(h->d.M, e.bm) * cdiv(h->d.N, e.bn) * h->split_cfg * groups;
  std::strncpy(info->name, e.name, sizeof(info->name) - 1);
  info->tail_tiles = h->tail_split > 1 ? h->tail_tiles : 0;
  info->tail_split = h->tail_split;
  info->repack = h->repack;
  info->sk_tiles = h->sk_tiles;
  info->sk_wgs = h->sk_tiles > 0 ? kCUs : 0;
  info->predicted_us = h->predicted_us;
  return GEMM_OK;
}

}  // extern "C"

namespace {

int run_impl(gemm_t h, const void* A, const void* B, const void* C, void* D, const void* bias,
             const float* row_scale, const float* col_scale, float alpha, float beta,
             float scale_a, float scale_b, void* workspace, const int32_t* offsets,
             float* row_sumsq, float* col_sum, void* stream) {
  const gemm_desc& d = h->d;
  if (d.grouped) return GEMM_ERR_INVALID_ARG;  // independent problems run through gemm_run_problems
  if ((d.has_row_sumsq != 0) != (row_sumsq != nullptr)) return GEMM_ERR_INVALID_ARG;
  if ((d.has_col_sum != 0) != (col_sum != nullptr)) return GEMM_ERR_INVALID_ARG;
  if ((row_sumsq && !aligned(row_sumsq, 4)) || (col_sum && !aligned(col_sum, 4)))
    return GEMM_ERR_MISALIGNED;
  if ((d.ragged_m != 0) != (offsets != nullptr)) return GEMM_ERR_INVALID_ARG;
  if (offsets && !aligned(offsets, 4)) return GEMM_ERR_MISALIGNED;
  const bool read_c = d.has_c && beta != 0.0f;
  if (!d.has_c && beta != 0.0f) return GEMM_ERR_INVALID_ARG;
  if ((d.has_row_scale != 0) != (row_scale != nullptr) || (d.has_col_scale != 0) != (col_scale != nullptr))
    return GEMM_ERR_INVALID_ARG;
  if (d.M == 0 || d.N == 0) return GEMM_OK;
  if (!D || (d.K > 0 && (!A || !B)) || (read_c && !C) || (d.has_bias && !bias))
    return GEMM_ERR_INVALID_ARG;
  if ((row_scale && !aligned(row_scale, 4)) || (col_scale && !aligned(col_scale, 4)))
    return GEMM_ERR_MISALIGNED;
  const size_t in_sz = dtype_size(d.a_type), out_sz = dtype_size(d.d_type);
  if (!aligned(A, in_sz) || !aligned(B, in_sz) || !aligned(D, out_sz) ||
      (read_c && !aligned(C, out_sz)) || (d.has_bias && !aligned(bias, out_sz)))
    return GEMM_ERR_MISALIGNED;

  // The operands the kernels read: A and B themselves, or (repack plan) their aligned K-major
  // copies in the workspace, written by one copy kernel each on `stream` before the product.
  const void* Ae = A;
  const void* Be = B;
  int64_t lda = h->a.ld, ldb = h->b.ld, Ke = d.K;
  if (h->repack) {
    if (!workspace || !aligned(workspace, 16)) return GEMM_ERR_INVALID_ARG;
    char* ws = static_cast<char*>(workspace);
    const bool a_direct = h->a.kmajor && (h->a.ld * (int64_t)in_sz) % 16 == 0 && h->a.ld >= d.K &&
                          h->kp == d.K && aligned(A, 16);
    const bool b_direct = h->b.kmajor && (h->b.ld * (int64_t)in_sz) % 16 == 0 && h->b.ld >= d.K &&
                          h->kp == d.K && aligned(B, 16);
    // both copies in one launch where the pair kernel can take them
    const hipError_t err = launch_repack_pair(
        a_direct ? nullptr : A, ws, d.M, d.a_stride_m, d.a_stride_k, b_direct ? nullptr : B,
        ws + h->repack_bytes_a, d.N, d.b_stride_n, d.b_stride_k, d.K, h->kp, (int)in_sz,
        (hipStream_t)stream);
    if (err != hipSuccess) return GEMM_ERR_LAUNCH;
    if (!a_direct) {
      Ae = ws;
      lda = h->kp;
    }
    if (!b_direct) {
      Be = ws + h->repack_bytes_a;
      ldb = h->kp;
    }
    Ke = h->kp;
    workspace = ws + h->repack_bytes_a + h->repack_bytes_b;
  }

  int idx = h->cfg;
  if (table()[idx].vec && (!aligned(Ae, 16) || !aligned(Be, 16))) idx = h->fallback;
  const KernelEntry& e = table()[idx];
  const int split = idx == h->cfg ? h->split_cfg : h->split_fb;
  const int64_t kps = idx == h->cfg ? h->kps_cfg : h->kps_fb;
  const bool tail = idx == h->cfg && h->tail_split > 1;
  const bool sk = idx == h->cfg && h->sk_tiles > 0;
  if ((split > 1 || tail || sk || row_sumsq || col_sum) && (!workspace || !aligned(workspace, 16)))
    return GEMM_ERR_INVALID_ARG;

  KParams p;
  std::memset(&p, 0, sizeof(p));
  p.A = Ae;
  p.B = Be;
  p.C = read_c ? C : nullptr;
  p.D = D;
  p.bias = d.has_bias ? bias : nullptr;
  p.M = d.M;
  p.N = d.N;
  p.K = Ke;
  p.lda = lda;
  p.ldb = ldb;
  p.c_sm = d.c_stride_m;
  p.c_sn = d.c_stride_n;
  p.d_sm = d.d_stride_m;
  p.d_sn = d.d_stride_n;
  p.alpha = alpha * scale_a * scale_b;
  p.beta = beta;
  p.has_c = read_c ? 1 : 0;
  p.has_bias = d.has_bias;
  p.act = d.act;
  p.tiles_m = (int)cdiv(d.M, e.bm);
  p.tiles_n = (int)cdiv(d.N, e.bn);
  p.tile_bm = e.bm;
  p.tile_bn = e.bn;
  p.group_m = h->group_m;
  p.split_k = split;
  p.k_per_split = (int)kps;
  p.workspace = split > 1 ? static_cast<float*>(workspace) : nullptr;
  size_t col_off = 0;
  if (row_sumsq || col_sum) reduction_bytes(*h, &col_off);
  p.rsq_ws = row_sumsq ? static_cast<float*>(workspace) : nullptr;
  p.csum_ws = col_sum ? reinterpret_cast<float*>(static_cast<char*>(workspace) + col_off) : nullptr;
  p.row_scale = row_scale;
  p.col_scale = col_scale;
  p.has_row_scale = row_scale ? 1 : 0;
  p.has_col_scale = col_scale ? 1 : 0;
  p.batch = d.batch > 1 ? (int)d.batch : 1;
  p.a_bstride = d.a_stride_l * (int64_t)in_sz;
  p.b_bstride = d.b_stride_l * (int64_t)in_sz;
  p.c_bstride = d.c_stride_l * (int64_t)out_sz;
  p.d_bstride = d.d_stride_l * (int64_t)out_sz;
  if (read_c) {
    const int64_t span = ((d.M - 1) * d.c_stride_m + (d.N - 1) * d.c_stride_n + 1) * (int64_t)out_sz;
    p.c_span = span < (int64_t(1) << 31) - 64 ? span : 0;
  }
  p.clock_rec = h->clock_rec;
  p.clock_cap = h->clock_rec ? h->clock_cap : 0;
  int64_t grid = int64_t(p.tiles_m) * p.tiles_n;
  unsigned gz = (unsigned)p.batch;
  if (offsets) {
    // grouped: every group's tiles in one x range, sized for the most tiles any split of the M
    // rows into `batch` groups can need (each group adds at most one partial tile row); the
    // groups' tile table is built on the stream first, in the workspace
    if (!workspace || !aligned(workspace, 16)) return GEMM_ERR_INVALID_ARG;
    int32_t* glo = static_cast<int32_t*>(workspace);
    int64_t* gbase = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + group_lo_bytes(d.batch));
    if (launch_group_scan(offsets, (int)d.batch, d.M, e.bm, p.tiles_n, glo, gbase,
                          (hipStream_t)stream) != hipSuccess)
      return GEMM_ERR_LAUNCH;
    p.group_lo = glo;
    p.group_base = gbase;
    p.offsets = offsets;
    p.a_row_bytes = h->a.ld * (int64_t)in_sz;
    p.c_row_bytes = d.c_stride_m * (int64_t)out_sz;
    p.d_row_bytes = d.d_stride_m * (int64_t)out_sz;
    grid = (int64_t(p.tiles_m) + p.batch) * p.tiles_n;
    gz = 1;
  }
  if (grid <= 0 || grid > INT32_MAX) return GEMM_ERR_INVALID_ARG;
  if (sk) {
    // the tiles before the Stream-K part whole (tile order 0 .. grid - sk_tiles - 1), then the
    // persistent workgroups over the rest, then the sum of the shared tiles' pieces
    const int64_t whole = grid - h->sk_tiles;
    hipError_t err = whole > 0 ? e.launch(p, (hipStream_t)stream, dim3((unsigned)whole, 1, 1))
                               : hipSuccess;
    KParams q = p;
    q.tile_base = (int)whole;
    q.sk_tiles = h->sk_tiles;
    q.sk_nkt = (int)cdiv(Ke, e.bk);
    q.sk_wgs = kCUs;  // a multiple of 8 (the kernel spreads shares over the 8 XCDs)
    q.workspace = static_cast<float*>(workspace);
    if (err == hipSuccess) err = e.launch_sk(q, (hipStream_t)stream, dim3((unsigned)kCUs, 1, 1));
    if (err == hipSuccess) err = launch_sk_fixup(q, d.d_type, (hipStream_t)stream);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
  }
  if (tail) {
    // whole tiles first (tile order 0 .. grid - R - 1), then the R tail tiles split along K,
    // then their fixed-order sum and epilogue
    const int64_t whole = grid - h->tail_tiles;
    hipError_t err = e.launch(p, (hipStream_t)stream, dim3((unsigned)whole, 1, 1));
    KParams q = p;
    q.tile_base = (int)whole;
    q.tail_tiles = h->tail_tiles;
    q.split_k = h->tail_split;
    q.k_per_split = (int)h->tail_kps;
    q.workspace = static_cast<float*>(workspace);
    if (err == hipSuccess)
      err = e.launch(q, (hipStream_t)stream, dim3((unsigned)h->tail_tiles, (unsigned)h->tail_split, 1));
    if (err == hipSuccess) err = launch_tail_reduce(q, d.d_type, (hipStream_t)stream);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
  }
  hipError_t err = e.launch(p, (hipStream_t)stream, dim3((unsigned)grid, (unsigned)split, gz));
  if (err == hipSuccess && split > 1) err = launch_splitk_reduce(p, d.d_type, (hipStream_t)stream);
  if (err == hipSuccess && row_sumsq)
    err = launch_row_sumsq_reduce(p.rsq_ws, row_sumsq, d.M, p.tiles_n, (hipStream_t)stream);
  if (err == hipSuccess && col_sum)
    err = launch_row_sumsq_reduce(p.csum_ws, col_sum, d.N, p.tiles_m * col_sum_row_groups(e),
                                  (hipStream_t)stream);
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_run(gemm_t h, const void* A, const void* B, const void* C, void* D, const void* bias,
             float alpha, float beta, float scale_a, float scale_b, void* workspace,
             void* stream) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  // a handle with scale vectors or a row reduction needs gemm_run_ex to receive them
  if (h->d.has_row_scale || h->d.has_col_scale || h->d.has_row_sumsq || h->d.has_col_sum)
    return GEMM_ERR_INVALID_ARG;
  return run_impl(h, A, B, C, D, bias, nullptr, nullptr, alpha, beta, scale_a, scale_b,
                  workspace, nullptr, nullptr, nullptr, stream);
}

int gemm_set_clock_record(gemm_t h, uint64_t* records, int64_t max_workgroups) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (records && (max_workgroups < 0 || !aligned(records, 8))) return GEMM_ERR_INVALID_ARG;
  h->clock_rec = reinterpret_cast<unsigned long long*>(records);
  h->clock_cap = records ? max_workgroups : 0;
  return GEMM_OK;
}

int gemm_run_ex(gemm_t h, const gemm_args* a, void* stream) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (!a) return GEMM_ERR_INVALID_ARG;
  return run_impl(h, a->A, a->B, a->C, a->D, a->bias, a->row_scale, a->col_scale, a->alpha,
                  a->beta, a->scale_a, a->scale_b, a->workspace, nullptr, a->row_sumsq, a->col_sum,
                  stream);
}

int gemm_run_grouped(gemm_t h, const gemm_args* a, const int32_t* offsets, void* stream) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (!a || !offsets) return GEMM_ERR_INVALID_ARG;
  return run_impl(h, a->A, a->B, a->C, a->D, a->bias, a->row_scale, a->col_scale, a->alpha,
                  a->beta, a->scale_a, a->scale_b, a->workspace, offsets, a->row_sumsq, a->col_sum,
                  stream);
}

int gemm_run_problems(gemm_t h, const gemm_problem* probs, int64_t count, const gemm_args* a,
                      void* stream) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  const gemm_desc& d = h->d;
  if (!d.grouped || !a) return GEMM_ERR_INVALID_ARG;
  if (count < 0 || count > d.batch || (count > 0 && !probs)) return GEMM_ERR_INVALID_ARG;
  // the per-problem pointers come with the problems; per-row and per-column vectors are refused
  if (a->A || a->B || a->C || a->D || a->bias || a->row_scale || a->col_scale || a->row_sumsq ||
      a->col_sum)
    return GEMM_ERR_INVALID_ARG;
  if (!d.has_c && a->beta != 0.0f) return GEMM_ERR_INVALID_ARG;
  const bool read_c = d.has_c && a->beta != 0.0f;
  const size_t in_sz = dtype_size(d.a_type), out_sz = dtype_size(d.d_type);
  const KernelEntry& vec_e = table()[h->cfg];
  const KernelEntry& fb_e = table()[h->fallback];
  // Is problem q within the reach of entry e (the 31-bit tile offsets of its loaders)?
  auto fits = [&](const KernelEntry& e, const gemm_problem& q) {
    gemm_handle_s t = *h;
    t.d.M = q.M;
    t.d.N = q.N;
    t.d.K = q.K;
    t.a.ld = q.lda;
    t.b.ld = q.ldb;
    return entry_fits(e, t, true, true);
  };
  // arguments of every problem first: an error launches nothing
  bool use_vec = vec_e.vec != 0;
  for (int64_t i = 0; i < count; ++i) {
    const gemm_problem& q = probs[i];
    if (q.M < 0 || q.N < 0 || q.K < 0) return GEMM_ERR_INVALID_ARG;
    if (q.M > INT32_MAX / 2 || q.N > INT32_MAX / 2 || q.K > INT32_MAX / 2) return GEMM_ERR_INVALID_ARG;
    if (q.lda < 0 || q.ldb < 0 || q.ldc < 0 || q.ldd < 0) return GEMM_ERR_LAYOUT;
    if (q.M == 0 || q.N == 0) continue;
    if (!q.D || (q.K > 0 && (!q.A || !q.B)) || (read_c && !q.C) || (d.has_bias && !q.bias))
      return GEMM_ERR_INVALID_ARG;
    if (!aligned(q.A, in_sz) || !aligned(q.B, in_sz) || !aligned(q.D, out_sz) ||
        (read_c && !aligned(q.C, out_sz)) || (d.has_bias && !aligned(q.bias, out_sz)))
      return GEMM_ERR_MISALIGNED;
    if (use_vec)
      use_vec = vec_ok(Operand{h->a.kmajor, q.lda}, q.M, q.K, d.a_type) &&
                vec_ok(Operand{h->b.kmajor, q.ldb}, q.N, q.K, d.b_type) && aligned(q.A, 16) &&
                aligned(q.B, 16) && fits(vec_e, q);
  }
  const KernelEntry& e = use_vec ? vec_e : fb_e;
  if (!use_vec)
    for (int64_t i = 0; i < count; ++i)
      if (probs[i].M > 0 && probs[i].N > 0 && !fits(fb_e, probs[i])) return GEMM_ERR_NO_CONFIG;
  // the problem table and the problems' first tiles, built here and copied into the workspace
  const size_t rec_bytes = problem_table_bytes(count);
  const size_t bytes = rec_bytes + (size_t)(count + 1) * 8;
  std::vector<uint64_t> host((bytes + 7) / 8, 0);
  GroupProblem* rec = reinterpret_cast<GroupProblem*>(host.data());
  int64_t* base = reinterpret_cast<int64_t*>(reinterpret_cast<char*>(host.data()) + rec_bytes);
  int64_t total = 0;
  for (int64_t i = 0; i < count; ++i) {
    const gemm_problem& q = probs[i];
    GroupProblem& r = rec[i];
    r.A = q.A;
    r.B = q.B;
    r.C = read_c ? q.C : nullptr;
    r.D = q.D;
    r.bias = d.has_bias ? q.bias : nullptr;
    r.M = q.M;
    r.N = q.N;
    r.K = q.K;
    r.lda = q.lda;
    r.ldb = q.ldb;
    r.ldc = q.ldc;
    r.ldd = q.ldd;
    const bool empty = q.M == 0 || q.N == 0;
    r.tiles_m = empty ? 0 : (int32_t)cdiv(q.M, e.bm);
    r.tiles_n = empty ? 0 : (int32_t)cdiv(q.N, e.bn);
    if (read_c && !empty) {
      const int64_t csm = d.c_stride_n == 1 ? q.ldc : d.c_stride_m;
      const int64_t csn = d.c_stride_n == 1 ? 1 : q.ldc;
      const int64_t span = ((q.M - 1) * csm + (q.N - 1) * csn + 1) * (int64_t)out_sz;
      r.c_span = span < (int64_t(1) << 31) - 64 ? span : 0;
    }
    base[i] = total;
    total += int64_t(r.tiles_m) * r.tiles_n;
  }
  base[count] = total;
  if (total > INT32_MAX) return GEMM_ERR_INVALID_ARG;
  if (total == 0) return GEMM_OK;
  void* ws = a->workspace;
  if (!ws || !aligned(ws, 16)) return GEMM_ERR_INVALID_ARG;
  if (hipMemcpyAsync(ws, host.data(), bytes, hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess)
    return GEMM_ERR_HIP;

  KParams p;
  std::memset(&p, 0, sizeof(p));
  p.c_sm = d.c_stride_m;
  p.c_sn = d.has_c ? (d.c_stride_n == 1 ? 1 : d.c_stride_n) : 1;
  p.d_sm = d.d_stride_m;
  p.d_sn = d.d_stride_n == 1 ? 1 : d.d_stride_n;
  p.alpha = a->alpha * a->scale_a * a->scale_b;
  p.beta = a->beta;
  p.has_c = read_c ? 1 : 0;
  p.has_bias = d.has_bias;
  p.act = d.act;
  p.tile_bm = e.bm;
  p.tile_bn = e.bn;
  p.group_m = h->group_m;
  p.split_k = 1;
  p.batch = (int)count;
  p.problems = reinterpret_cast<const GroupProblem*>(ws);
  p.group_base = reinterpret_cast<const int64_t*>(static_cast<char*>(ws) + rec_bytes);
  const hipError_t err = e.launch(p, (hipStream_t)stream, dim3((unsigned)total, 1, 1));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"

// ---- the entry point that allocates nothing ----------------------------------------------
// Scratch for gemm_run_noalloc: one static device array per GPU, held until the process ends.
// Host code never uses the array's name as an address (it is a host-side stand-in); the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMM_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run_noalloc(gemm_t h, const gemm_args* a, void* stream) {
  if (!h || h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  if (!a || a->workspace) return GEMM_ERR_INVALID_ARG;  // the library supplies the scratch
  // grouped handles run through their own entry points
  if (h->d.ragged_m || h->d.grouped) return GEMM_ERR_INVALID_ARG;
  size_t need = 0;
  int rc = gemm_workspace_size(h, &need);
  if (rc) return rc;
  if (need > (size_t)GEMM_NOALLOC_SCRATCH_BYTES) return GEMM_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return run_impl(h, a->A, a->B, a->C, a->D, a->bias, a->row_scale, a->col_scale, a->alpha,
                  a->beta, a->scale_a, a->scale_b, ws, nullptr, a->row_sumsq, a->col_sum, stream);
}

int gemm_destroy(gemm_t h) {
  if (!h) return GEMM_OK;
  if (h->magic != kMagic) return GEMM_ERR_BAD_HANDLE;
  h->magic = kDead;
  delete h;
  return GEMM_OK;
}

const char* gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_DTYPE_COMBO: return "unsupported type combination";
    case GEMM_ERR_LAYOUT: return "operand has no unit stride";
    case GEMM_ERR_MISALIGNED: return "pointer not aligned to its element size";
    case GEMM_ERR_ARCH: return "device is not gfx950";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_ERR_BAD_HANDLE: return "invalid or destroyed handle";
    case GEMM_ERR_NO_CONFIG: return "no tile-table entry can run this problem";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_LANE_MAP: return "a kernel lane map disagrees with the layout helper";
    case GEMM_ERR_SCRATCH_LIMIT: return "the problem needs more scratch than gemm_run_noalloc holds";
    default: return "unknown status";
  }
}

int gemm_num_configs(void) { return table_size(); }

int gemm_atom_layouts(int dtype, int mi, char* op, char* acc, size_t cap) {
  const int idx = atom_index(dtype, mi);
  if (idx < 0 || !op || !acc) return GEMM_ERR_INVALID_ARG;
  const AtomMaps& M = kAtomMaps[idx];
  const size_t a = std::strlen(M.op.text), c = std::strlen(M.acc.text);
  if (a + 1 > cap || c + 1 > cap) return GEMM_ERR_INVALID_ARG;
  std::memcpy(op, M.op.text, a + 1);
  std::memcpy(acc, M.acc.text, c + 1);
  return atom_ok(dtype, mi) ? GEMM_OK : GEMM_ERR_LANE_MAP;
}

int gemm_config_name(int idx, char* out, size_t cap) {
  if (idx < 0 || idx >= table_size() || !out) return GEMM_ERR_INVALID_ARG;
  const char* n = table()[idx].name;
  size_t len = std::strlen(n);
  if (len + 1 > cap) return GEMM_ERR_INVALID_ARG;
  std::memcpy(out, n, len + 1);
  return GEMM_OK;
}

}  // extern "C"
