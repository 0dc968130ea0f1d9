// gemm_internal.h -- declarations shared by the host API (api.cpp) and the kernels (kernels.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace htk {

// Operand element types; the numbering matches gemm_dtype in htgemm.h.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_F8 = 3 };

// One problem of a grouped launch of independent problems, as the device reads it (the host
// builds the table in the workspace).  lda / ldb are the non-unit strides of A and B; ldc / ldd
// replace the stride of C / D that is not the unit one; c_span as in KParams.
struct GroupProblem {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  const void* bias;
  int64_t M, N, K;
  int64_t lda, ldb, ldc, ldd;
  int64_t c_span;
  int32_t tiles_m, tiles_n;
};
static_assert(sizeof(GroupProblem) == 112, "the table entry size the header documents");

// Arguments of one launch.  The operand of A or B with unit stride is implied by the kernel
// variant; lda / ldb is the other stride.  alpha already includes scale_a * scale_b.
struct KParams {
  const void* A;
  const void* B;
  const void* C;      // read only when has_c != 0
  void* D;
  const void* bias;   // read only when has_bias != 0
  int64_t M, N, K;
  int64_t lda, ldb;
  int64_t c_sm, c_sn, d_sm, d_sn;
  float alpha, beta;
  int has_c, has_bias, act;
  int tiles_m, tiles_n, group_m;
  int split_k;        // workgroups per output tile along K (1: none)
  int k_per_split;    // K elements per split (a multiple of the tile's K step)
  float* workspace;   // fp32 partials when split_k > 1
  const float* row_scale;  // read only when has_row_scale != 0: M values
  const float* col_scale;  // read only when has_col_scale != 0: N values
  int has_row_scale, has_col_scale;
  int batch;               // problems per launch (gridDim.z); 1: one
  int64_t c_span;          // bytes from C's base to the end of its last element when below
                           // 2^31 - 64 (range-checked buffer loads), else 0
  const int32_t* offsets;  // grouped launch: batch + 1 row offsets (device); nullptr otherwise
  const int32_t* group_lo;    // grouped: batch + 1 effective row offsets (gemm_group_scan)
  const int64_t* group_base;  // grouped: batch + 1 first tile indices of the groups
  int64_t a_row_bytes, c_row_bytes, d_row_bytes;  // bytes between consecutive rows (grouped)
  float* rsq_ws;           // row sums of squares: one partial per (tile column, row), or nullptr
  float* csum_ws;          // column sums: one partial per (tile row, row group, column), or nullptr
  int64_t a_bstride, b_bstride, c_bstride, d_bstride;  // bytes between consecutive problems
  // Split tail: the tiles of an incomplete last round, each split along K.  Workgroup x of such
  // a launch takes tile order index tile_base + (its place in the tile order of gridDim.x
  // workgroups); with tail_tiles > 0 its fp32 partials go to a compact workspace of
  // split_k x tail_tiles tiles of tile_bm x tile_bn (plane blockIdx.y, slot blockIdx.x).
  int tile_base, tail_tiles, tile_bm, tile_bn;
  // Grouped launch of independent problems: `batch` entries, and their first tiles in
  // group_base (batch + 1 values); nullptr otherwise.
  const GroupProblem* problems;
  // Stream-K launch (sk_wgs > 0): sk_wgs persistent workgroups share the sk_tiles * sk_nkt
  // k-tile iterations of the tiles from tile order tile_base on; pieces of shared tiles go to
  // compact BM x BN slots of the workspace (2 per workgroup).
  int sk_tiles, sk_nkt, sk_wgs;
  // Clock record (kernels that support it: the ping-pong kernel): workgroup w < clock_cap of the
  // launch (linear id over x, y, z) writes clock_rec[4w .. 4w + 3] = the shader-clock counter at
  // its start and end, then the constant-rate real-time counter at its start and end; nullptr
  // otherwise.
  unsigned long long* clock_rec;
  int64_t clock_cap;
};

typedef hipError_t (*launch_fn)(const KParams&, hipStream_t, dim3 grid);

// One entry of the tile table.
struct KernelEntry {
  const char* name;
  int dtype;          // operand type of A and B
  int a_kmajor;       // 1: A has unit stride along K (row-major A); 0: along M
  int b_kmajor;       // 1: B has unit stride along K (column-major B); 0: along N
  int vec;            // 1: 16-byte loads (needs aligned pointers / leading dims); 0: any alignment
  int skinny;         // 1: streaming kernel for small M
  int bm, bn, bk;     // workgroup tile
  int waves;          // waves per workgroup
  int stages;         // LDS stages
  int lds_bytes;      // LDS per workgroup
  int max_split_k;    // largest split along K the kernel supports (1: none)
  launch_fn launch;
  int realign;        // 1: realigned 16-byte loads of 2-byte elements (31-bit tile offsets)
  int mi;             // MFMA atom: MI x MI output block (its layouts are in atom_maps.h)
  int lds_row_chunks; // 16-byte chunks per swizzled LDS row of the operand tiles (4 or 8)
  int mn_rows;        // 1: an MN-major operand is kept as rows of k and read by transposing reads
  launch_fn launch_sk;  // the kernel's Stream-K form (persistent workgroups), or nullptr
  const struct EntryCost* cost;  // measured costs (set from the cost table by name), or nullptr:
                                 // then the entry runs only when forced
};

const KernelEntry* table();
int table_size();

// Measured cost of one entry on MI355X (cost_table.cpp, written by calibrate.py).  Index i =
// 0..10 stands for the load 1/4, 1/2, 3/4, 1, 2, ..., 8 (workgroups per compute unit): a launch
// of 256 * load workgroups of kt k-tiles each took f[i] + kt * c[i] microseconds.
constexpr int kCostLoads = 11;
constexpr int kCostLoadOne = 3;  // index of the load 1
struct EntryCost {
  const char* name;
  float f[kCostLoads];
  float c[kCostLoads];
  float edge_k;   // extra time of a partial last k-tile, per workgroup on the busiest CU
  float edge_mn;  // extra time of partial last tile rows or columns, once per launch
  float edge_d;   // extra time of D rows off 16 bytes, per workgroup on the busiest CU
};
extern const EntryCost kEntryCosts[];
extern const int kEntryCostCount;
// split-K second kernel and partial stores: kSplitFixedUs + kSplitUsPerByte * (partial bytes,
// written and read, plus output bytes)
extern const double kSplitFixedUs, kSplitUsPerByte;
// copies into aligned K-major buffers: kRepackFixedUs + kRepackUsPerByte * (bytes read and written)
extern const double kRepackFixedUs, kRepackUsPerByte;
// Stream-K launch and fix-up beyond the whole tiles: kSkFixedUs + kSkShareFactor * (the entry's
// time for 256 workgroups of one share of k-tiles)
extern const double kSkFixedUs, kSkShareFactor;

// Second kernel of a split-K run: D = act(alpha * sum of the split_k fp32 planes in
// p.workspace + beta * C + bias), with out_type the type of C, D and bias.
hipError_t launch_splitk_reduce(const KParams& p, int out_type, hipStream_t s);
// Second kernel of a split tail: for each of the p.tail_tiles tiles, D = act(alpha * sum of its
// split_k compact fp32 partials + beta * C + bias) over that tile.
hipError_t launch_tail_reduce(const KParams& p, int out_type, hipStream_t s);
// Second kernel of a Stream-K launch: each of the p.sk_tiles tiles that several workgroups
// shared gets D = act(alpha * (sum of its pieces in K order) + beta * C + bias).
hipError_t launch_sk_fixup(const KParams& p, int out_type, hipStream_t s);
// Sums the per-tile-column partials of the row sums of squares in fixed order: out[m] =
// sum over t < tiles_n of ws[t * M + m].
hipError_t launch_row_sumsq_reduce(const float* ws, float* out, int64_t M, int tiles_n, hipStream_t s);
// The same fixed-order sum for the column sums: out[n] = sum over t < planes of ws[t * N + n].
// (The row reduction is this with N = M and planes = tiles_n.)

// Copy of an operand into a K-major, 16-byte aligned, zero-padded buffer: dst[r * Kp + k] =
// src(r, k) (element offset r * s_row + k * s_k) for k < K, 0 for K <= k < Kp (repack.hip).
hipError_t launch_repack(const void* src, void* dst, int64_t rows, int64_t K, int64_t Kp,
                         int64_t s_row, int64_t s_k, int esize, hipStream_t s);
// The copies of both operands of a product (a NULL source skips that operand), in one launch
// when both are 2-byte copies the pair kernel takes, else one launch_repack each.
hipError_t launch_repack_pair(const void* a_src, void* a_dst, int64_t a_rows, int64_t a_srow,
                              int64_t a_sk, const void* b_src, void* b_dst, int64_t b_rows,
                              int64_t b_srow, int64_t b_sk, int64_t K, int64_t Kp, int esize,
                              hipStream_t s);

// Grouped launches: from the caller's G + 1 device row offsets, the effective offsets lo[0..G]
// (clamped into [0, M] and made non-decreasing) and the first tile of each group base[0..G]
// (base[G] = all tiles), groups of ceil((lo[e+1] - lo[e]) / bm) * tiles_n tiles in order.  One
// workgroup; the tile kernels then find their group by binary search.
hipError_t launch_group_scan(const int32_t* offsets, int G, int64_t M, int bm, int tiles_n,
                             int32_t* lo, int64_t* base, hipStream_t s);

// Output type of a given operand type (htgemm.h type table).
constexpr int out_dtype(int dt) { return dt == DT_F8 ? DT_BF16 : dt; }
constexpr int dtype_size(int dt) { return dt == DT_F32 ? 4 : (dt == DT_F8 ? 1 : 2); }

}  // namespace htk
