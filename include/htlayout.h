/*
 * htlayout.h -- host-side shape:stride layout functions and tile arithmetic (C ABI).
 *
 * A layout is a pair Shape:Stride of congruent (possibly nested) integer tuples; it is a function
 * from a coordinate to an offset, the inner product of the natural coordinate with the stride.
 * A single integer coordinate is first split over the shape with the leftmost mode fastest.
 * Sources: "CUTLASS, CuTe, and CUDA Tile" (learn-kernels.com), introduction and "Partitioning:
 * complement and divide"; "A10 - CuTe, CUTLASS & CuTile", sections 2 and 3.4; "CUTLASS"
 * (stanleyjacob.dev), Part V "CuTe layout algebra".
 *
 * Layouts cross this interface as text in the pages' notation, for example "(4,3):(3,1)",
 * "((2,2),3):((24,2),8)" or "12:1" (leading underscores as in "_12:_1" are accepted).
 * Coordinates are arrays of integers (ht_layout_eval) or text (ht_layout_eval_str, "(1,(0,1))");
 * an integer entry may stand for a whole nested mode and is split over it.
 *
 * Output strings are written to caller-owned buffers `out` of `cap` bytes, NUL-terminated;
 * HT_ERR_CAPACITY means the buffer was too small (nothing useful is written).  Every function is
 * pure host code, thread-safe and allocation-free from the caller's view.
 */
#ifndef HTLAYOUT_H
#define HTLAYOUT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HT_OK = 0,
  HT_ERR_PARSE = 1,           /* text is not a layout / coordinate, or not congruent        */
  HT_ERR_RANGE = 2,           /* coordinate outside the shape, or an argument out of range   */
  HT_ERR_NOT_COMPOSABLE = 3,  /* the divisibility conditions of composition fail             */
  HT_ERR_CAPACITY = 4,        /* output buffer too small                                      */
  HT_ERR_NO_COMPLEMENT = 5    /* no ordered complement exists under the given size           */
};

/* Offset of a coordinate in `layout` ("CUTLASS, CuTe, and CUDA Tile", introduction:
 * (4,3):(3,1) maps (1,0) to 3 and (0,1) to 1).  `coord` holds `rank` integers owned by the
 * caller: rank 1 is a single integer over the whole layout (split over its modes, leftmost
 * fastest, as a 1-D coordinate); rank r > 1 gives one integer per top-level mode of a layout
 * with r top-level modes, each split over its mode if that mode is nested.  HT_ERR_RANGE for
 * another rank or a coordinate outside the shape; HT_ERR_PARSE for bad text or NULL. */
int ht_layout_eval(const char* layout, const int64_t* coord, int rank, int64_t* out);

/* The same with the coordinate as text in the pages' notation, nested as deep as the shape:
 * "(1,0)", "5", "(1,(0,1))". */
int ht_layout_eval_str(const char* layout, const char* coord, int64_t* out);

/* Number of coordinates (product of the shape). */
int ht_layout_size(const char* layout, int64_t* out);

/* The layout on 1-D coordinates 0 .. size-1, written to out[0 .. size-1]; cap is in elements. */
int ht_layout_table(const char* layout, int64_t* out, int64_t cap);

/* Shortest spelling of the same 1-D function: flatten, drop size-1 modes, merge neighbours
 * (s0:d0)(s1:d1) whenever d1 == s0*d0 (introduction: coalesce of (2,(1,6)):(1,(6,2)) is 12:1). */
int ht_layout_coalesce(const char* layout, char* out, size_t cap);

/* Functional composition R = A o B, R(c) = A(B(c)), with R compatible with B (introduction:
 * (6,2):(8,2) o (4,3):(3,1) = ((2,2),3):((24,2),8)).  HT_ERR_NOT_COMPOSABLE when a stride of B
 * does not divide through A's modes or a size of B does not fit them. */
int ht_layout_compose(const char* a, const char* b, char* out, size_t cap);

/* complement(A, M): the ordered layout (positive increasing strides) whose image together with
 * A's tiles 0 .. M-1 without overlap ("Partitioning: complement and divide":
 * complement(4:1,24) = 6:4, complement(6:4,24) = 4:1). */
int ht_layout_complement(const char* a, int64_t m, char* out, size_t cap);

/* logical_divide(A, B) = A o (B, complement(B, size(A))): mode 0 is the tile B selects, mode 1
 * iterates over the tiles ("Partitioning: complement and divide":
 * logical_divide((4,2,3):(2,1,8), 4:2) = ((2,2),(2,3)):((4,1),(2,8))). */
int ht_layout_logical_divide(const char* a, const char* b, char* out, size_t cap);

/* zipped_divide of a rank-2 layout by one tiler per mode, "<t0,t1>" with each t a layout:
 * ((tile0,tile1),(rest0,rest1)) -- tile modes first, rest modes second. */
int ht_layout_zipped_divide(const char* a, const char* tiler0, const char* tiler1, char* out,
                            size_t cap);

/* local_tile: a block's view of a big layout ("CUTLASS, CuTe, and CUDA Tile", "Partitioning:
 * complement and divide", the local_tile listing; "CUTLASS" (stanleyjacob.dev), Part V).  Two
 * steps: zipped_divide of `a` by the tiler, then the rest part sliced at `coord`.
 *   tiler  tile sizes, one per leading mode of `a`, e.g. "(128,64)"; mode i is divided by the
 *          tile t_i:1 and must have a size that t_i divides (else HT_ERR_NOT_COMPOSABLE); modes
 *          past the tiler are kept whole in the rest part.
 *   coord  one entry per mode of `a`: an integer selects that tile (1-D index into the mode's
 *          rest part), "_" keeps the whole rest mode, e.g. "(1,_)".
 *   proj   NULL, or a step tuple such as "(1,X,1)" with one entry per tiler and coord entry:
 *          entries marked X are dropped from both before the two steps.
 * The result is written as one layout whose modes are the tile modes followed by the kept rest
 * modes, e.g. (BLK_M,BLK_K,k), plus the base offset of the selected tile in *offset: element c
 * of the view is at *offset + result(c).  HT_ERR_RANGE for a coordinate outside its mode or a
 * rank mismatch. */
int ht_layout_local_tile(const char* a, const char* tiler, const char* coord, const char* proj,
                         int64_t* offset, char* out, size_t cap);

/* local_partition: a thread's elements of a tile under a thread layout of shape `thr_shape`
 * (same pages; "A10 - CuTe, CUTLASS & CuTile", "Partitioning Tensors").  The pages give only
 * the purpose; the reading implemented is zipped_divide of `a` by the thread shape (one entry per
 * leading mode) with the tile part sliced at thread `idx`'s coordinate (leftmost mode fastest),
 * keeping every rest mode: thread idx owns one element per tile, at the same place in each.
 * The result is the rest layout plus *offset, as for local_tile.  HT_ERR_RANGE when idx is not
 * below the number of threads. */
int ht_layout_local_partition(const char* a, const char* thr_shape, int64_t idx, int64_t* offset,
                              char* out, size_t cap);

/* Swizzle<BBits, MBase, SShift>: offset XOR ((offset & mask) >> SShift), where mask is BBits
 * ones starting at bit MBase + SShift ("A10 - CuTe, CUTLASS & CuTile", section 3.4). */
int64_t ht_swizzle(int64_t offset, int bbits, int mbase, int sshift);

/* ---- tile arithmetic ("CuTe DSL / CUDA Tile" blog post, "A tile is a plan for reuse") ---- */
typedef struct ht_tile_stats {
  int64_t flops;              /* 2*m*n*k                                                      */
  int64_t bytes;              /* b*(m*k + k*n + m*n): inputs read once, output written once    */
  double intensity;           /* flops / bytes                                                 */
  int64_t double_buffer_bytes;/* two stages of the A and B tiles: 2*b*(m*k + k*n)              */
  int32_t fits;               /* double_buffer_bytes <= budget_bytes                           */
} ht_tile_stats;

int ht_tile_plan(int64_t m, int64_t n, int64_t k, int bytes_per_elem, int64_t budget_bytes,
                 ht_tile_stats* out);

/* Ideal two-engine pipeline time for n tiles ("Pipelining hides a wait only when another
 * resource can work"): load + compute + (n - 1) * max(load, compute); n == 0 gives 0. */
double ht_pipeline_time(int64_t n, double load, double compute);

#ifdef __cplusplus
}
#endif
#endif /* HTLAYOUT_H */
