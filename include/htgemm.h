/*
 * htgemm.h -- C ABI of the MI355X (gfx950) hierarchically tiled GEMM library.
 *
 * Operation (all entry points below compute or describe this one operation):
 *
 *     D = act( alpha * scale_a * scale_b * row_scale[m] * col_scale[n] * (A @ B)
 *              +  beta * C  +  bias )
 *
 * with A an M x K matrix, B a K x N matrix, C and D M x N matrices and bias a length-N vector
 * added to every row; row_scale (length M) and col_scale (length N) are optional fp32 vectors
 * (1 when absent), and a batch of L problems of one shape may run in one call (D_l from A_l,
 * B_l, C_l, sharing bias and the scale vectors).  This is the GEMM the reference pages are built around ("CUTLASS",
 * stanleyjacob.dev, Part I "The mental model": D = alpha * (A @ B) + beta * C; Part II "Using
 * it": the problem shape, a {pointer, leading dimension} per operand and {alpha, beta}, checked
 * against a success status).  The epilogue order -- alpha/beta, then bias, then activation --
 * follows the same page's Part I diagram and Part IV Stage 5 ("The epilogue and fusion"); the
 * per-tensor dequantisation scales of a narrow-type GEMM are folded into the epilogue as the
 * page's Part V "Data types and quantization" describes.  The per-column scale vector is the
 * per-channel dequantisation scale an epilogue visitor tree fuses (Part IV Stage 5); the per-row
 * vector is the same broadcast along M (per-token activation scales), and SiLU is a further
 * activation of the kind the "A10 - CuTe, CUTLASS & CuTile" page's drill answer 8 names (a
 * custom fused epilogue of bias, a nonstandard activation and a quantisation scale).  The batch
 * is the fourth mode L of the problem shape [M, N, K, L] ("CUTLASS, CuTe, and CUDA Tile",
 * "Assembling a CUTLASS kernel").  Products accumulate in fp32 whatever the operand type.
 *
 * Handle life cycle ("CUTLASS", Part IV Stage 1: get_workspace_size, can_implement, initialize,
 * run; and "CUTLASS, CuTe, and CUDA Tile", section "Assembling a CUTLASS kernel": a stateful,
 * reusable handle whose kernel chooses its own grid):
 *   gemm_create         validates the problem ("can_implement") and picks a kernel from the
 *                       tile table; it allocates host memory only.
 *   gemm_workspace_size reports the device scratch the caller must pass to gemm_run (non-zero
 *                       only for a problem split along K).
 *   gemm_run            enqueues the kernel on the caller's HIP stream; asynchronous.
 *   gemm_run_ex         the same with the arguments in a struct, including the scale vectors.
 *   gemm_run_grouped    a grouped GEMM whose groups split M by device offsets.
 *   gemm_run_problems   a grouped GEMM of independent problems of any shapes.
 *   gemm_set_clock_record  asks the product kernel to record the clock of each launch
 *                       (measurement).
 *   gemm_destroy        frees the handle.
 *
 * Ownership: the caller owns every device buffer (A, B, C, D, bias, row_scale, col_scale,
 * workspace) and the stream.
 * A handle holds host memory only and is immutable after gemm_create (except for the clock
 * record that gemm_set_clock_record attaches), so one handle may be run concurrently on several
 * streams.  Nothing throws across this interface; every function returns
 * a status code (GEMM_OK == 0) that gemm_status_string() describes.
 *
 * Element addressing: element (i, j) of an operand with strides (s0, s1) is at element offset
 * i * s0 + j * s1 from its base pointer.  Each of A and B must have one unit stride (row-major A
 * has a_stride_k == 1; column-major B has b_stride_k == 1).  C and D may have any strides.
 * D may alias C only when their strides are identical; any other overlap is undefined.
 *
 * Conventions where the pages are silent:
 *   - beta == 0 means C is not read at all (C may be NULL; NaNs in C do not propagate).
 *   - alpha == 0 is not special-cased: NaN or Inf in A or B still propagate through 0 * x.
 *   - GELU is the exact form x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt(2))); the kernels evaluate
 *     erf with the branch-free Abramowitz-Stegun formula 7.1.26 (|error| <= 1.5e-7, far below
 *     the output rounding), not the tanh approximation.
 *   - fp8 is OCP E4M3 ("fn": bias 7, max 448, no infinities); outputs round to nearest even.
 *   - M == 0 or N == 0 is a valid empty problem; K == 0 gives D = act(beta*C + bias).
 *   - SiLU is x * sigmoid(x) = x / (1 + exp(-x)), evaluated with the hardware exponential and
 *     reciprocal (each within 1 ulp).
 *   - The scale vectors multiply the product before beta*C and bias are added, in the order
 *     ((alpha * scale_a * scale_b) * sum) * row_scale[m] * col_scale[n], in fp32.
 *
 * Supported type combinations (A and B share a type; C, D and bias share the output type):
 *     A/B      C/D/bias
 *     f32      f32
 *     f16      f16
 *     bf16     bf16
 *     e4m3     bf16
 */
#ifndef HTGEMM_H
#define HTGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, missing C with beta != 0, ...   */
  GEMM_ERR_DTYPE_COMBO = 2,  /* type combination not in the table above                       */
  GEMM_ERR_LAYOUT = 3,       /* an operand of A or B has no unit stride                         */
  GEMM_ERR_MISALIGNED = 4,   /* a pointer is not aligned to its element size                    */
  GEMM_ERR_ARCH = 5,         /* the current device is not gfx950                                 */
  GEMM_ERR_LAUNCH = 6,       /* the kernel launch failed (hipGetLastError)                       */
  GEMM_ERR_BAD_HANDLE = 7,   /* NULL or destroyed handle                                         */
  GEMM_ERR_NO_CONFIG = 8,    /* the forced tile-table entry cannot run this problem              */
  GEMM_ERR_HIP = 9,          /* another HIP runtime error (device query failed, ...)            */
  GEMM_ERR_LANE_MAP = 10,    /* a kernel's lane map disagrees with the layout helper (a defect  */
                             /* of the build, never of the arguments)                            */
  GEMM_ERR_SCRATCH_LIMIT = 11 /* gemm_run_noalloc: the handle needs more than                    */
                             /* GEMM_NOALLOC_SCRATCH_BYTES of workspace                          */
};

/* ---- element types and activations ----------------------------------------------------- */
typedef enum { GEMM_F32 = 0, GEMM_F16 = 1, GEMM_BF16 = 2, GEMM_F8E4M3 = 3 } gemm_dtype;
/* GEMM_ACT_GELU_ERF is the exact (erf) GELU; GEMM_ACT_GELU is the same value under a shorter
 * name. */
typedef enum {
  GEMM_ACT_NONE = 0,
  GEMM_ACT_RELU = 1,
  GEMM_ACT_GELU_ERF = 2,
  GEMM_ACT_GELU = GEMM_ACT_GELU_ERF,
  GEMM_ACT_SILU = 3
} gemm_act;

/* ---- problem descriptor ------------------------------------------------------------------ */
typedef struct gemm_desc {
  int64_t M, N, K;            /* problem shape; each >= 0                                       */
  int32_t a_type, b_type;     /* gemm_dtype of A and B                                           */
  int32_t c_type, d_type;     /* gemm_dtype of C (ignored if has_c == 0) and D                   */
  int32_t bias_type;          /* gemm_dtype of bias (ignored if has_bias == 0)                   */
  int32_t has_c;              /* 1: gemm_run reads C whenever beta != 0                          */
  int32_t has_bias;           /* 1: add bias[n] to every row                                     */
  int32_t act;                /* gemm_act, applied last                                          */
  int64_t a_stride_m, a_stride_k;   /* A(m, k) at A[m * a_stride_m + k * a_stride_k]            */
  int64_t b_stride_k, b_stride_n;   /* B(k, n) at B[k * b_stride_k + n * b_stride_n]            */
  int64_t c_stride_m, c_stride_n;   /* C(m, n); ignored if has_c == 0                            */
  int64_t d_stride_m, d_stride_n;   /* D(m, n)                                                    */
  int32_t force_config;       /* -1: choose from the tile table; else a table index (tuning)     */
  int32_t split_k;            /* split of K across workgroups per output tile: 0 = automatic,    */
                              /* 1 = never, 2..64 = that many slices (capped at one per k-tile); */
                              /* automatic also splits the tiles of a mostly idle last round     */
                              /* (the split tail, see gemm_workspace_size)                       */
  int32_t has_row_scale;      /* 1: gemm_run_ex multiplies row m of the product by row_scale[m]  */
  int32_t has_col_scale;      /* 1: gemm_run_ex multiplies column n by col_scale[n]              */
  int64_t batch;              /* problems of this shape per call, 0..65535 (0 and 1: one); with  */
                              /* batch > 1 split_k must be 0 or 1 and no split is made           */
  int64_t a_stride_l, b_stride_l;   /* elements from problem l's A (B) to problem l+1's; >= 0    */
  int64_t c_stride_l, d_stride_l;   /* the same for C and D; d_stride_l != 0 when batch > 1      */
  int32_t ragged_m;           /* 1: grouped GEMM with ragged M, run by gemm_run_grouped: the     */
                              /* `batch` >= 1 groups share A's, C's and D's M rows (row_scale),  */
                              /* split by device offsets; B of group e is at B + e*b_stride_l;   */
                              /* A must be K-major (row-major); a/c/d_stride_l are ignored       */
  int32_t has_row_sumsq;      /* 1: gemm_run_ex also writes row_sumsq[m] = sum over n of D(m,n)^2 */
                              /* of the stored (rounded) D; one problem, no split (see gemm_args) */
  int32_t has_col_sum;        /* 1: gemm_run_ex also writes col_sum[n] = sum over m of D(m,n) of  */
                              /* the stored D; the same conditions                               */
  int32_t grouped;            /* 1: grouped GEMM of independent problems, run by               */
                              /* gemm_run_problems: up to `batch` (>= 1) problems per call, each */
                              /* with its own M, N, K, pointers and leading dimensions; M, N, K  */
                              /* above describe a typical problem (the kernel is chosen for      */
                              /* `batch` problems of that shape) and the strides give each       */
                              /* operand's unit-stride direction; ragged_m, split_k > 1, scale   */
                              /* vectors and the reductions are refused                          */
  int32_t decomposition;      /* how output tiles are spread over the CUs: 0 = the library       */
                              /* decides, 1 = no Stream-K (a tile per workgroup, K slices as     */
                              /* split_k says), 2 = Stream-K, and no other split, wherever the   */
                              /* chosen kernel has a Stream-K form (gemm_info.sk_tiles > 0 then; */
                              /* with 2 the library chooses among the kernels that have one,     */
                              /* if any fits);                                                   */
                              /* 2 is refused with split_k > 1, a batch, a grouped handle or a   */
                              /* reduction                                                       */
} gemm_desc;

typedef struct gemm_handle_s* gemm_t;

/* Validate `desc` and pick a kernel.  On success *out is a new handle.  Host-only: allocates
 * no device memory and launches nothing.  The chosen kernels' MFMA lane maps and LDS swizzle
 * are checked once per process against the layout helper (htlayout.h).  Errors:
 * GEMM_ERR_INVALID_ARG, GEMM_ERR_DTYPE_COMBO, GEMM_ERR_LAYOUT, GEMM_ERR_ARCH, GEMM_ERR_NO_CONFIG,
 * GEMM_ERR_HIP, GEMM_ERR_LANE_MAP. */
int gemm_create(const gemm_desc* desc, gemm_t* out);

/* Bytes of device workspace gemm_run needs for this handle: 0 unless the problem is split along
 * K ("CUTLASS", Part III: split-K for outputs with too few tiles to fill the GPU), in which case
 * it is split_k * M * N * 4 (one fp32 plane of partial sums per slice).  A large product whose A
 * or B the 16-byte loaders cannot read (a leading dimension off 16 bytes, K not a multiple of
 * 16 bytes' worth of elements, or an fp8 operand that is not K-contiguous) runs on K-major,
 * aligned copies of both (gemm_info.repack): the workspace then starts with M * Kp and N * Kp
 * elements (each rounded up to 256 bytes), Kp being K rounded up to 16 bytes' worth, and
 * gemm_run writes them with one copy kernel per operand on the stream before the product.  A split tail (the
 * Stream-K idea, same Part: the tiles of a last round that would leave most CUs idle are each
 * split along K) needs tail_split * tail_tiles * bm * bn * 4 (gemm_info).  Stream-K (gemm_info.sk_tiles
 * > 0: the last tiles of the tile order shared out as equal runs of k-tiles among sk_wgs
 * persistent workgroups, "CUTLASS", Part IV Stage 2) needs 2 * sk_wgs * bm * bn * 4 for the
 * pieces of the tiles they share.  A grouped handle
 * (ragged_m) needs (G + 1) * 4 bytes rounded up to 256, plus (G + 1) * 8; a handle of independent
 * problems (grouped) needs 112 * batch bytes rounded up to 256, plus (batch + 1) * 8.  With has_row_sumsq it
 * is the number of N tiles * M * 4, and has_col_sum adds (M tiles * row groups) * N * 4.  The caller owns the
 * workspace; its contents after a run are unspecified, and two runs in flight at once need two
 * workspaces. */
int gemm_workspace_size(gemm_t h, size_t* bytes);

/* Enqueue D = act(alpha*scale_a*scale_b*(A@B) + beta*C + bias) on `stream` (a hipStream_t;
 * NULL is the default stream).  A, B, D are device pointers; C may be NULL when beta == 0 or the
 * handle was created with has_c == 0 (then beta must be 0); bias must be non-NULL iff the handle
 * has has_bias == 1.  For a batch (desc.batch > 1) A, B, C, D address problem 0 and the others
 * follow at the *_stride_l element offsets; the 16-byte kernels are used only when those
 * offsets keep every problem's A and B 16-byte aligned.  scale_a and scale_b are the per-tensor dequantisation scales (pass 1.0f for
 * non-fp8 operands).  Pointers only need element alignment: the library falls back to a
 * narrow-load kernel when a pointer is not 16-byte aligned.  `workspace` is a device buffer of
 * gemm_workspace_size() bytes, 16-byte aligned (GEMM_ERR_INVALID_ARG if it is needed and missing;
 * ignored when that size is 0).  A split run is two kernels on `stream`: the K slices, then their
 * fixed-order sum and the epilogue; a split-tail run is three: the whole tiles, the tail tiles'
 * K slices, then their fixed-order sum and epilogue; a Stream-K run is three: the whole tiles
 * before the Stream-K part, the persistent workgroups, then the sum of the shared tiles' pieces
 * in K order with the epilogue.  Returns after the launches are queued; launch failures
 * return GEMM_ERR_LAUNCH. */
int gemm_run(gemm_t h, const void* A, const void* B, const void* C, void* D, const void* bias,
             float alpha, float beta, float scale_a, float scale_b, void* workspace,
             void* stream);

/* Arguments of gemm_run_ex: the pointers and scalars of gemm_run plus the scale vectors and the
 * row reduction.  row_sumsq receives, for every row m, the sum over n of the squares of the
 * stored D(m, n) (the rounded outputs), accumulated in fp32 in a fixed order; it is the
 * reduction a following RMS normalisation needs ("CUTLASS", Part IV Stage 5: a fused reduction
 * for the next layer's normalisation).  col_sum receives, for every column n, the sum over m of
 * the stored D(m, n) (the reduction over rows, e.g. a bias gradient when D is an upstream
 * gradient).  Both are accumulated in fp32 in a fixed order, use the workspace
 * (gemm_workspace_size bytes of per-tile partials) and one more kernel each on the same stream.
 * row_scale (M floats) must be non-NULL iff the handle has has_row_scale == 1, col_scale (N
 * floats) iff has_col_scale == 1; both are device pointers aligned to 4 bytes and shared by every
 * problem of a batch, like bias.  For a batch, A, B, C and D point at problem 0 and the others
 * follow at the descriptor's *_stride_l element offsets. */
typedef struct gemm_args {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  const void* bias;
  const float* row_scale;
  const float* col_scale;
  float alpha, beta, scale_a, scale_b;
  void* workspace;
  float* row_sumsq;   /* M floats, non-NULL iff the handle has has_row_sumsq == 1 */
  float* col_sum;     /* N floats, non-NULL iff the handle has has_col_sum == 1 */
} gemm_args;

/* Enqueue the handle's operation with the arguments in `args` on `stream`; the same checks and
 * errors as gemm_run, plus GEMM_ERR_INVALID_ARG when a scale vector's presence does not match the
 * handle and GEMM_ERR_MISALIGNED when one is not 4-byte aligned.  gemm_run itself returns
 * GEMM_ERR_INVALID_ARG for a handle with scale vectors. */
int gemm_run_ex(gemm_t h, const gemm_args* args, void* stream);

/* Grouped GEMM with ragged M, the mixture-of-experts case ("CUTLASS", Part V: a grouped GEMM in
 * which each expert is one problem of a batch of differently shaped problems).  For a handle
 * created with ragged_m == 1 and batch == G groups: group e computes rows
 * [offsets[e], offsets[e+1]) of D from the same rows of A (and C, row_scale) and its own
 * B_e = B + e * b_stride_l, with shared N, K, bias, col_scale, alpha and beta.  `offsets` is a
 * device array of G + 1 int32 values, 4-byte aligned, non-decreasing from 0 to M; it is read
 * on the device, so routing decided on the GPU needs no host round trip.  Out-of-range or
 * decreasing offsets are clamped into [0, M] and made non-decreasing (offset e becomes
 * min(M, max(0, offsets[0..e]))), so they cannot send the kernel outside the operands, but the
 * rows they drop are not written.  args->workspace must hold gemm_workspace_size bytes: a first
 * kernel on `stream` writes there each group's clamped rows and first tile (a prefix over the
 * groups), and each workgroup of the product finds its group by binary search.  The other
 * pointers and scalars are those of gemm_run_ex.  gemm_run and gemm_run_ex refuse a ragged
 * handle, and this entry point refuses any other (GEMM_ERR_INVALID_ARG). */
int gemm_run_grouped(gemm_t h, const gemm_args* args, const int32_t* offsets, void* stream);

/* One problem of a grouped call (gemm_run_problems).  Shapes and pointers as in gemm_run; each
 * leading dimension replaces the descriptor's stride along that operand's other direction
 * (lda: a_stride_m for a K-major A, a_stride_k for an M-major one; ldb likewise; ldc and ldd:
 * the row stride of a row-major C or D (descriptor stride along n == 1), else the column
 * stride).  C is read only when beta != 0; bias (N values) only when the handle has has_bias. */
typedef struct gemm_problem {
  int64_t M, N, K;
  const void* A;
  const void* B;
  const void* C;
  void* D;
  const void* bias;
  int64_t lda, ldb, ldc, ldd;
} gemm_problem;

/* Grouped GEMM of independent problems ("CUTLASS", Part III: a grouped GEMM runs many problems
 * of irregular shapes in one launch; "CUTLASS, CuTe, and CUDA Tile", "Assembling a CUTLASS
 * kernel": the problem shape [M, N, K, L] with a problem per L index).  For a handle created
 * with grouped == 1: problem i computes D_i = act(alpha*scale_a*scale_b*(A_i @ B_i) + beta*C_i
 * + bias_i) for i < count (0 <= count <= the handle's batch), all with the handle's types,
 * layouts and epilogue and the scalars of `args` (whose A, B, C, D, bias, scale-vector and
 * reduction pointers must be NULL).  `problems` is a host array read during the call: it is
 * checked, the tile count of every problem is taken, and a table of the problems and of their
 * first tiles is copied into args->workspace (gemm_workspace_size bytes, 16-byte aligned) with
 * hipMemcpyAsync on `stream` -- from pageable memory that copy completes before the call returns
 * -- and one launch then runs the tiles of every problem, each workgroup finding its problem by
 * binary search.  The 16-byte kernel runs when every problem's A and B meet its alignment,
 * otherwise the narrow-load kernel runs them all.  Errors: those of gemm_run for any problem
 * (the call launches nothing then), GEMM_ERR_INVALID_ARG for a handle that is not grouped or a
 * count above its batch, GEMM_ERR_NO_CONFIG when a problem's operands exceed the chosen
 * kernels' 31-bit tile offsets. */
int gemm_run_problems(gemm_t h, const gemm_problem* problems, int64_t count, const gemm_args* args,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): gemm_run_ex with the workspace taken from a static
 * device array of GEMM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends.  args->workspace must be NULL.  It allocates nothing and calls no allocating
 * routine; the first call on a device looks up that device's copy of the array.  Returns
 * GEMM_ERR_SCRATCH_LIMIT when gemm_workspace_size(h) exceeds GEMM_NOALLOC_SCRATCH_BYTES (create
 * the handle with split_k = 1 to need none), GEMM_ERR_INVALID_ARG for a grouped handle or a
 * non-NULL workspace, otherwise the results and errors of gemm_run_ex.  All calls on one GPU share
 * its array, which keeps the last call's contents (every byte a run reads there it has written
 * first), so calls that overlap in time on one GPU -- on different streams or threads -- race
 * and give undefined results; calls ordered on one stream do not. */
#define GEMM_NOALLOC_SCRATCH_BYTES (32u << 20)
int gemm_run_noalloc(gemm_t h, const gemm_args* args, void* stream);

/* Free a handle.  NULL is accepted. */
int gemm_destroy(gemm_t h);

/* Static text for a status code. */
const char* gemm_status_string(int status);

/* ---- introspection (tile table) --------------------------------------------------------- */
typedef struct gemm_info {
  int32_t config;         /* tile-table index chosen for 16-byte aligned pointers             */
  int32_t fallback;       /* index used when a pointer is not 16-byte aligned (may equal it)   */
  int32_t bm, bn, bk;     /* workgroup tile                                                     */
  int32_t waves;          /* waves per workgroup                                                */
  int32_t stages;         /* LDS pipeline stages                                                */
  int32_t lds_bytes;      /* LDS bytes per workgroup                                            */
  int32_t split_k;        /* workgroups sharing one output tile along K (1: none)              */
  int64_t grid;           /* workgroups per launch (all problems of a batch)                    */
  char name[96];          /* kernel name                                                        */
  int32_t tail_tiles;     /* tiles of an incomplete last round run split along K (0: none)      */
  int32_t tail_split;     /* K slices of each such tile (1: none)                               */
  int32_t repack;         /* 1: A and B are read through aligned K-major copies in the workspace */
  int32_t sk_tiles;       /* tiles run Stream-K (the last ones of the tile order; 0: none)      */
  int32_t sk_wgs;         /* persistent workgroups of the Stream-K launch                       */
  double predicted_us;    /* the cost model's time of one run, in microseconds (0: the entry has
                             no measured costs); the choice took the least of these             */
} gemm_info;

int gemm_get_info(gemm_t h, gemm_info* info);

/* Clock record, for measurement ("CuTe DSL / CUDA Tile" post, "Build the benchmark before tuning
 * the tile": record the conditions a number was measured under).  After this call, every launch
 * of the handle's product kernel has each workgroup w < max_workgroups (its linear id over the
 * launch's x, y and z) write four 64-bit values to records[4w .. 4w + 3]: the shader-clock
 * counter (s_memtime) at the workgroup's start and at its end, then the constant-rate real-time
 * counter (s_memrealtime; 100 MHz on MI355X) at its start and at its end, so that
 * (records[4w+1] - records[4w]) / (records[4w+3] - records[4w+2]) x 100 MHz is the mean shader
 * clock the workgroup ran at.  records is a device buffer of 4 * max_workgroups uint64_t, owned
 * by the caller, 8-byte aligned; later launches overwrite it; records == NULL turns recording
 * off.  Only the ping-pong kernel (entries whose name ends in "_pp") records; other kernels, the
 * copy, sum and fix-up kernels leave the buffer untouched.  The cost is four scalar timer reads
 * and one store per workgroup.  Not thread-safe against concurrent runs of the same handle.
 * Returns GEMM_ERR_BAD_HANDLE, or GEMM_ERR_INVALID_ARG for a negative count or a misaligned
 * buffer. */
int gemm_set_clock_record(gemm_t h, uint64_t* records, int64_t max_workgroups);

/* Number of entries in the compiled tile table, and the name of entry `idx`. */
int gemm_num_configs(void);
int gemm_config_name(int idx, char* out, size_t cap);

/* ---- MFMA lane maps ("A10 - CuTe, CUTLASS & CuTile", section 3.3: an MMA atom's fragments are
 * layouts from (thread, value) to the instruction's tile; section 6 Pitfall 2) ------------------ */
/* The layouts the kernels use for the atom of operand type `dtype` (gemm_dtype) with an MI x MI
 * output block (MI = 16 or 32), in the pages' shape:stride notation, written to `op` and `acc`
 * (caller buffers of `cap` bytes).  Index i = lane + 64 * v (lane fastest).  op maps to
 * m + MI * k of A (and n + MI * k of B, which uses the same map); acc maps to m + MI * n.
 * Returns GEMM_OK, GEMM_ERR_INVALID_ARG (no such atom, NULL, or cap too small) or
 * GEMM_ERR_LANE_MAP (the layouts disagree with the layout helper). */
int gemm_atom_layouts(int dtype, int mi, char* op, char* acc, size_t cap);

/* Index probe: runs the atom (dtype, mi) on the current device, on `stream`, and writes into
 * the caller's device buffer `out` (GEMM_PROBE_INTS int32 values, four sections of 2048):
 *   [0, 2048)     for each accumulator slot i = lane + 64 r: m + MI * n of the output element the
 *                 hardware placed there, with the operands fed through the kernels' LDS tiles,
 *                 swizzle and fragment addressing from inputs that encode m and n in D;
 *   [2048, 4096)  the kernels' belief for the same slot: acc_row + MI * acc_col;
 *   [4096, 6144)  for each operand slot i = lane + 64 v: the row of D that a one-hot A in that
 *                 slot (B all ones) makes non-zero, the hardware's m of the slot;
 *   [6144, 8192)  for the same slot: the number of columns n for which D(m, n) is 1 when B holds
 *                 ones exactly in the slots the op layout gives the same k (MI if those slots
 *                 meet A's slot in the hardware's k, fewer otherwise), or -1 if D is non-zero off
 *                 row m.
 * Unused entries are -2.  Asynchronous; GEMM_ERR_INVALID_ARG for an unknown atom or NULL out,
 * GEMM_ERR_LAUNCH if the launch fails. */
#define GEMM_PROBE_INTS 8192
int gemm_probe_atom(int dtype, int mi, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HTGEMM_H */
