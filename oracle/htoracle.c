/*
 * htoracle.c -- CPU oracle for the tiled dense GEMM  D = act(alpha*sA*sB*(A@B) + beta*C + bias).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant with the GPU
 * library, and it includes nothing from it.
 *
 * What it computes (sources are the reference pages, cited by page title and section):
 *  - The problem is D = alpha * (A @ B) + beta * C with A MxK, B KxN, D MxN
 *    ("CUTLASS", stanleyjacob.dev, Part I "The mental model"; Part II "Using it": the default
 *    LinearCombination epilogue computes alpha*accumulator + beta*C and casts to the output type).
 *  - Tiling only changes the order of the additions, so the oracle is the plain definition:
 *    for every (i, j), s = sum over k of A(i,k)*B(k,j) in IEEE double, k ascending.
 *  - The epilogue order is alpha/beta, then bias, then activation ("CUTLASS", Part I diagram and
 *    Part IV Stage 5 "The epilogue and fusion"); the bias is one value per output column n.
 *  - A narrow-type GEMM folds a per-tensor dequantisation scale into the epilogue ("CUTLASS",
 *    Part V "Data types and quantization"): y = alpha * sA * sB * s.
 *  - A fused epilogue may also scale by a per-channel (per output column) dequantisation vector
 *    and apply other activations ("CUTLASS", Part IV Stage 5 "The epilogue and fusion": the
 *    epilogue visitor tree fuses bias, activation and a per-channel scale; "A10 - CuTe, CUTLASS &
 *    CuTile", drill answer 8: bias plus a nonstandard activation plus a quantisation scale in one
 *    kernel).  Here y = alpha * sA * sB * row_scale[i] * col_scale[j] * s before C and bias; the
 *    per-row vector is the same broadcast along the other mode (per-token activation scales).
 *  - Inputs are compared on the same rounded inputs ("A10 - CuTe, CUTLASS & CuTile", section 6
 *    Pitfall 5 and drill answer 7): every element is decoded exactly from its stored bits to
 *    double by this file's own codecs; the result is left in double, unrounded.
 *
 * Readings where the pages are silent:
 *  - beta == 0 means C is not read at all (it may be NULL and NaNs in it do not propagate).
 *  - GELU is the exact erf form 0.5*x*(1+erf(x/sqrt(2))), computed with the C library's erf.
 *  - SiLU is x * sigmoid(x) = x / (1 + exp(-x)), computed with the C library's exp.
 *  - e4m3 is the OCP "fn" flavour: bias 7, no infinities, S.1111.111 is NaN, max 448
 *    (the FP8 formats paper listed in "CUTLASS", Part XI).
 *
 * Element (i, k) of an operand with strides (s0, s1) sits at element offset i*s0 + k*s1.
 * Threads split the rows (or the sampled elements); each dot product stays one sequential loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_E4M3 = 3 };
enum { OR_ACT_NONE = 0, OR_ACT_RELU = 1, OR_ACT_GELU = 2, OR_ACT_SILU = 3 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENOMEM = 2 };

/* ------------------------------------------------------------------------------------------ */
/* Codecs: exact decode of stored bits to double, and round-to-nearest-even encode.             */
/* ------------------------------------------------------------------------------------------ */

/* IEEE binary32: reinterpret the 32 bits. */
static double dec_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Generic sign/exponent/mantissa decode: value = (-1)^s * 2^(e - bias) * (1 + m/2^mbits) for
 * normal numbers, (-1)^s * 2^(1 - bias) * (m/2^mbits) for e == 0. */
static double dec_generic(uint32_t s, uint32_t e, uint32_t m, int mbits, int bias) {
  double mag;
  if (e == 0)
    mag = ldexp((double)m, 1 - bias - mbits);
  else
    mag = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  return s ? -mag : mag;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa; e == 31 is inf/NaN. */
static double dec_f16(uint16_t h) {
  uint32_t s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
  return dec_generic(s, e, m, 10, 15);
}

/* bfloat16: the upper half of a binary32. 1 sign, 8 exponent (bias 127), 7 mantissa. */
static double dec_bf16(uint16_t b) {
  uint32_t s = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
  if (e == 255) return m ? NAN : (s ? -INFINITY : INFINITY);
  return dec_generic(s, e, m, 7, 127);
}

/* OCP E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa; no infinities; S.1111.111 is NaN. */
static double dec_e4m3(uint8_t q) {
  uint32_t s = q >> 7, e = (q >> 3) & 0xf, m = q & 0x7;
  if (e == 15 && m == 7) return NAN;
  return dec_generic(s, e, m, 3, 7);
}

static int elem_size(int t) {
  switch (t) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_E4M3: return 1;
    default: return 0;
  }
}

static double dec_at(int t, const void* base, int64_t idx) {
  switch (t) {
    case OR_F32: return dec_f32(((const uint32_t*)base)[idx]);
    case OR_F16: return dec_f16(((const uint16_t*)base)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case OR_E4M3: return dec_e4m3(((const uint8_t*)base)[idx]);
    default: return NAN;
  }
}

/* Round a finite double to a binary format with `mbits` stored mantissa bits, exponent bias
 * `bias`, and largest biased exponent `emax_biased` for finite numbers, to nearest, ties to
 * even.  Returns the magnitude bits (exponent|mantissa) and sets *overflow when the rounded
 * magnitude is beyond the largest finite value. */
static uint32_t rne_bits(double a, int mbits, int bias, int emax_biased, int* overflow) {
  *overflow = 0;
  if (a == 0.0) return 0;
  int ex;
  frexp(a, &ex); /* a = f * 2^ex, 0.5 <= f < 1, so the leading bit has weight 2^(ex-1) */
  int unbiased = ex - 1;
  int emin = 1 - bias; /* smallest normal exponent */
  int q = (unbiased < emin ? emin : unbiased) - mbits; /* weight of the last kept bit */
  double scaled = ldexp(a, -q); /* exact: a power-of-two scaling */
  double fl = floor(scaled);
  double rem = scaled - fl; /* exact */
  uint64_t n = (uint64_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (n & 1))) n += 1;
  /* n * 2^q is the rounded magnitude. Re-normalise. */
  if (n == 0) return 0;
  int e_biased;
  uint64_t mant;
  if (n < (1ull << mbits)) { /* subnormal result (only possible when q == emin - mbits) */
    e_biased = 0;
    mant = n;
  } else {
    int shift = 0;
    while ((n >> shift) >= (2ull << mbits)) shift++; /* n may be 2^(mbits+1) after carry */
    /* after a carry n == 2^(mbits+1) exactly, so the shift loses no bits */
    n >>= shift;
    e_biased = (q + shift + mbits) + bias;
    mant = n & ((1ull << mbits) - 1);
  }
  if (e_biased > emax_biased) *overflow = 1;
  return ((uint32_t)e_biased << mbits) | (uint32_t)mant;
}

static uint16_t enc_f16(double x) {
  uint16_t s = (signbit(x) ? 0x8000 : 0);
  if (isnan(x)) return 0x7e00;
  if (isinf(x)) return s | 0x7c00;
  int of;
  uint32_t b = rne_bits(fabs(x), 10, 15, 30, &of);
  if (of) return s | 0x7c00; /* IEEE overflow under round-to-nearest goes to infinity */
  return s | (uint16_t)b;
}

static uint16_t enc_bf16(double x) {
  uint16_t s = (signbit(x) ? 0x8000 : 0);
  if (isnan(x)) return 0x7fc0;
  if (isinf(x)) return s | 0x7f80;
  int of;
  uint32_t b = rne_bits(fabs(x), 7, 127, 254, &of);
  if (of) return s | 0x7f80;
  return s | (uint16_t)b;
}

static uint32_t enc_f32(double x) {
  float f = (float)x; /* the C conversion rounds to nearest even under the default mode */
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* e4m3 "fn" with saturation to +-448: values beyond the largest finite magnitude clamp
 * (the convention used to quantise inputs); NaN maps to 0x7f. */
static uint8_t enc_e4m3(double x) {
  uint8_t s = (signbit(x) ? 0x80 : 0);
  if (isnan(x)) return 0x7f;
  if (isinf(x)) return s | 0x7e;
  int of;
  uint32_t b = rne_bits(fabs(x), 3, 7, 15, &of);
  if (of || b > 0x7e) return s | 0x7e; /* 0x7f would be NaN: clamp to 448 */
  return s | (uint8_t)b;
}

int oracle_decode(int dtype, const void* src, int64_t n, double* dst) {
  if (!elem_size(dtype) || (n > 0 && (!src || !dst)) || n < 0) return OR_EINVAL;
  for (int64_t i = 0; i < n; i++) dst[i] = dec_at(dtype, src, i);
  return OR_OK;
}

int oracle_encode_rne(int dtype, const double* src, int64_t n, void* dst) {
  if (!elem_size(dtype) || (n > 0 && (!src || !dst)) || n < 0) return OR_EINVAL;
  for (int64_t i = 0; i < n; i++) {
    switch (dtype) {
      case OR_F32: ((uint32_t*)dst)[i] = enc_f32(src[i]); break;
      case OR_F16: ((uint16_t*)dst)[i] = enc_f16(src[i]); break;
      case OR_BF16: ((uint16_t*)dst)[i] = enc_bf16(src[i]); break;
      case OR_E4M3: ((uint8_t*)dst)[i] = enc_e4m3(src[i]); break;
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* The GEMM.                                                                                     */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int64_t M, N, K;
  int a_type, b_type, c_type, bias_type;
  const void *A, *B, *C, *bias;
  const float *row_scale, *col_scale; /* NULL: not applied */
  int64_t a_sm, a_sk, b_sk, b_sn, c_sm, c_sn;
  double alpha, beta, scale_a, scale_b;
  int act;
} problem;

static double activation(int act, double y) {
  switch (act) {
    case OR_ACT_RELU: return y > 0.0 ? y : (y == y ? 0.0 : y); /* max(0, y); NaN stays NaN */
    case OR_ACT_GELU: return 0.5 * y * (1.0 + erf(y / sqrt(2.0)));
    case OR_ACT_SILU: return y / (1.0 + exp(-y));
    default: return y;
  }
}

/* One output element from the definition; arow[k] = A(i,k), bcol[k] = B(k,j) already decoded. */
static double finish(const problem* p, int64_t i, int64_t j, double s) {
  double y = p->alpha * p->scale_a * p->scale_b * s;
  if (p->row_scale) y *= (double)p->row_scale[i];
  if (p->col_scale) y *= (double)p->col_scale[j];
  if (p->beta != 0.0) y += p->beta * dec_at(p->c_type, p->C, i * p->c_sm + j * p->c_sn);
  if (p->bias) y += dec_at(p->bias_type, p->bias, j);
  return activation(p->act, y);
}

static double dot(const double* a, const double* b, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; k++) s += a[k] * b[k];
  return s;
}

/* Full GEMM: every operand is decoded once into dense double arrays (Ad[i][k], Bt[j][k]) so the
 * dot product of the definition runs over contiguous memory; the sum order is still k = 0..K-1. */
typedef struct {
  const problem* p;
  const double *Ad, *Bt;
  double* out;
  int64_t o_sm, o_sn;
  int64_t row0, row1;
} full_job;

static void* full_worker(void* arg) {
  full_job* j = (full_job*)arg;
  const problem* p = j->p;
  for (int64_t i = j->row0; i < j->row1; i++)
    for (int64_t c = 0; c < p->N; c++) {
      double s = dot(j->Ad + i * p->K, j->Bt + c * p->K, p->K);
      j->out[i * j->o_sm + c * j->o_sn] = finish(p, i, c, s);
    }
  return NULL;
}

typedef struct {
  const problem* p;
  const double *Ad, *Bt;
  int64_t lo, hi;
  int which; /* 0: decode A rows, 1: decode B columns */
} dec_job;

static void* dec_worker(void* arg) {
  dec_job* j = (dec_job*)arg;
  const problem* p = j->p;
  for (int64_t r = j->lo; r < j->hi; r++)
    for (int64_t k = 0; k < p->K; k++) {
      if (j->which == 0)
        ((double*)j->Ad)[r * p->K + k] = dec_at(p->a_type, p->A, r * p->a_sm + k * p->a_sk);
      else
        ((double*)j->Bt)[r * p->K + k] = dec_at(p->b_type, p->B, k * p->b_sk + r * p->b_sn);
    }
  return NULL;
}

static int check_problem(const problem* p) {
  if (p->M < 0 || p->N < 0 || p->K < 0) return OR_EINVAL;
  if (!elem_size(p->a_type) || !elem_size(p->b_type)) return OR_EINVAL;
  if ((p->M > 0 && p->K > 0 && !p->A) || (p->N > 0 && p->K > 0 && !p->B)) return OR_EINVAL;
  if (p->beta != 0.0 && (!p->C || !elem_size(p->c_type))) return OR_EINVAL;
  if (p->bias && !elem_size(p->bias_type)) return OR_EINVAL;
  if (p->act < OR_ACT_NONE || p->act > OR_ACT_SILU) return OR_EINVAL;
  return OR_OK;
}

static int run_threads(void* (*fn)(void*), void* jobs, size_t job_size, int n) {
  pthread_t* th = (pthread_t*)calloc((size_t)n, sizeof(pthread_t));
  if (!th) return OR_ENOMEM;
  int started = 0;
  for (int t = 0; t < n; t++) {
    if (pthread_create(&th[t], NULL, fn, (char*)jobs + (size_t)t * job_size) == 0)
      started++;
    else
      fn((char*)jobs + (size_t)t * job_size), th[t] = 0;
  }
  for (int t = 0; t < n; t++)
    if (th[t]) pthread_join(th[t], NULL);
  free(th);
  (void)started;
  return OR_OK;
}

int oracle_gemm(int64_t M, int64_t N, int64_t K, int a_type, const void* A, int64_t a_sm,
                int64_t a_sk, int b_type, const void* B, int64_t b_sk, int64_t b_sn, int c_type,
                const void* C, int64_t c_sm, int64_t c_sn, int bias_type, const void* bias,
                const float* row_scale, const float* col_scale,
                double alpha, double beta, double scale_a, double scale_b, int act, double* out,
                int64_t o_sm, int64_t o_sn, int nthreads) {
  problem p = {M, N, K, a_type, b_type, c_type, bias_type, A, B, C, bias, row_scale, col_scale,
               a_sm, a_sk, b_sk, b_sn, c_sm, c_sn, alpha, beta, scale_a, scale_b, act};
  int rc = check_problem(&p);
  if (rc) return rc;
  if (M == 0 || N == 0) return OR_OK;
  if (!out) return OR_EINVAL;
  if (nthreads < 1) nthreads = 1;
  double* Ad = (double*)malloc((size_t)(M * (K ? K : 1)) * sizeof(double));
  double* Bt = (double*)malloc((size_t)(N * (K ? K : 1)) * sizeof(double));
  if (!Ad || !Bt) {
    free(Ad);
    free(Bt);
    return OR_ENOMEM;
  }
  int nt = nthreads;
  dec_job* dj = (dec_job*)calloc((size_t)nt, sizeof(dec_job));
  full_job* fj = (full_job*)calloc((size_t)nt, sizeof(full_job));
  if (!dj || !fj) {
    free(Ad); free(Bt); free(dj); free(fj);
    return OR_ENOMEM;
  }
  for (int which = 0; which < 2; which++) {
    int64_t rows = which ? N : M;
    for (int t = 0; t < nt; t++) {
      dj[t].p = &p; dj[t].Ad = Ad; dj[t].Bt = Bt; dj[t].which = which;
      dj[t].lo = rows * t / nt; dj[t].hi = rows * (t + 1) / nt;
    }
    run_threads(dec_worker, dj, sizeof(dec_job), nt);
  }
  for (int t = 0; t < nt; t++) {
    fj[t].p = &p; fj[t].Ad = Ad; fj[t].Bt = Bt; fj[t].out = out;
    fj[t].o_sm = o_sm; fj[t].o_sn = o_sn;
    fj[t].row0 = M * t / nt; fj[t].row1 = M * (t + 1) / nt;
  }
  run_threads(full_worker, fj, sizeof(full_job), nt);
  free(Ad); free(Bt); free(dj); free(fj);
  return OR_OK;
}

/* Selected elements only: out[e] = D(rows[e], cols[e]).  Used where the whole product would take
 * too long on the host; each element is the same definition. */
typedef struct {
  const problem* p;
  const int64_t *rows, *cols;
  double* out;
  int64_t lo, hi;
} elem_job;

static void* elem_worker(void* arg) {
  elem_job* j = (elem_job*)arg;
  const problem* p = j->p;
  int64_t K = p->K;
  double* a = (double*)malloc((size_t)(K ? K : 1) * sizeof(double));
  double* b = (double*)malloc((size_t)(K ? K : 1) * sizeof(double));
  if (!a || !b) {
    free(a); free(b);
    for (int64_t e = j->lo; e < j->hi; e++) j->out[e] = NAN;
    return NULL;
  }
  for (int64_t e = j->lo; e < j->hi; e++) {
    int64_t i = j->rows[e], c = j->cols[e];
    for (int64_t k = 0; k < K; k++) {
      a[k] = dec_at(p->a_type, p->A, i * p->a_sm + k * p->a_sk);
      b[k] = dec_at(p->b_type, p->B, k * p->b_sk + c * p->b_sn);
    }
    j->out[e] = finish(p, i, c, dot(a, b, K));
  }
  free(a); free(b);
  return NULL;
}

int oracle_gemm_elems(int64_t M, int64_t N, int64_t K, int a_type, const void* A, int64_t a_sm,
                      int64_t a_sk, int b_type, const void* B, int64_t b_sk, int64_t b_sn,
                      int c_type, const void* C, int64_t c_sm, int64_t c_sn, int bias_type,
                      const void* bias, const float* row_scale, const float* col_scale,
                      double alpha, double beta, double scale_a, double scale_b,
                      int act, int64_t count, const int64_t* rows, const int64_t* cols,
                      double* out, int nthreads) {
  problem p = {M, N, K, a_type, b_type, c_type, bias_type, A, B, C, bias, row_scale, col_scale,
               a_sm, a_sk, b_sk, b_sn, c_sm, c_sn, alpha, beta, scale_a, scale_b, act};
  int rc = check_problem(&p);
  if (rc) return rc;
  if (count < 0 || (count > 0 && (!rows || !cols || !out))) return OR_EINVAL;
  for (int64_t e = 0; e < count; e++)
    if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return OR_EINVAL;
  if (count == 0) return OR_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > count) nthreads = (int)count;
  elem_job* ej = (elem_job*)calloc((size_t)nthreads, sizeof(elem_job));
  if (!ej) return OR_ENOMEM;
  for (int t = 0; t < nthreads; t++) {
    ej[t].p = &p; ej[t].rows = rows; ej[t].cols = cols; ej[t].out = out;
    ej[t].lo = count * t / nthreads; ej[t].hi = count * (t + 1) / nthreads;
  }
  run_threads(elem_worker, ej, sizeof(elem_job), nthreads);
  free(ej);
  return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Reductions of the stored output for the next layer ("CUTLASS", stanleyjacob.dev, Part IV      */
/* Stage 5 "The epilogue and fusion": an epilogue visitor tree can fuse a reduction that a       */
/* following normalisation needs).  The pages name the reduction without fixing it; the reading  */
/* taken here is the plain definition over what a caller would read back from D:                */
/*   row_sumsq[i] = sum over j of  r(D[i][j])^2,   col_sum[j] = sum over i of  r(D[i][j]),       */
/* with r() the round-to-nearest-even of the double result to the output type (the stored value) */
/* and both sums in double, in index order.                                                      */
/* ------------------------------------------------------------------------------------------ */

static double round_to(int t, double x) {
  switch (t) {
    case OR_F32: return dec_f32(enc_f32(x));
    case OR_F16: return dec_f16(enc_f16(x));
    case OR_BF16: return dec_bf16(enc_bf16(x));
    case OR_E4M3: return dec_e4m3(enc_e4m3(x));
    default: return NAN;
  }
}

/* D is M x N with element (i, j) at D[i * ld + j]. */
int oracle_row_sumsq(int out_type, const double* D, int64_t M, int64_t N, int64_t ld, double* out) {
  if (!elem_size(out_type) || M < 0 || N < 0 || ld < N || (M > 0 && (!D || !out))) return OR_EINVAL;
  for (int64_t i = 0; i < M; i++) {
    double s = 0.0;
    for (int64_t j = 0; j < N; j++) {
      double v = round_to(out_type, D[i * ld + j]);
      s += v * v;
    }
    out[i] = s;
  }
  return OR_OK;
}

int oracle_col_sum(int out_type, const double* D, int64_t M, int64_t N, int64_t ld, double* out) {
  if (!elem_size(out_type) || M < 0 || N < 0 || ld < N || (N > 0 && (!D || !out))) return OR_EINVAL;
  for (int64_t j = 0; j < N; j++) {
    double s = 0.0;
    for (int64_t i = 0; i < M; i++) s += round_to(out_type, D[i * ld + j]);
    out[j] = s;
  }
  return OR_OK;
}
