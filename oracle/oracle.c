/*
 * oracle.c -- plain, slow CPU oracle for the factored dictionary projection.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The HIP library never
 * calls it, and the two share no source, header, table or helper.
 *
 * Pages followed (cited by title and section):
 *   [Review]    "DictLLM: Shared Dictionaries for Post-Training Compression"
 *               (technical review of the DictLLM paper).
 *   [Explainer] "DictLLM compresses LLaMA-7B 5.1x -- Shared dictionary plus
 *               sparse coefficients -- What does it mean?"
 *   [Tables]    "DictLLM: Post-training Compression of Large Language Model
 *               with Dictionary Kernels" (figures and tables page).
 *
 * What it computes:
 *   forward    Y = (X D) C evaluated in float64 exactly as written in
 *              [Review] "Prerequisites: projections, rank and calibration",
 *              Eq. (1): Z = X D (sum over d_in, ascending), then
 *              Y[t,j] = sum over the stored entries of column j, ascending.
 *   pack_csc   Column-compressed export of a dense coefficient matrix that
 *              keeps the support and drops zeros ([Review] Algorithm 2, the
 *              export of dictionary, codes, scales and support).
 *   nvfp4      4-bit E2M1 values with one 8-bit (E4M3) scale per block of
 *              sixteen consecutive values ([Review] "From retained values to
 *              measured decoding"; [Tables] Table 4) plus one fp32 tensor
 *              scale.  The scale recipe below is a reading, not printed on
 *              the pages (parity unpinned against the pages; pinned against
 *              format definitions, brute force and error bounds).
 *   codes8     8-bit coefficient values, FP8 (E4M3) or INT8, for the mixed
 *              precision rows of [Tables] Table 4 (NVFP4 dictionary with FP8
 *              or INT8 coefficients; also [Review] "From retained values to
 *              measured decoding", mixed precision).  The pages do not say
 *              how those codes are scaled; the reading taken here is one
 *              fp32 scale per column of C, symmetric, amax / 448 (E4M3) or
 *              amax / 127 (INT8), nearest code with ties to even.
 *   bcsc       Block-structured support, the variant the Review asks for
 *              ("Let the accelerator constrain the support"; [Explainer]:
 *              block-structured sparsity named as future work): each column
 *              keeps whole blocks of 8 consecutive atoms; a block is kept
 *              iff one of its entries is nonzero, and stores its block index
 *              and all 8 values (zeros included).
 *   producer   The steps that produce D and C ([Review] "Method II: prune in
 *              coefficient space" and "Method III: refit the dictionary"):
 *              the inverse P = (D^T S D + lambda I)^-1 of Eq. (6)-(7), the
 *              fixed-inverse pruning of each coefficient column (the
 *              Review's Algorithm 1), with the compensation and saliency of
 *              Eq. (7), and the refit D (C C^T + lambda I) = W C^T of
 *              Eq. (9).  Symmetric positive definite systems are solved by
 *              Cholesky factorisation, written out below.
 *
 * Every floating-point step that decides an integer code is done in fp32,
 * each operation correctly rounded (compile with -ffp-contract=off, no
 * -ffast-math).  Everything else is float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_NVFP4 2
#define ORC_FP8 3
#define ORC_INT8 4

/* A read-only view of a stored tensor (flat element index). */
typedef struct {
  int32_t dtype;        /* ORC_F32, ORC_F16, ORC_NVFP4, ORC_FP8 or ORC_INT8 */
  const void* data;     /* f32 / f16 elements; FP8 / INT8: one code byte each */
  const uint8_t* codes; /* NVFP4: two 4-bit codes per byte, element 2i low */
  const uint8_t* scales;/* NVFP4: one E4M3 code per 16 elements */
  float ts;             /* NVFP4: fp32 tensor scale */
  const float* col_scale; /* FP8 / INT8 coefficients: fp32 scale per column */
} orc_tensor;

/* IEEE 754 binary16, decoded from its definition: sign, 5-bit exponent with
 * bias 15, 10-bit fraction; exponent 0 is subnormal. */
double orc_half_value(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + m, e - 25);
  return s ? -v : v;
}

/* E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa, no inf/NaN.
 * Exponent 0 is subnormal (0 or 0.5). */
double orc_e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 ("fn" variant): sign, 4-bit exponent (bias 7), 3-bit mantissa; no
 * infinities; exponent 15 with mantissa 7 is NaN; exponent 0 subnormal. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(8.0 + m, e - 10);
  return s ? -mag : mag;
}

/* Nearest non-negative finite E4M3 code to s >= 0 (values beyond 448 take
 * 448), ties to the even code.  Brute force over the 127 candidates; every
 * difference is exact in float64 for fp32 s in the range that can tie. */
int orc_e4m3_nearest(float s) {
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs((double)s - orc_e4m3_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Nearest E2M1 magnitude code (0..7) to |v|, ties to the even code,
 * values beyond 6 take 6.  Brute force over the 8 candidates. */
int orc_e2m1_nearest(float v) {
  double a = fabs((double)v);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 7; ++c) {
    double d = fabs(a - orc_e2m1_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Tensor scale rule: amax / (6 * 448), so that the largest block scale is
 * the largest finite E4M3 value; 1 when that quotient is 0. */
float orc_nvfp4_tensor_scale(float amax) {
  float ts = amax / 2688.0f;
  return ts == 0.0f ? 1.0f : ts;
}

/* Quantise x[0..n) to NVFP4.  Returns 0, or -1 (nothing written) if x holds
 * a NaN or an infinity.  codes[(n+1)/2], scales[(n+15)/16]. */
int orc_nvfp4_pack(const float* x, int64_t n, uint8_t* codes, uint8_t* scales,
                   float* ts_out) {
  if (n < 0) return -1;
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(x[i])) return -1;
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float ts = orc_nvfp4_tensor_scale(amax);
  memset(codes, 0, (size_t)((n + 1) / 2));
  int64_t nb = (n + 15) / 16;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = 16 * b, hi = lo + 16 < n ? lo + 16 : n;
    float bmax = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float a = fabsf(x[i]);
      if (a > bmax) bmax = a;
    }
    float six_ts = 6.0f * ts;
    float sf = bmax / six_ts;               /* wanted block scale */
    int sc = orc_e4m3_nearest(sf);          /* stored 8-bit scale */
    float s = (float)orc_e4m3_value(sc);    /* exact */
    float denom = s * ts;                   /* one fp32 rounding */
    scales[b] = (uint8_t)sc;
    for (int64_t i = lo; i < hi; ++i) {
      int mag = 0;
      if (denom != 0.0f) {
        float v = x[i] / denom;             /* one fp32 rounding */
        mag = orc_e2m1_nearest(v);
      }
      int code = mag | (signbit(x[i]) ? 8 : 0);
      codes[i / 2] |= (uint8_t)((i & 1) ? (code << 4) : code);
    }
  }
  *ts_out = ts;
  return 0;
}

/* Exact value of an F32 or F16 element (the quantiser's inputs). */
static double elem_plain(const orc_tensor* t, int64_t i) {
  return t->dtype == ORC_F32 ? (double)((const float*)t->data)[i]
                             : orc_half_value(((const uint16_t*)t->data)[i]);
}

static int nibble(const uint8_t* codes, int64_t i) {
  return (i & 1) ? (codes[i / 2] >> 4) & 15 : codes[i / 2] & 15;
}

/* y[i] = e2m1(code_i) * e4m3(scale_{i/16}) * ts: the product is exact in
 * float64 (2 + 4 + 24 significant bits), then rounded once to fp32. */
void orc_nvfp4_unpack(const uint8_t* codes, const uint8_t* scales, float ts,
                      int64_t n, float* y) {
  for (int64_t i = 0; i < n; ++i)
    y[i] = (float)(orc_e2m1_value(nibble(codes, i)) *
                   orc_e4m3_value(scales[i / 16]) * (double)ts);
}

/* Nearest integer in [-127, 127] to v, ties to the even integer, values
 * beyond the ends take the end.  Brute force over the 255 candidates; every
 * difference is exact in float64. */
int orc_int8_nearest(float v) {
  int best = 0;
  double bestd = INFINITY;
  for (int c = -127; c <= 127; ++c) {
    double d = fabs((double)v - (double)c);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Value of the stored code of element i, without any scale: E4M3 or a
 * two's-complement byte.  The column scale is applied by the caller. */
static double code8_value(const orc_tensor* t, int64_t i) {
  uint8_t b = ((const uint8_t*)t->data)[i];
  return t->dtype == ORC_FP8 ? orc_e4m3_value(b) : (double)(int8_t)b;
}

/* Quantise the stored values of a CSC (vals[colptr[d_out]], F32 or F16, in
 * CSC order) to 8-bit codes with one scale per column.  Every step that
 * decides a code is one correctly rounded fp32 operation:
 *   amax_j = max |v| over column j;  s_j = amax_j / qmax, or 1 if that is 0
 *   (qmax = 448 for E4M3, the largest finite value; 127 for INT8);
 *   q = v / s_j;
 *   E4M3: code = (sign bit of v) << 7 | nearest magnitude code of |q|;
 *   INT8: code = nearest integer to q in [-127, 127], as a byte.
 * Decoded value of entry p in column j: value(code_p) * s_j.
 * Returns 0, or -1 (nothing written) if a value is NaN or infinite or kind
 * is neither ORC_FP8 nor ORC_INT8. */
int orc_quant8_csc(const void* vals, int32_t dtype, const int32_t* colptr, int32_t d_out,
                   int32_t kind, uint8_t* codes, float* col_scale) {
  if (kind != ORC_FP8 && kind != ORC_INT8) return -1;
  orc_tensor t = {dtype, vals, NULL, NULL, 0.0f, NULL};
  int64_t nnz = colptr[d_out];
  for (int64_t p = 0; p < nnz; ++p)
    if (!isfinite(elem_plain(&t, p))) return -1;
  const float qmax = kind == ORC_FP8 ? 448.0f : 127.0f;
  for (int32_t j = 0; j < d_out; ++j) {
    float amax = 0.0f;
    for (int64_t p = colptr[j]; p < colptr[j + 1]; ++p) {
      float a = fabsf((float)elem_plain(&t, p));
      if (a > amax) amax = a;
    }
    float s = amax / qmax;
    if (s == 0.0f) s = 1.0f;
    col_scale[j] = s;
    for (int64_t p = colptr[j]; p < colptr[j + 1]; ++p) {
      float v = (float)elem_plain(&t, p); /* exact: v is an f32 or f16 value */
      float q = v / s;
      if (kind == ORC_FP8)
        codes[p] = (uint8_t)(orc_e4m3_nearest(fabsf(q)) | (signbit(v) ? 0x80 : 0));
      else
        codes[p] = (uint8_t)(int8_t)orc_int8_nearest(q);
    }
  }
  return 0;
}

/* Exact float64 value of stored element i (8-bit codes: without their
 * column scale). */
static double elem(const orc_tensor* t, int64_t i) {
  switch (t->dtype) {
    case ORC_F32:
      return (double)((const float*)t->data)[i];
    case ORC_F16:
      return orc_half_value(((const uint16_t*)t->data)[i]);
    case ORC_FP8:
    case ORC_INT8:
      return code8_value(t, i);
    default:
      return orc_e2m1_value(nibble(t->codes, i)) *
             orc_e4m3_value(t->scales[i / 16]) * (double)t->ts;
  }
}

/* Dense row-major C (k x d_out, leading dimension ldc, dtype F32 or F16) to
 * CSC: for each column j, rows r ascending, keep C[r,j] iff it compares
 * unequal to zero (so +-0 are dropped and NaN is kept); the row index is
 * stored as uint16 and the value bit-copied.  colptr[0] = 0,
 * colptr[j+1] = colptr[j] + count_j.  Returns nnz, or -1 if nnz exceeds
 * capacity (then only colptr is written).  rowidx == NULL: colptr only. */
int64_t orc_pack_csc(const void* C, int32_t dtype, int32_t k, int32_t d_out,
                     int64_t ldc, int32_t* colptr, uint16_t* rowidx, void* vals,
                     int64_t capacity) {
  orc_tensor t = {dtype, C, NULL, NULL, 0.0f, NULL};
  int64_t nnz = 0;
  colptr[0] = 0;
  for (int32_t j = 0; j < d_out; ++j) {
    for (int32_t r = 0; r < k; ++r)
      if (elem(&t, (int64_t)r * ldc + j) != 0.0) ++nnz;
    colptr[j + 1] = (int32_t)nnz;
  }
  if (rowidx == NULL) return nnz;
  if (nnz > capacity) return -1;
  int64_t p = 0;
  size_t esz = dtype == ORC_F32 ? 4 : 2;
  for (int32_t j = 0; j < d_out; ++j)
    for (int32_t r = 0; r < k; ++r) {
      int64_t src = (int64_t)r * ldc + j;
      if (elem(&t, src) != 0.0) {
        rowidx[p] = (uint16_t)r;
        memcpy((char*)vals + p * esz, (const char*)C + src * esz, esz);
        ++p;
      }
    }
  return nnz;
}

/* Z = X D in float64 (T x k row-major), Eq. (1) of [Review], i ascending.
 * Returns a malloc'ed array, or NULL on allocation failure. */
/* A column-compressed index: colptr[0] = 0, colptr non-decreasing, and
 * every stored row (or block of `rows_per` rows) below k. */
static int csc_valid(int32_t k, int32_t d_out, const int32_t* colptr, const uint16_t* rowidx,
                     int32_t rows_per) {
  if (d_out < 0 || colptr[0] != 0) return 0;
  for (int32_t j = 0; j < d_out; ++j)
    if (colptr[j + 1] < colptr[j]) return 0;
  for (int32_t p = 0; p < colptr[d_out]; ++p)
    if ((int64_t)rowidx[p] * rows_per >= k) return 0;
  return 1;
}

static double* compute_z(int32_t T, const orc_tensor* X, int64_t ldx, int32_t d_in, int32_t k,
                         const orc_tensor* D, int64_t ldd) {
  double* Z = (double*)malloc(sizeof(double) * (size_t)T * (size_t)k);
  double* Xd = (double*)malloc(sizeof(double) * (size_t)T * (size_t)d_in);
  if (!Z || !Xd) {
    free(Z);
    free(Xd);
    return NULL;
  }
  for (int32_t t = 0; t < T; ++t)
    for (int32_t i = 0; i < d_in; ++i)
      Xd[(size_t)t * d_in + i] = elem(X, (int64_t)t * ldx + i);

#pragma omp parallel
  {
    double* atom = (double*)malloc(sizeof(double) * (size_t)d_in);
#pragma omp for schedule(static)
    for (int32_t a = 0; a < k; ++a) {
      for (int32_t i = 0; i < d_in; ++i) atom[i] = elem(D, (int64_t)a * ldd + i);
      for (int32_t t = 0; t < T; ++t) {
        const double* x = Xd + (size_t)t * d_in;
        double sum = 0.0;
        for (int32_t i = 0; i < d_in; ++i) sum += x[i] * atom[i];
        Z[(size_t)t * k + a] = sum;
      }
    }
    free(atom);
  }
  free(Xd);
  return Z;
}

/* Factored projection, Eq. (1) of [Review]:
 *   Z[t,a] = sum_{i=0..d_in-1} X[t,i] * D[i,a]        (i ascending)
 *   Y[t,j] = sum_{p=colptr[j]..colptr[j+1]-1} Z[t,rowidx[p]] * C_p  (p asc.)
 * X: T x d_in row-major (leading dim ldx).  D: d_in x k stored atom by atom
 * (element (i,a) at flat index a*ldd + i).  C: k x d_out in CSC; with 8-bit
 * codes C_p = value(code_p) * col_scale[j], exact in float64.
 * Y: T x d_out row-major float64, leading dimension d_out.
 * Returns 0; -1 on allocation failure; -2 (nothing computed) if the CSC is
 * not one: colptr[0] != 0, colptr decreasing somewhere, or a row index >= k.
 */
int orc_forward(int32_t T, const orc_tensor* X, int64_t ldx, int32_t d_in,
                int32_t k, const orc_tensor* D, int64_t ldd, int32_t d_out,
                const int32_t* colptr, const uint16_t* rowidx,
                const orc_tensor* C, double* Y) {
  if (!csc_valid(k, d_out, colptr, rowidx, 1)) return -2;
  if (T <= 0) return 0;
  double* Z = compute_z(T, X, ldx, d_in, k, D, ldd);
  if (!Z) return -1;
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < d_out; ++j)
    for (int32_t t = 0; t < T; ++t) {
      double sum = 0.0;
      for (int32_t p = colptr[j]; p < colptr[j + 1]; ++p) {
        double c = elem(C, p);
        if (C->col_scale) c *= (double)C->col_scale[j];
        sum += Z[(size_t)t * k + rowidx[p]] * c;
      }
      Y[(size_t)t * d_out + j] = sum;
    }
  free(Z);
  return 0;
}

/* Dense row-major C (k x d_out, dtype F32 or F16) to block-structured CSC
 * with blocks of 8 consecutive rows: for each column j and block b
 * ascending (rows 8b .. 8b+7, rows past k count as 0), the block is kept
 * iff one of its entries compares unequal to zero; a kept block stores b
 * as uint16 in bidx and its 8 values, bit-copied (rows past k as +0), in
 * vals[8 q .. 8 q + 7] for the q-th kept block.  bcolptr[j+1] - bcolptr[j]
 * counts the kept blocks of column j.  Returns the number of kept blocks,
 * or -1 if it exceeds capacity (then only bcolptr is written).  bidx ==
 * NULL: bcolptr only. */
int64_t orc_pack_bcsc(const void* C, int32_t dtype, int32_t k, int32_t d_out, int64_t ldc,
                      int32_t* bcolptr, uint16_t* bidx, void* vals, int64_t capacity) {
  orc_tensor t = {dtype, C, NULL, NULL, 0.0f, NULL};
  const int32_t nb = (k + 7) / 8;
  size_t esz = dtype == ORC_F32 ? 4 : 2;
  int64_t n = 0;
  bcolptr[0] = 0;
  for (int32_t j = 0; j < d_out; ++j) {
    for (int32_t b = 0; b < nb; ++b) {
      int any = 0;
      for (int32_t e = 0; e < 8 && 8 * b + e < k; ++e)
        if (elem(&t, (int64_t)(8 * b + e) * ldc + j) != 0.0) any = 1;
      n += any;
    }
    bcolptr[j + 1] = (int32_t)n;
  }
  if (bidx == NULL) return n;
  if (n > capacity) return -1;
  int64_t q = 0;
  for (int32_t j = 0; j < d_out; ++j)
    for (int32_t b = 0; b < nb; ++b) {
      int any = 0;
      for (int32_t e = 0; e < 8 && 8 * b + e < k; ++e)
        if (elem(&t, (int64_t)(8 * b + e) * ldc + j) != 0.0) any = 1;
      if (!any) continue;
      bidx[q] = (uint16_t)b;
      for (int32_t e = 0; e < 8; ++e) {
        char* dst = (char*)vals + (size_t)(8 * q + e) * esz;
        if (8 * b + e < k)
          memcpy(dst, (const char*)C + (size_t)((int64_t)(8 * b + e) * ldc + j) * esz, esz);
        else
          memset(dst, 0, esz);
      }
      ++q;
    }
  return n;
}

/* Factored projection with block-structured coefficients:
 *   Y[t,j] = sum over the kept blocks b of column j (ascending), over
 *            e = 0..7 with 8b+e < k, of Z[t, 8b+e] * vals[8 q + e]
 * (zeros inside a kept block included).  Z as in orc_forward.  C: the
 * values tensor (F32 or F16, 8 per kept block).  Returns 0, -1 on
 * allocation failure, -2 if the block index is not one (as orc_forward,
 * with block indices: 8 * bidx[q] < k). */
int orc_forward_bcsc(int32_t T, const orc_tensor* X, int64_t ldx, int32_t d_in, int32_t k,
                     const orc_tensor* D, int64_t ldd, int32_t d_out, const int32_t* bcolptr,
                     const uint16_t* bidx, const orc_tensor* C, double* Y) {
  if (!csc_valid(k, d_out, bcolptr, bidx, 8)) return -2;
  if (T <= 0) return 0;
  double* Z = compute_z(T, X, ldx, d_in, k, D, ldd);
  if (!Z) return -1;
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < d_out; ++j)
    for (int32_t t = 0; t < T; ++t) {
      double sum = 0.0;
      for (int32_t q = bcolptr[j]; q < bcolptr[j + 1]; ++q)
        for (int32_t e = 0; e < 8; ++e) {
          int32_t r = 8 * (int32_t)bidx[q] + e;
          if (r < k) sum += Z[(size_t)t * k + r] * elem(C, (int64_t)8 * q + e);
        }
      Y[(size_t)t * d_out + j] = sum;
    }
  free(Z);
  return 0;
}

/* ---------------------------------------------------------------- producer */

/* In-place Cholesky factorisation of the n x n symmetric positive definite
 * matrix A (row-major, lower triangle used): A = L L^T, L left in the lower
 * triangle.  Returns 0, or -1 if a pivot is not positive. */
static int cholesky(int n, double* A) {
  for (int j = 0; j < n; ++j) {
    double d = A[(size_t)j * n + j];
    for (int q = 0; q < j; ++q) d -= A[(size_t)j * n + q] * A[(size_t)j * n + q];
    if (!(d > 0.0)) return -1;
    double ljj = sqrt(d);
    A[(size_t)j * n + j] = ljj;
    for (int i = j + 1; i < n; ++i) {
      double v = A[(size_t)i * n + j];
      for (int q = 0; q < j; ++q) v -= A[(size_t)i * n + q] * A[(size_t)j * n + q];
      A[(size_t)i * n + j] = v / ljj;
    }
  }
  return 0;
}

/* Solve (L L^T) x = b in place for one right-hand side (stride 1). */
static void cholesky_solve(int n, const double* L, double* b) {
  for (int i = 0; i < n; ++i) {
    double v = b[i];
    for (int q = 0; q < i; ++q) v -= L[(size_t)i * n + q] * b[q];
    b[i] = v / L[(size_t)i * n + i];
  }
  for (int i = n - 1; i >= 0; --i) {
    double v = b[i];
    for (int q = i + 1; q < n; ++q) v -= L[(size_t)q * n + i] * b[q];
    b[i] = v / L[(size_t)i * n + i];
  }
}

/* P = (D^T S D + lambda I)^-1, Eq. (6)-(7) of [Review].  D is d_in x k,
 * given atom by atom: Dt[a * d_in + i] = D[i, a] (fp32); S is d_in x d_in
 * row-major fp32 (symmetric).  P out: k x k row-major float64.  Returns 0,
 * -1 if K is not positive definite, -2 on allocation failure. */
int orc_gram_inverse(int32_t d_in, int32_t k, const float* Dt, const float* S, double lambda,
                     double* P) {
  double* U = (double*)malloc(sizeof(double) * (size_t)k * d_in);
  double* K = (double*)malloc(sizeof(double) * (size_t)k * k);
  double* e = (double*)malloc(sizeof(double) * (size_t)k);
  if (!U || !K || !e) {
    free(U);
    free(K);
    free(e);
    return -2;
  }
  /* U = D^T S (k x d_in), then K = U D + lambda I */
#pragma omp parallel for schedule(static)
  for (int32_t a = 0; a < k; ++a)
    for (int32_t j = 0; j < d_in; ++j) {
      double v = 0.0;
      for (int32_t i = 0; i < d_in; ++i)
        v += (double)Dt[(size_t)a * d_in + i] * (double)S[(size_t)i * d_in + j];
      U[(size_t)a * d_in + j] = v;
    }
#pragma omp parallel for schedule(static)
  for (int32_t a = 0; a < k; ++a)
    for (int32_t b = 0; b < k; ++b) {
      double v = 0.0;
      for (int32_t j = 0; j < d_in; ++j) v += U[(size_t)a * d_in + j] * (double)Dt[(size_t)b * d_in + j];
      K[(size_t)a * k + b] = v + (a == b ? lambda : 0.0);
    }
  int rc = cholesky(k, K);
  if (rc == 0) {
    /* column b of P solves K x = e_b */
    for (int32_t b = 0; b < k; ++b) {
      for (int32_t a = 0; a < k; ++a) e[a] = a == b ? 1.0 : 0.0;
      cholesky_solve(k, K, e);
      for (int32_t a = 0; a < k; ++a) P[(size_t)a * k + b] = e[a];
    }
  }
  free(U);
  free(K);
  free(e);
  return rc;
}

/* One deletion with compensation, Eq. (7): remove coordinate i of c by the
 * move delta = -(c_i / P_ii) P e_i (P symmetric, row-major k x k), applied
 * to c in place (c_i becomes 0 up to rounding).  Returns the saliency
 * c_i^2 / P_ii of the deleted value. */
double orc_obs_delete(int32_t k, const double* P, double* c, int32_t i) {
  double ci = c[i], pii = P[(size_t)i * k + i];
  double f = ci / pii;
  for (int32_t a = 0; a < k; ++a) c[a] -= P[(size_t)i * k + a] * f;
  return ci * ci / pii;
}

typedef struct {
  float s;
  int32_t row;
} score_t;

static int score_cmp(const void* x, const void* y) {
  const score_t* a = (const score_t*)x;
  const score_t* b = (const score_t*)y;
  if (a->s < b->s) return -1;
  if (a->s > b->s) return 1;
  return a->row < b->row ? -1 : (a->row > b->row);
}

/* Fixed-inverse pruning of every column of C ([Review] Algorithm 1, a
 * reading of the paper's Algorithm 2).  C: k x d_out row-major fp32, the
 * unpruned coefficients.  P: k x k row-major fp32 (the fixed inverse).  Per
 * column j, independently (the blocks of the algorithm only batch work):
 *   score_i = (c_i * c_i) / P_ii in fp32 (each operation rounded), from the
 *   column's values before any deletion;
 *   the n_prune rows of smallest score, ties to the lower row, are marked;
 *   for each marked row i in that order: read the current c_i and apply the
 *   Eq. (7) move c -= P[:, i] * c_i / P_ii (float64);
 *   finally every marked entry is set to exactly 0.
 * C_out: k x d_out row-major float64.  keep: k x d_out bytes, 1 where the
 * entry stays in the support, 0 where it was pruned.  Returns 0, or -1 on
 * allocation failure or a non-positive P_ii. */
int orc_obs_prune(int32_t k, int32_t d_out, const float* C, const float* P, int32_t n_prune,
                  double* C_out, uint8_t* keep) {
  if (n_prune < 0) n_prune = 0;
  if (n_prune > k) n_prune = k;
  for (int32_t i = 0; i < k; ++i)
    if (!(P[(size_t)i * k + i] > 0.0f)) return -1;
  double* Pd = (double*)malloc(sizeof(double) * (size_t)k * k);
  if (!Pd) return -1;
  for (size_t q = 0; q < (size_t)k * k; ++q) Pd[q] = (double)P[q];
  int bad = 0;
#pragma omp parallel
  {
    score_t* sc = (score_t*)malloc(sizeof(score_t) * (size_t)k);
    double* c = (double*)malloc(sizeof(double) * (size_t)k);
    if (!sc || !c) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int32_t j = 0; j < d_out; ++j) {
      if (!sc || !c) continue;
      for (int32_t i = 0; i < k; ++i) {
        float ci = C[(size_t)i * d_out + j];
        float sq = ci * ci;
        sc[i].s = sq / P[(size_t)i * k + i];
        sc[i].row = i;
        c[i] = (double)ci;
      }
      qsort(sc, (size_t)k, sizeof(score_t), score_cmp);
      for (int32_t t = 0; t < n_prune; ++t) orc_obs_delete(k, Pd, c, sc[t].row);
      for (int32_t i = 0; i < k; ++i) keep[(size_t)i * d_out + j] = 1;
      for (int32_t t = 0; t < n_prune; ++t) {
        c[sc[t].row] = 0.0;
        keep[(size_t)sc[t].row * d_out + j] = 0;
      }
      for (int32_t i = 0; i < k; ++i) C_out[(size_t)i * d_out + j] = c[i];
    }
    free(sc);
    free(c);
  }
  free(Pd);
  return bad ? -1 : 0;
}

/* Dictionary refit, Eq. (9) of [Review]: D (C C^T + lambda I) = W C^T, with
 * W = [W_1 .. W_n] (d_in x N row-major fp32, N = n d_out) and the pruned
 * coefficients C = [C_1 .. C_n] (k x N row-major fp32, zeros kept).  The
 * result is returned atom by atom: Dt[a * d_in + i] = D[i, a] (float64),
 * i.e. Dt = (C C^T + lambda I)^-1 (W C^T)^T.  Returns 0, -1 if the Gram
 * matrix is not positive definite, -2 on allocation failure. */
int orc_refit(int32_t d_in, int32_t N, int32_t k, const float* W, const float* Cm, double lambda,
              double* Dt) {
  double* G = (double*)malloc(sizeof(double) * (size_t)k * k);
  if (!G) return -2;
#pragma omp parallel for schedule(static)
  for (int32_t a = 0; a < k; ++a)
    for (int32_t b = 0; b < k; ++b) {
      double v = 0.0;
      for (int32_t j = 0; j < N; ++j) v += (double)Cm[(size_t)a * N + j] * (double)Cm[(size_t)b * N + j];
      G[(size_t)a * k + b] = v + (a == b ? lambda : 0.0);
    }
  int rc = cholesky(k, G);
  if (rc == 0) {
#pragma omp parallel
    {
      double* r = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
      for (int32_t i = 0; i < d_in; ++i) {
        if (!r) continue;
        /* row i of W C^T, then solve G x = that row: x is row i of D */
        for (int32_t a = 0; a < k; ++a) {
          double v = 0.0;
          for (int32_t j = 0; j < N; ++j) v += (double)W[(size_t)i * N + j] * (double)Cm[(size_t)a * N + j];
          r[a] = v;
        }
        cholesky_solve(k, G, r);
        for (int32_t a = 0; a < k; ++a) Dt[(size_t)a * d_in + i] = r[a];
      }
      free(r);
    }
  }
  free(G);
  return rc;
}

/* Set the number of threads of the parallel loops above (n >= 1). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int orc_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
