/*
 * oracle.c -- plain, slow, float64 CPU definitions of the CSR sparse-dense
 * operations.  TEST INFRASTRUCTURE ONLY: nothing in the library's product
 * path may call, link or load this file; only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header or table with the GPU library.
 *
 * Source of the definitions: the spops README (IST-DASLab), section "Usage"
 * (the CSR layout: values, row_offsets[m+1], col_idx, row_idx) and the four
 * operation paragraphs ("Sparse Addition", "Sparse Matrix Multiplication
 * (SpMM)", "Sampled Dense-Dense Matrix Multiplication (SDDMM)", "CSR
 * Transpose").  Each function below states the definition it writes out.
 *
 * Numerics: every floating input is widened exactly to double (own decoders
 * for binary16 and bfloat16 bit patterns below); sums are taken in double in
 * the stated order; results are returned in double, except csr_add, whose
 * definition stores into the dense operand's own dtype (round to nearest,
 * ties to even, with an own encoder).
 *
 * dtype codes: 0 = float32, 1 = float16 (binary16 bits), 2 = bfloat16 bits.
 * index codes: 0 = int16, 1 = int32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_I16 = 0, OR_I32 = 1 };

/* ---------------------------------------------------------------- decoders */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + f, e - 25);             /* (1 + f/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 7) & 0xff, f = h & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(128.0 + f, e - 134);             /* (1 + f/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* ---------------------------------------------------------------- encoders */

/* Round x to the nearest value with `mant` fraction bits and minimum normal
 * exponent `emin`, ties to even, then encode it.  Values that round past the
 * largest finite value become infinity.  Implementation: the spacing of
 * representable values at x's binade is q = 2^(max(e, emin) - mant) with
 * e = floor(log2|x|); x/q is exact and rint() rounds it to the nearest
 * integer, ties to even (the default rounding mode). */
static uint16_t encode_small_float(double x, int mant, int emin, int ebits) {
  int bias = (1 << (ebits - 1)) - 1;
  uint16_t sign = signbit(x) ? (uint16_t)(1u << (mant + ebits)) : 0;
  uint16_t inf = (uint16_t)(((1u << ebits) - 1) << mant);
  if (isnan(x)) return (uint16_t)(inf | (1u << (mant - 1)));
  double a = fabs(x);
  if (isinf(a)) return sign | inf;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1)  =>  floor(log2 a) = e-1 */
  e -= 1;
  int eq = e < emin ? emin : e;
  double q = ldexp(1.0, eq - mant);
  double r = rint(a / q) * q;                  /* rounded magnitude */
  if (r == 0.0) return sign;
  if (r >= ldexp(1.0, bias + 1)) return sign | inf;
  frexp(r, &e);
  e -= 1;
  if (e < emin) /* subnormal */
    return sign | (uint16_t)(r / ldexp(1.0, emin - mant));
  uint32_t frac = (uint32_t)((r / ldexp(1.0, e) - 1.0) * (double)(1u << mant));
  return sign | (uint16_t)(((uint32_t)(e + bias) << mant) | frac);
}

uint16_t oracle_encode_f16(double x) { return encode_small_float(x, 10, -14, 5); }
uint16_t oracle_encode_bf16(double x) { return encode_small_float(x, 7, -126, 8); }

/* ----------------------------------------------------------------- access */

/* Every 16-bit pattern decoded once by the decoders above (speed only). */
static double f16_table[65536], bf16_table[65536];
static int tables_ready = 0;

static void init_tables(void) {
  if (tables_ready) return;
  for (int i = 0; i < 65536; ++i) {
    f16_table[i] = oracle_decode_f16((uint16_t)i);
    bf16_table[i] = oracle_decode_bf16((uint16_t)i);
  }
  tables_ready = 1;
}

static double load_val(const void* p, int dt, int64_t i) {
  switch (dt) {
    case OR_F32: return (double)((const float*)p)[i];
    case OR_F16: return f16_table[((const uint16_t*)p)[i]];
    default:     return bf16_table[((const uint16_t*)p)[i]];
  }
}

static void store_val(void* p, int dt, int64_t i, double x) {
  switch (dt) {
    case OR_F32: ((float*)p)[i] = (float)x; break;  /* C conversion: RNE */
    case OR_F16: ((uint16_t*)p)[i] = oracle_encode_f16(x); break;
    default:     ((uint16_t*)p)[i] = oracle_encode_bf16(x); break;
  }
}

static int64_t load_idx(const void* p, int it, int64_t i) {
  return it == OR_I16 ? (int64_t)((const int16_t*)p)[i] : (int64_t)((const int32_t*)p)[i];
}

static void store_idx(void* p, int it, int64_t i, int64_t v) {
  if (it == OR_I16) ((int16_t*)p)[i] = (int16_t)v;
  else ((int32_t*)p)[i] = (int32_t)v;
}

/* Structural check of a CSR: offsets start at 0, never decrease, end at nnz;
 * every column index lies in [0, n).  Returns 0 when valid. */
int oracle_check_csr(int64_t m, int64_t n, const int32_t* ro, const void* col, int ct) {
  if (ro[0] != 0) return 1;
  for (int64_t r = 0; r < m; ++r)
    if (ro[r + 1] < ro[r]) return 2;
  for (int64_t p = 0; p < ro[m]; ++p) {
    int64_t c = load_idx(col, ct, p);
    if (c < 0 || c >= n) return 3;
  }
  return 0;
}

/* ------------------------------------------------------------------- SpMM */

/* SpMM (spops README, section "Sparse Matrix Multiplication (SpMM)"):
 * C = A * B with A m x k in CSR and B k x N dense (row-major, row
 * stride ldb).  Definition:
 *     C[r][j] = sum over p in [row_offsets[r], row_offsets[r+1])
 *               of values[p] * B[col_idx[p]][j],
 * summed in stored order; a row with no entries gives zeros.  row_idx only
 * orders the work and does not enter the definition.  C is m x N, row-major,
 * contiguous, float64. */
int oracle_spmm(int64_t m, int64_t k, int64_t N, const int32_t* ro, const void* col, int ct,
                const void* val, int vt, const void* B, int bt, int64_t ldb, double* C) {
  init_tables();
  (void)k;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < m; ++r) {
    double* crow = C + r * N;
    for (int64_t j = 0; j < N; ++j) crow[j] = 0.0;
    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {
      double a = load_val(val, vt, p);
      int64_t c = load_idx(col, ct, p);
      for (int64_t j = 0; j < N; ++j) crow[j] += a * load_val(B, bt, c * ldb + j);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ SDDMM */

/* SDDMM (spops README, section "Sampled Dense-Dense Matrix Multiplication
 * (SDDMM)"): the product A * B is evaluated only at the
 * positions of the output mask, with B supplied transposed (BT, n x K).
 * Definition, for each stored position p of row r with column c = col_idx[p]:
 *     out[p] = sum_{k=0}^{K-1} A[r][k] * BT[c][k]
 * (summed in k order), out in the mask's CSR order.  The mask carries no
 * values, so nothing multiplies the sum.  Both backends the page lists
 * ("sputnik", "structure_aware") compute this same quantity. */
int oracle_sddmm(int64_t m, int64_t n, int64_t K, const int32_t* ro, const void* col, int ct,
                 const void* A, int64_t lda, const void* BT, int64_t ldbt, int it,
                 double* out) {
  init_tables();
  (void)n;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {
      int64_t c = load_idx(col, ct, p);
      double s = 0.0;
      for (int64_t kk = 0; kk < K; ++kk)
        s += load_val(A, it, r * lda + kk) * load_val(BT, it, c * ldbt + kk);
      out[p] = s;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- csr_add */

/* Sparse addition (spops README, section "Sparse Addition"): the sparse
 * matrix is added into the dense one, taken in place on the dense operand W (m x n, row stride ldw):
 *     W[r][col_idx[p]] <- round(W[r][col_idx[p]] + values[p])
 * for every stored position p of row r; every other element of W is left as
 * it was.  The sum is formed in double and then rounded to W's dtype
 * (nearest, ties to even).  For operands of p significant bits (24, 11 or 8)
 * that double rounding equals a single correct rounding of the exact sum,
 * because 53 >= 2p + 1 (Figueroa, "When is double rounding innocuous?",
 * 1995).  Positions repeated within a row would be added one after the
 * other. */
int oracle_csr_add(int64_t m, int64_t n, const int32_t* ro, const void* col, int ct,
                   const void* val, int vt, void* W, int wt, int64_t ldw) {
  init_tables();
  (void)n;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {
      int64_t i = r * ldw + load_idx(col, ct, p);
      store_val(W, wt, i, load_val(W, wt, i) + load_val(val, vt, p));
    }
  }
  return 0;
}

/* ---------------------------------------------------------- csr_transpose */

/* CSR transpose (spops README, section "CSR Transpose"): A^T of the m x n matrix A,
 * stored as an n x m CSR (the CSC of A).  Definition as a stable counting
 * sort of the stored entries by column:
 *   cnt[c] = number of entries with column c;
 *   out_ro[0] = 0, out_ro[c+1] = out_ro[c] + cnt[c];
 *   visiting rows r = 0..m-1 in order and the entries of each row in stored
 *   order, the entry (r, c, v) goes to slot q = next[c]++ (next starts at
 *   out_ro[c]) with out_col[q] = r and out_val[q] = v.
 * Within each output row the source rows therefore ascend.  Values are moved,
 * not converted: val_bytes is the size of one value (0 = no values). */
int oracle_csr_transpose(int64_t m, int64_t n, const int32_t* ro, const void* col, int ct,
                         const void* val, int64_t val_bytes, void* out_val, int32_t* out_ro,
                         void* out_col, int out_ct) {
  int64_t nnz = ro[m];
  int64_t* next = (int64_t*)calloc((size_t)n + 1, sizeof(int64_t));
  if (!next) return -1;
  for (int64_t p = 0; p < nnz; ++p) next[load_idx(col, ct, p) + 1] += 1;
  out_ro[0] = 0;
  for (int64_t c = 0; c < n; ++c) {
    next[c + 1] += next[c];
    out_ro[c + 1] = (int32_t)next[c + 1];
  }
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {
      int64_t c = load_idx(col, ct, p);
      int64_t q = next[c]++;
      store_idx(out_col, out_ct, q, r);
      if (val_bytes)
        memcpy((char*)out_val + q * val_bytes, (const char*)val + p * val_bytes,
               (size_t)val_bytes);
    }
  }
  free(next);
  return 0;
}

/* ---------------------------------------------------------------- row_idx */

/* row_idx (spops README, section "Usage"): a permutation of 0..m-1 ordering the rows
 * by their number of stored entries.  Reading taken: most entries first,
 * equal counts in ascending row order.  Written as a stable counting sort on
 * the key (maxcount - count). */
int oracle_row_idx(int64_t m, const int32_t* ro, void* row_idx, int rt) {
  int64_t maxc = 0;
  for (int64_t r = 0; r < m; ++r)
    if (ro[r + 1] - ro[r] > maxc) maxc = ro[r + 1] - ro[r];
  int64_t* start = (int64_t*)calloc((size_t)maxc + 2, sizeof(int64_t));
  if (!start) return -1;
  for (int64_t r = 0; r < m; ++r) start[maxc - (ro[r + 1] - ro[r]) + 1] += 1;
  for (int64_t b = 0; b <= maxc; ++b) start[b + 1] += start[b];
  for (int64_t r = 0; r < m; ++r) {
    int64_t b = maxc - (ro[r + 1] - ro[r]);
    store_idx(row_idx, rt, start[b]++, r);
  }
  free(start);
  return 0;
}

/* -------------------------------------------------------------- utilities */

/* Conversion helpers exposed so that tests can pin the decoders/encoders. */
void oracle_decode_array(const uint16_t* in, int dt, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = dt == OR_F16 ? oracle_decode_f16(in[i]) : oracle_decode_bf16(in[i]);
}

void oracle_encode_array(const double* in, int dt, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = dt == OR_F16 ? oracle_encode_f16(in[i]) : oracle_encode_bf16(in[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
