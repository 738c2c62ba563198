/*
 * Reference ("oracle") for C = A * B^T with IEEE binary16 (or bfloat16) inputs.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no source with the GPU path.
 *
 * What it computes follows the problem statement of "SASS-Level Kernel
 * Generation for Blackwell" (section "The numbers", Setup): fp16 inputs,
 * fp32 accumulation and output, C = A B^T.  The oracle keeps the definition
 * and raises the accumulation to binary64, as the double-accumulated CPU
 * reference of the handbook page "Asynchronous copies and the Hopper/Blackwell
 * features" (section "Thread-block clusters and distributed shared memory")
 * does, and stays a plain triple loop like that page's cp.async example check
 * (section "cp.async and multi-stage pipelines").
 *
 *   C[i][j] = sum_{k=0}^{K-1} a_ik * b_jk     (binary64, k increasing)
 *   S[i][j] = sum_{k=0}^{K-1} |a_ik * b_jk|   (same loop, same order)
 *
 * A is M x K, row i at A + i*lda; B is N x K, row j at B + j*ldb; both hold
 * binary16 bit patterns (the *_bf16 entry points: bfloat16 bit patterns).
 * Every fp16 x fp16 product is exact in binary64 (11-bit significands give
 * at most 22 significant bits; bfloat16's 8-bit significands give 16, and
 * its exponent range stays far inside binary64's), so the only rounding is
 * the binary64 running sum.
 *
 * Threads split the rows i among themselves; each element is still summed by
 * one thread in increasing k, so the result does not depend on the thread
 * count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0      : subnormal, value = fraction * 2^-24
 * exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)
 * exponent 31     : fraction 0 -> infinity, otherwise NaN                   */
double oracle_half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 0x1f;
  const int frac = h & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24);
  } else if (expo == 31) {
    mag = frac == 0 ? INFINITY : NAN;
  } else {
    mag = ldexp((double)(1024 + frac), expo - 25);
  }
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits -- the
 * upper half of an IEEE 754 binary32 pattern.
 * exponent 0      : subnormal, value = fraction * 2^-133   (2^(1-127) * 2^-7)
 * exponent 1..254 : normal,    value = (128 + fraction) * 2^(exponent-134)
 * exponent 255    : fraction 0 -> infinity, otherwise NaN                   */
double oracle_bf16_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 7) & 0xff;
  const int frac = h & 0x7f;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -133);
  } else if (expo == 255) {
    mag = frac == 0 ? INFINITY : NAN;
  } else {
    mag = ldexp((double)(128 + frac), expo - 134);
  }
  return sign ? -mag : mag;
}

/* Decoded value of every 16-bit pattern in each format, filled once from the
 * functions above. */
static double g_half_table[65536];
static double g_bf16_table[65536];
static pthread_once_t g_table_once = PTHREAD_ONCE_INIT;

static void fill_tables(void) {
  for (uint32_t h = 0; h < 65536u; ++h) {
    g_half_table[h] = oracle_half_to_double((uint16_t)h);
    g_bf16_table[h] = oracle_bf16_to_double((uint16_t)h);
  }
}

/* fmt 0: binary16, fmt 1: bfloat16 */
static const double* decode_table(int fmt) {
  pthread_once(&g_table_once, fill_tables);
  return fmt == 1 ? g_bf16_table : g_half_table;
}

/* One output element: the definition written out. */
static void dot_one(const uint16_t* a_row, const uint16_t* b_row, int64_t K,
                    const double* dec, double* c_out, double* s_out) {
  double c = 0.0, s = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double p = dec[a_row[k]] * dec[b_row[k]];
    c += p;
    s += fabs(p);
  }
  *c_out = c;
  *s_out = s;
}

typedef struct {
  int64_t M, N, K;
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  double* C;
  int64_t ldc;
  double* S;
  int64_t lds;
  /* element list mode (rows/cols non-NULL): n entries */
  const int64_t* rows;
  const int64_t* cols;
  int64_t n;
  int64_t lo, hi; /* this worker's share: rows [lo,hi) or entries [lo,hi) */
  int fmt;        /* operand format: 0 binary16, 1 bfloat16 */
} job_t;

static void* full_worker(void* arg) {
  const job_t* j = (const job_t*)arg;
  const double* dec = decode_table(j->fmt);
  for (int64_t i = j->lo; i < j->hi; ++i)
    for (int64_t c = 0; c < j->N; ++c)
      dot_one(j->A + i * j->lda, j->B + c * j->ldb, j->K, dec,
              &j->C[i * j->ldc + c], &j->S[i * j->lds + c]);
  return NULL;
}

static void* elems_worker(void* arg) {
  const job_t* j = (const job_t*)arg;
  const double* dec = decode_table(j->fmt);
  for (int64_t e = j->lo; e < j->hi; ++e)
    dot_one(j->A + j->rows[e] * j->lda, j->B + j->cols[e] * j->ldb, j->K, dec,
            &j->C[e], &j->S[e]);
  return NULL;
}

/* Split [0,total) into `threads` contiguous shares and run `fn` on each. */
static int run_split(job_t base, int64_t total, int threads, void* (*fn)(void*)) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((int64_t)threads > total) threads = total > 0 ? (int)total : 1;
  pthread_t tid[256];
  job_t jobs[256];
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    jobs[t] = base;
    jobs[t].lo = total * t / threads;
    jobs[t].hi = total * (t + 1) / threads;
  }
  for (int t = 1; t < threads; ++t) {
    if (pthread_create(&tid[t], NULL, fn, &jobs[t]) != 0) break;
    started = t;
  }
  /* shares whose thread did not start run here, in order */
  fn(&jobs[0]);
  for (int t = started + 1; t < threads; ++t) fn(&jobs[t]);
  for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
  return threads;
}

/* Full M x N result. C and S are row-major binary64 with strides ldc, lds;
 * A and B hold patterns of format fmt (0 binary16, 1 bfloat16).
 * Returns the number of threads used, or -1 on invalid arguments. */
static int gemm_full(int fmt, int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     double* C, int64_t ldc, double* S, int64_t lds, int threads) {
  if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N || lds < N) return -1;
  if (M == 0 || N == 0) return 0;
  job_t j = {M, N, K, A, lda, B, ldb, C, ldc, S, lds, NULL, NULL, 0, 0, 0, fmt};
  return run_split(j, M, threads, full_worker);
}

/* Selected elements (rows[e], cols[e]) for e < n, into C[e] and S[e].
 * Returns the number of threads used, or -1 on invalid arguments. */
static int gemm_elems(int fmt, int64_t n, const int64_t* rows, const int64_t* cols, int64_t K,
                      const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      double* C, double* S, int threads) {
  if (n < 0 || K < 0 || lda < K || ldb < K) return -1;
  if (n == 0) return 0;
  job_t j = {0, 0, K, A, lda, B, ldb, C, 0, S, 0, rows, cols, n, 0, 0, fmt};
  return run_split(j, n, threads, elems_worker);
}

/* binary16 operands */
int oracle_gemm_abt(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    double* C, int64_t ldc, double* S, int64_t lds, int threads) {
  return gemm_full(0, M, N, K, A, lda, B, ldb, C, ldc, S, lds, threads);
}

int oracle_gemm_abt_elems(int64_t n, const int64_t* rows, const int64_t* cols, int64_t K,
                          const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                          double* C, double* S, int threads) {
  return gemm_elems(0, n, rows, cols, K, A, lda, B, ldb, C, S, threads);
}

/* bfloat16 operands */
int oracle_gemm_abt_bf16(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                         double* C, int64_t ldc, double* S, int64_t lds, int threads) {
  return gemm_full(1, M, N, K, A, lda, B, ldb, C, ldc, S, lds, threads);
}

int oracle_gemm_abt_elems_bf16(int64_t n, const int64_t* rows, const int64_t* cols, int64_t K,
                               const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               double* C, double* S, int threads) {
  return gemm_elems(1, n, rows, cols, K, A, lda, B, ldb, C, S, threads);
}
