/*
 * Oracle for the fused all-gather + GEMM: a plain, slow, obviously correct CPU
 * implementation of what the operation computes.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this
 * code: only the tests, the package smoke check and the bench's CPU-baseline leg use it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What is computed (pytorch/helion PR "[Benchmark] Add all gather matmul benchmark",
 * the Kraken-optimization comment: a = all_gather(a_shared), out = a @ b; the same
 * comment's local-tile index formula fixes that shard r holds global rows
 * [r*M_per_rank, (r+1)*M_per_rank)):
 *
 *   A[d*M_s + i][k] = shard_d[i][k]                      (concatenate in rank order)
 *   C[i][j]         = sum_{k=0..K-1} A[i][k] * B[k][j]   (fp64, k ascending)
 *                     (+ bias[j], the optional bias of ROCm/iris issue "Fused
 *                      all-gather+GEMM HBM-buffer kernel for iris.ops", "New kernel")
 *   out[i][j]       = round-to-nearest-even of C[i][j] into the 16-bit type,
 *                     rounded once, straight from the double.
 *
 * Every product of two 16-bit floats is exact in double; the sum's rounding error is
 * bounded by K * 2^-53 * sum|a*b|.
 *
 * 16-bit formats are handled as raw bit patterns (uint16_t) and decoded / encoded
 * from the IEEE 754 definitions: binary16 (1 sign, 5 exponent, 10 fraction bits,
 * bias 15) and bfloat16 (1 sign, 8 exponent, 7 fraction bits, bias 127).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC agmm_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F16 0
#define ORACLE_BF16 1

/* Format parameters: p = significand bits including the implicit one,
 * emin/emax = exponent range of normal numbers, ebits = exponent field width. */
typedef struct { int p, emin, emax, ebits; } fmt_t;
static const fmt_t FMT_F16 = {11, -14, 15, 5};
static const fmt_t FMT_BF16 = {8, -126, 127, 8};

static fmt_t fmt_of(int dtype) { return dtype == ORACLE_BF16 ? FMT_BF16 : FMT_F16; }

/* Decode a 16-bit pattern to the exact double it denotes. */
static double decode16(uint16_t h, fmt_t f) {
  int fbits = f.p - 1;                       /* stored fraction bits */
  int bias = f.emax;                         /* 15 or 127 */
  int sign = (h >> 15) & 1;
  int e = (h >> fbits) & ((1 << f.ebits) - 1);
  int frac = h & ((1 << fbits) - 1);
  double v;
  if (e == (1 << f.ebits) - 1) {
    v = frac ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)frac, f.emin - fbits);             /* subnormal or zero */
  } else {
    v = ldexp((double)((1 << fbits) | frac), e - bias - fbits);
  }
  return sign ? -v : v;
}

/* Round-half-to-even of a non-negative double holding a value < 2^53. */
static double rne_integer(double n) {
  double fl = floor(n);
  double diff = n - fl;                      /* exact */
  if (diff > 0.5) return fl + 1.0;
  if (diff < 0.5) return fl;
  return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/* Encode a double into the 16-bit format with round-to-nearest-even, directly
 * from the double (no intermediate float). Overflow gives +-inf, NaN a quiet NaN. */
static uint16_t encode16(double x, fmt_t f) {
  int fbits = f.p - 1;
  int bias = f.emax;
  uint16_t inf_bits = (uint16_t)(((1 << f.ebits) - 1) << fbits);
  if (isnan(x)) return (uint16_t)(inf_bits | (1 << (fbits - 1)));
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | inf_bits);
  int E;
  frexp(a, &E);                              /* a = m * 2^E, m in [0.5, 1) */
  int e = E - 1;                             /* a in [2^e, 2^(e+1)) */
  if (e < f.emin) e = f.emin;                /* subnormal range shares emin's quantum */
  double n = ldexp(a, fbits - e);            /* a / quantum, exact scaling, < 2^p */
  double r = rne_integer(n);
  if (r >= ldexp(1.0, f.p)) {                /* rounding carried into the next binade */
    r = ldexp(1.0, f.p - 1);
    e += 1;
  }
  if (e > f.emax) return (uint16_t)(sign | inf_bits);
  uint32_t ri = (uint32_t)r;
  if (ri < (1u << fbits)) {                  /* subnormal: exponent field 0 */
    return (uint16_t)(sign | ri);
  }
  uint32_t efield = (uint32_t)(e + bias);
  return (uint16_t)(sign | (efield << fbits) | (ri - (1u << fbits)));
}

/* ---- exported scalar codecs ---- */
double oracle_decode(int dtype, uint16_t h) { return decode16(h, fmt_of(dtype)); }
uint16_t oracle_encode_rne(int dtype, double x) { return encode16(x, fmt_of(dtype)); }

void oracle_decode_array(int dtype, int64_t n, const uint16_t* in, double* out) {
  fmt_t f = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i) out[i] = decode16(in[i], f);
}

void oracle_encode_array(int dtype, int64_t n, const double* in, uint16_t* out) {
  fmt_t f = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i) out[i] = encode16(in[i], f);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Global row i of the gathered A: shard i / M_s, local row i - shard * M_s. */
static const uint16_t* gathered_row(const uint16_t* const* shards, int64_t M_s, int64_t K,
                                    int64_t i) {
  int64_t d = i / M_s;
  return shards[d] + (i - d * M_s) * K;
}

/*
 * Full oracle: C (M x N doubles, unrounded, required) and out16 (M x N rounded
 * patterns, optional). Rows [row_begin, row_end) only, so that a bounded sample of
 * a large workload can be timed; pass 0 and M for the whole result. C and out16
 * hold row_end - row_begin rows, the first being global row row_begin. Loop order
 * i, k, j keeps every C[i][j] summed in ascending k. Returns the thread count used.
 */
int oracle_agmm_rows(int dtype, int D, int64_t M, int64_t N, int64_t K,
                     const uint16_t* const* shards, const uint16_t* B, const uint16_t* bias,
                     int64_t row_begin, int64_t row_end, double* C, uint16_t* out16) {
  fmt_t f = fmt_of(dtype);
  int64_t M_s = M / D;
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
  for (int64_t t = 0; t < K * N; ++t) Bd[t] = decode16(B[t], f);
  int used = 1;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double* arow = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
      const uint16_t* src = gathered_row(shards, M_s, K, i);
      for (int64_t k = 0; k < K; ++k) arow[k] = decode16(src[k], f);
      double* c = C + (i - row_begin) * N;
      for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double a = arow[k];
        const double* brow = Bd + k * N;
        for (int64_t j = 0; j < N; ++j) c[j] += a * brow[j];
      }
      if (bias)
        for (int64_t j = 0; j < N; ++j) c[j] += decode16(bias[j], f);
      if (out16)
        for (int64_t j = 0; j < N; ++j) out16[(i - row_begin) * N + j] = encode16(c[j], f);
    }
    free(arow);
  }
  free(Bd);
  return used;
}

/*
 * The gathered A itself, the first result of the op a = all_gather(a_shared) (same
 * comment as above): A_out[i][k] = A[i][k] for i in [0, D*M_s), a bit copy, row by row.
 */
void oracle_all_gather(int D, int64_t M_s, int64_t K, const uint16_t* const* shards,
                       uint16_t* A_out) {
  for (int64_t i = 0; i < (int64_t)D * M_s; ++i) {
    const uint16_t* src = gathered_row(shards, M_s, K, i);
    for (int64_t k = 0; k < K; ++k) A_out[i * K + k] = src[k];
  }
}

/* Selected outputs one by one: C_out[s] = C[rows[s]][cols[s]] (unrounded). */
void oracle_agmm_at(int dtype, int D, int64_t M, int64_t N, int64_t K,
                    const uint16_t* const* shards, const uint16_t* B, const uint16_t* bias,
                    int64_t count, const int64_t* rows, const int64_t* cols, double* C_out) {
  fmt_t f = fmt_of(dtype);
  int64_t M_s = M / D;
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < count; ++s) {
    const uint16_t* arow = gathered_row(shards, M_s, K, rows[s]);
    int64_t j = cols[s];
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += decode16(arow[k], f) * decode16(B[k * N + j], f);
    if (bias) acc += decode16(bias[j], f);
    C_out[s] = acc;
  }
}

/*
 * Tolerance check of a 16-bit result against the unrounded reference:
 *   |got - C| <= rtol * |C| + atol  for every element; a NaN in got fails.
 * Returns the number of failing elements; reports the largest absolute error, the
 * largest err / tol ratio, and the first failing flat index (-1 if none).
 */
int64_t oracle_check(int dtype, int64_t n, const uint16_t* got, const double* C, double rtol,
                     double atol, double* max_abs_err, double* max_ratio, int64_t* first_bad) {
  fmt_t f = fmt_of(dtype);
  int64_t bad = 0;
  double mae = 0.0, mr = 0.0;
  *first_bad = -1;
  for (int64_t i = 0; i < n; ++i) {
    double g = decode16(got[i], f);
    double err = fabs(g - C[i]);
    double tol = rtol * fabs(C[i]) + atol;
    if (isnan(g) || isnan(err) || err > tol) {
      if (*first_bad < 0) *first_bad = i;
      ++bad;
    }
    if (!isnan(err)) {
      if (err > mae) mae = err;
      if (err / tol > mr) mr = err / tol;
    } else {
      mae = INFINITY;
      mr = INFINITY;
    }
  }
  *max_abs_err = mae;
  *max_ratio = mr;
  return bad;
}
