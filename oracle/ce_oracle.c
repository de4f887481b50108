/*
 * ce_oracle.c -- float64 CPU reference for token-level softmax cross-entropy,
 * forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, constant or table
 * with the HIP library, and the library never calls it.
 *
 * What it computes.  The pages (PyPI "fms-acceleration-foak 0.7.4", list
 * "Fast Cross Entropy Triton Kernels"; fms-acceleration PR #79, section
 * "Improvements to Full Finetuning", where FastCrossEntropyLoss replaces the
 * model's loss) name a cross-entropy kernel but never print its formula, so
 * the oracle writes out the textbook definition of softmax cross-entropy of a
 * logit row x[0..V) against an integer label y:
 *
 *     m    = max_j x_j
 *     lse  = m + ln( sum_j exp(x_j - m) )            (log-sum-exp)
 *     p_j  = exp(x_j - lse)                           (softmax)
 *     l    = lse - x_y                                (per-token loss, nats)
 *     L    = (sum over valid rows of l) / n_valid     (token mean; fms-hf-tuning
 *            PR #280, "Early Version Of This Plugin": straight per-token
 *            averaging, `--loss_across_gpus mean token`)
 *     g_j  = (dloss / n_valid) * (p_j - [j == y])     (dL/dx times dloss)
 *
 * Rows whose label equals ignore_index contribute l = 0, g = +0 and do not
 * count in n_valid.  A label outside [0, V) that is not ignore_index is an
 * error: it is counted and reported to the caller.
 *
 * Precision.  Every element is widened exactly to double; all arithmetic is
 * double with libm exp/log/log1p; sums use Neumaier compensation in index
 * order, so results do not depend on the thread count.  The gradient is
 * rounded once from double to the logits' format, round-to-nearest-even,
 * with subnormals kept.
 *
 * One reformulation, for confident rows.  When p_y > 1/2, p_y - 1 and
 * lse - x_y lose digits to cancellation.  There the oracle uses the identity
 * 1 - p_y = sum_{j != y} p_j =: q (softmax sums to one), writing
 * g_y = -(dloss/n) * q and l = -log1p(-q).  Both are the same quantities,
 * computed without cancellation.
 *
 * Vocabulary chunking (PR #79 "TODO": chunked loss) does not change the
 * definition; ceo_chunked_lse() computes the per-chunk log-sum-exp merge
 *     lse = M + ln sum_c exp(lse_c - M),  M = max_c lse_c
 * so that tests can check that it equals the unchunked value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Format codes used by this file's own C interface. */
#define CEO_F32 0
#define CEO_BF16 1
#define CEO_F16 2

/* ---------------------------------------------------------------------- */
/* Exact widening of one stored element to double.                        */
/* ---------------------------------------------------------------------- */

static double widen_f16(uint16_t h) {
  int sign = h >> 15;
  int ex = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + man), ex - 25); /* (1 + man/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

static double widen_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double widen(const void* base, int dtype, int64_t i) {
  if (dtype == CEO_F32) return (double)((const float*)base)[i];
  if (dtype == CEO_BF16) return widen_bf16(((const uint16_t*)base)[i]);
  return widen_f16(((const uint16_t*)base)[i]);
}

/* ---------------------------------------------------------------------- */
/* Rounding double -> storage format, round to nearest, ties to even.     */
/* A format with p significand bits (leading bit included) and exponent   */
/* range [emin, emax] holds, near x, the multiples of 2^(e - p + 1) where */
/* e = max(floor(log2|x|), emin).  Dividing by that power of two is exact,*/
/* so nearbyint() (ties-to-even in the default mode) rounds correctly.    */
/* ---------------------------------------------------------------------- */

static double round_to_format(double x, int p, int emin, int emax) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e2;
  frexp(fabs(x), &e2); /* |x| = f * 2^e2, f in [0.5, 1) */
  int lead = e2 - 1;   /* exponent of the leading bit */
  if (lead < emin) lead = emin;
  double quantum = ldexp(1.0, lead - (p - 1));
  double r = nearbyint(x / quantum) * quantum;
  double largest = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (fabs(r) > largest) return copysign(INFINITY, x);
  return r;
}

static uint16_t encode_f16(double r) { /* r already representable in binary16 */
  uint16_t sign = signbit(r) ? 0x8000 : 0;
  double a = fabs(r);
  if (isnan(r)) return 0x7e00;
  if (isinf(a)) return sign | 0x7c00;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);
  int lead = e2 - 1;
  if (lead < -14) return sign | (uint16_t)(a * 16777216.0); /* a / 2^-24 */
  uint16_t man = (uint16_t)((ldexp(a, -lead) - 1.0) * 1024.0);
  return sign | (uint16_t)((lead + 15) << 10) | man;
}

static void store_rounded(void* base, int dtype, int64_t i, double x) {
  if (dtype == CEO_F32) {
    float f = (float)round_to_format(x, 24, -126, 127); /* exact */
    ((float*)base)[i] = f;
  } else if (dtype == CEO_BF16) {
    float f = (float)round_to_format(x, 8, -126, 127); /* exact in binary32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) u = 0x7fc00000u;
    ((uint16_t*)base)[i] = (uint16_t)(u >> 16);
  } else {
    ((uint16_t*)base)[i] = encode_f16(round_to_format(x, 11, -14, 15));
  }
}

/* ---------------------------------------------------------------------- */
/* Compensated (Neumaier) summation.                                      */
/* ---------------------------------------------------------------------- */

typedef struct {
  double s, c;
} ksum;

static void kadd(ksum* k, double v) {
  double t = k->s + v;
  if (fabs(k->s) >= fabs(v))
    k->c += (k->s - t) + v;
  else
    k->c += (v - t) + k->s;
  k->s = t;
}

static double kval(const ksum* k) { return k->s + k->c; }

/* ---------------------------------------------------------------------- */
/* Log-sum-exp of x[j0..j1) of one row.                                    */
/* ---------------------------------------------------------------------- */

static double slab_lse(const double* x, int64_t j0, int64_t j1) {
  double m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j)
    if (x[j] > m) m = x[j];
  ksum s = {0.0, 0.0};
  for (int64_t j = j0; j < j1; ++j) kadd(&s, exp(x[j] - m));
  return m + log(kval(&s));
}

/* ---------------------------------------------------------------------- */
/* Public C interface (called through ctypes by oracle/__init__.py).       */
/* ---------------------------------------------------------------------- */

/* Widen n stored elements to double. */
void ceo_widen(const void* src, int dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = widen(src, dtype, i);
}

/* Round n doubles to the storage format (RNE, subnormals kept). */
void ceo_round(const double* src, int64_t n, int dtype, void* dst) {
  for (int64_t i = 0; i < n; ++i) store_rounded(dst, dtype, i, src[i]);
}

/* Number of rows whose label is not ignore_index. */
int64_t ceo_count_valid(const int64_t* labels, int64_t n_rows, int64_t ignore_index) {
  int64_t n = 0;
  for (int64_t i = 0; i < n_rows; ++i) n += (labels[i] != ignore_index);
  return n;
}

/*
 * Per-row forward and backward for n_rows rows.
 *   logits   : n_rows rows of V elements in `dtype`, row i at element i*ld
 *   labels   : n_rows int64
 *   scale    : dloss / n_valid of the whole batch (the caller supplies it, so
 *              a sample of rows of a larger batch is computed exactly as in
 *              the full batch)
 *   lse      : out, n_rows doubles (computed for every row, ignored or not)
 *   loss     : out, n_rows doubles (0 for ignored rows, NaN for bad labels)
 *   grad     : out or NULL, n_rows*V elements in `dtype` (row-major, ld = V)
 *   grad64   : out or NULL, n_rows*V doubles before rounding
 * Returns the number of rows whose label is outside [0, V) and is not
 * ignore_index (their loss and gradient rows are NaN).
 */
int64_t ceo_rows(const void* logits, int64_t ld, int dtype, const int64_t* labels,
                 int64_t n_rows, int64_t V, int64_t ignore_index, double scale,
                 double* lse, double* loss, void* grad, double* grad64, int nthreads) {
  int64_t bad = 0;
  if (nthreads < 1) nthreads = 1;
  size_t esz = dtype == CEO_F32 ? 4 : 2;
#pragma omp parallel num_threads(nthreads) reduction(+ : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_rows; ++i) {
      const char* row = (const char*)logits + (size_t)i * (size_t)ld * esz;
      for (int64_t j = 0; j < V; ++j) x[j] = widen(row, dtype, j);
      double row_lse = slab_lse(x, 0, V);
      lse[i] = row_lse;
      int64_t y = labels[i];
      if (y == ignore_index) {
        loss[i] = 0.0;
        for (int64_t j = 0; j < V; ++j) g[j] = 0.0;
      } else if (y < 0 || y >= V) {
        bad += 1;
        loss[i] = NAN;
        for (int64_t j = 0; j < V; ++j) g[j] = NAN;
      } else {
        for (int64_t j = 0; j < V; ++j) g[j] = scale * exp(x[j] - row_lse);
        double p_y = exp(x[y] - row_lse);
        if (p_y > 0.5) {
          ksum q = {0.0, 0.0}; /* q = 1 - p_y, summed without cancellation */
          for (int64_t j = 0; j < V; ++j)
            if (j != y) kadd(&q, exp(x[j] - row_lse));
          loss[i] = -log1p(-kval(&q));
          g[y] = -scale * kval(&q);
        } else {
          loss[i] = row_lse - x[y];
          g[y] = scale * (p_y - 1.0);
        }
      }
      if (grad64)
        for (int64_t j = 0; j < V; ++j) grad64[(size_t)i * (size_t)V + (size_t)j] = g[j];
      if (grad)
        for (int64_t j = 0; j < V; ++j) store_rounded(grad, dtype, i * V + j, g[j]);
    }
    free(x);
    free(g);
  }
  return bad;
}

/* Token mean of the per-row losses over valid rows, in row order.
 * NaN when no row is valid (0/0). */
double ceo_mean(const double* loss, const int64_t* labels, int64_t n_rows, int64_t ignore_index) {
  ksum s = {0.0, 0.0};
  int64_t n = 0;
  for (int64_t i = 0; i < n_rows; ++i) {
    if (labels[i] == ignore_index) continue;
    kadd(&s, loss[i]);
    n += 1;
  }
  return kval(&s) / (double)n;
}

/* Log-sum-exp of one row computed per vocabulary chunk of width `chunk`
 * (the last chunk holds the remainder) and merged. */
double ceo_chunked_lse(const void* row, int dtype, int64_t V, int64_t chunk) {
  double* x = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  for (int64_t j = 0; j < V; ++j) x[j] = widen(row, dtype, j);
  if (chunk <= 0 || chunk > V) chunk = V;
  int64_t C = (V + chunk - 1) / chunk;
  double* part = (double*)malloc(sizeof(double) * (size_t)C);
  double M = -INFINITY;
  for (int64_t c = 0; c < C; ++c) {
    int64_t j1 = (c + 1) * chunk < V ? (c + 1) * chunk : V;
    part[c] = slab_lse(x, c * chunk, j1);
    if (part[c] > M) M = part[c];
  }
  ksum s = {0.0, 0.0};
  for (int64_t c = 0; c < C; ++c) kadd(&s, exp(part[c] - M));
  double r = M + log(kval(&s));
  free(part);
  free(x);
  return r;
}
