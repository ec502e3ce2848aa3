/*
 * attn_oracle.c -- fp64 CPU oracle for the scaled-dot-product attention
 * forward pass.  TEST INFRASTRUCTURE ONLY: this file is built into
 * oracle/liboracle.so and may be used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares
 * no code, header or constant with the HIP library.
 *
 * What it computes (the plain three-step definition, not the streaming
 * algorithm; the streaming algorithm reaches the same value up to rounding):
 *
 *   for every batch b, query head h and query row i, with the key/value head
 *   g = floor(h / (Hq / Hkv))  (grouped-query attention: each key/value head
 *   is repeated for Hq/Hkv consecutive query heads, the grouped-head fallback
 *   the SyclKittens summary, section E.1, describes as the GQA baseline),
 *
 *   1. scores   s_j = scale * sum_d Q[b,h,i,d] * K[b,g,j,d]      j < Lk
 *   2. softmax  p_j = exp(s_j - m) / sum_k exp(s_k - m),  m = max_j s_j
 *   3. output   O[b,h,i,:] = sum_j p_j * V[b,g,j,:]
 *   4. LSE[b,h,i] = m + ln(sum_j exp(s_j - m))     (natural logarithm)
 *
 * Steps 1-3 follow the data flow of "Xe2 Sdp Bf16", section "Kernel
 * Architecture: bf16io", data-flow diagram (QK product, softmax in fp32,
 * weighted sum of V, normalisation by the reciprocal of the row sum); the
 * "Xe2 ... Flash Attention -- HD=256" page, header, fixes the GQA shape
 * (32 query heads over 2 key/value heads).  The pages never mention the
 * log-sum-exp; step 4 is its textbook definition (natural log, scale
 * included).  Subtracting m in step 2 is exact algebra for stability, not a
 * step of the online softmax.
 *
 * Causal masking (optional).  Query row i sees key j only if
 * j <= i + (Lk - Lq): the diagonal is aligned to the end of both sequences, so
 * the Lq queries are read as the last Lq positions of a sequence whose first
 * Lk positions are the keys.  The SyclKittens summary (sections B.1.2, E.4,
 * E.6) names partial-tile causal masking and causal runs with as few as 8
 * query rows against long key sequences, for which only this alignment gives
 * every query a key; with Lq = Lk it is the usual lower-triangular mask.  The
 * pages do not spell the alignment out; this is the reading taken.  A row that
 * sees no key at all (possible only when Lq > Lk) has an empty sum: its output
 * is 0 and its LSE is ln 0 = -inf.
 *
 * Key ranges (optional).  K and V may hold a slice [key_begin, key_begin + Lk)
 * of a longer key sequence of length lk_total: the causal test then uses the
 * slice's global key index, and the result is the attention of each row over
 * the keys of the slice alone -- the partial result that, merged by LSE with
 * the partials over the other slices, gives the full one.
 *
 * Precision: every product and sum is fp64.  16-bit inputs are widened
 * exactly to double first ("Xe2 Sdp Bf16", section "Correctness Testing",
 * "CPU reference must match input type": the reference consumes the same
 * type-quantised values the kernel reads).  Outputs are left unrounded.
 *
 * Layouts: Q [B,Hq,Lq,D], K and V [B,Hkv,Lk,D], row-major, D fastest.
 * A selected row is the flat index (b*Hq + h)*Lq + i.
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

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Exact. */
double oracle_f16_to_double(uint16_t bits) {
  const int sign = (bits >> 15) & 1;
  const int expo = (bits >> 10) & 0x1f;
  const int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + frac), expo - 25); /* (1.frac) * 2^(e-15) */
  }
  return sign ? -mag : mag;
}

/* bfloat16 -> double: bfloat16 is the upper half of an IEEE binary32.  Exact. */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double widen(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? oracle_bf16_to_double(bits) : oracle_f16_to_double(bits);
}

/* One query row against the first nvis keys of one key/value head (nvis <= Lk
 * of the slice; nvis = Lk without causal masking).  e is caller scratch. */
static void attend_row(const double* qrow, const double* K, const double* V, int64_t nvis,
                       int64_t D, double scale, double* orow, double* lse, double* e) {
  for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
  if (nvis <= 0) { /* no key visible: empty sum */
    *lse = -INFINITY;
    return;
  }
  /* step 1: scores */
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    const double* kj = K + j * D;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qrow[d] * kj[d];
    e[j] = scale * dot;
    if (e[j] > m) m = e[j];
  }
  /* step 2: softmax weights (unnormalised) and their sum */
  double sum = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    e[j] = exp(e[j] - m);
    sum += e[j];
  }
  /* step 3: weighted sum of value rows, normalised */
  for (int64_t j = 0; j < nvis; ++j) {
    const double p = e[j] / sum;
    const double* vj = V + j * D;
    for (int64_t d = 0; d < D; ++d) orow[d] += p * vj[d];
  }
  /* step 4: log-sum-exp of the scaled scores */
  *lse = m + log(sum);
}

/* Keys of the slice visible to query row i. */
static int64_t visible_keys(int64_t i, int64_t Lq, int64_t Lk, int causal, int64_t key_begin,
                            int64_t lk_total) {
  if (!causal) return Lk;
  /* last visible global key index: i + lk_total - Lq */
  const int64_t n = i + (lk_total - Lq) - key_begin + 1;
  return n < 0 ? 0 : (n > Lk ? Lk : n);
}

static int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                       int causal, int64_t key_begin, int64_t lk_total) {
  /* Zero batches, heads or query rows: no row to compute.  Zero keys: every row sees
     none (O = 0, LSE = -inf, as for a causal row before the first key). */
  if (B < 0 || Hq < 0 || Hkv <= 0 || Lq < 0 || Lk < 0 || D <= 0) return -2;
  if (Hq % Hkv != 0) return -4;
  if (causal != 0 && causal != 1) return -11;
  if (key_begin < 0 || lk_total < key_begin + Lk) return -12;
  return 0;
}

static int run_rows(const double* q /* NULL: use q16 */, const uint16_t* q16, int dtype,
                    const double* K, const double* V, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Lq, int64_t Lk, int64_t D, double scale, int causal,
                    int64_t key_begin, int64_t lk_total, const int64_t* rows, int64_t nrows,
                    double* o_out, double* lse_out, int nthreads) {
  const int64_t G = Hq / Hkv;
  const int64_t total = B * Hq * Lq;
  int bad = 0;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t flat = rows ? rows[r] : r;
    if (flat < 0 || flat >= total) bad = 1;
  }
  if (bad) return -9;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int oom = 0;
  /* rows in runs of four (neighbouring rows share their key/value head in cache), one at a
     time when there are too few rows to keep every thread busy that way */
#ifdef _OPENMP
  const int chunk = nrows >= 16 * (int64_t)omp_get_max_threads() ? 4 : 1;
#endif
#pragma omp parallel
  {
    double* e = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!e || !qrow) {
#pragma omp atomic write
      oom = 1;
    } else {
#pragma omp for schedule(dynamic, chunk)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t i = flat % Lq;
        const int64_t h = (flat / Lq) % Hq;
        const int64_t b = flat / (Lq * Hq);
        const int64_t g = h / G; /* grouped-query head map */
        if (q) {
          memcpy(qrow, q + flat * D, sizeof(double) * (size_t)D);
        } else {
          for (int64_t d = 0; d < D; ++d) qrow[d] = widen(q16[flat * D + d], dtype);
        }
        const int64_t kv = (b * Hkv + g) * Lk * D;
        const int64_t nvis = visible_keys(i, Lq, Lk, causal, key_begin, lk_total);
        attend_row(qrow, K + kv, V + kv, nvis, D, scale, o_out + r * D, lse_out + r, e);
      }
    }
    free(e);
    free(qrow);
  }
  return oom ? -10 : 0;
}

/* fp64 inputs.  rows == NULL selects all B*Hq*Lq rows in order (nrows must
 * then equal that count).  o_out is nrows x D, lse_out is nrows.  causal is
 * 0 or 1; K and V hold keys [key_begin, key_begin + Lk) of a sequence of
 * lk_total keys (0 and Lk for the whole sequence).
 * Returns 0, or a negative code for a bad shape / row index / allocation. */
int oracle_attn_rows_f64(const double* q, const double* k, const double* v, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         double scale, int causal, int64_t key_begin, int64_t lk_total,
                         const int64_t* rows, int64_t nrows, double* o_out, double* lse_out,
                         int nthreads) {
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, causal, key_begin, lk_total);
  if (rc) return rc;
  if (!rows && nrows != B * Hq * Lq) return -9;
  return run_rows(q, NULL, 0, k, v, B, Hq, Hkv, Lq, Lk, D, scale, causal, key_begin, lk_total,
                  rows, nrows, o_out, lse_out, nthreads);
}

/* 16-bit inputs (raw fp16 or bf16 bit patterns, dtype 0 or 1), widened
 * exactly to double before any arithmetic. */
int oracle_attn_rows_u16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         double scale, int causal, int64_t key_begin, int64_t lk_total,
                         const int64_t* rows, int64_t nrows, double* o_out, double* lse_out,
                         int nthreads) {
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, causal, key_begin, lk_total);
  if (rc) return rc;
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -5;
  if (!rows && nrows != B * Hq * Lq) return -9;
  const size_t nkv = (size_t)(B * Hkv * Lk * D);
  double* K = (double*)malloc(sizeof(double) * (nkv > 0 ? nkv : 1));
  double* V = (double*)malloc(sizeof(double) * (nkv > 0 ? nkv : 1));
  if (!K || !V) {
    free(K);
    free(V);
    return -10;
  }
#pragma omp parallel for schedule(static)
  for (int64_t x = 0; x < (int64_t)nkv; ++x) {
    K[x] = widen(k[x], dtype);
    V[x] = widen(v[x], dtype);
  }
  rc = run_rows(NULL, q, dtype, K, V, B, Hq, Hkv, Lq, Lk, D, scale, causal, key_begin, lk_total,
                rows, nrows, o_out, lse_out, nthreads);
  free(K);
  free(V);
  return rc;
}

/* Merge of partial results over disjoint key ranges.  o_parts is
 * [nparts][nrows][D], lse_parts [nparts][nrows]: part g of row r is the
 * attention of row r over key range g alone, with its log-sum-exp.  Since
 * exp(LSE_g) is that range's sum of exp(scores) and O_g its weighted average,
 * the whole row has
 *
 *   LSE = ln sum_g exp(LSE_g),   O = sum_g exp(LSE_g - LSE) * O_g,
 *
 * the merge of online-softmax state that the SyclKittens summary (section I,
 * context-parallel ring attention) applies after each key shard.  Parts with
 * LSE_g = -inf (no visible key) carry no weight; if every part is empty the
 * row is empty too: O = 0, LSE = -inf.  Computed around the largest LSE_g for
 * range, in fp64.  Returns 0 or a negative code for a bad size. */
int oracle_merge(const double* o_parts, const double* lse_parts, int64_t nparts, int64_t nrows,
                 int64_t D, double* o_out, double* lse_out) {
  if (nparts <= 0 || nrows < 0 || D <= 0) return -2;
  for (int64_t r = 0; r < nrows; ++r) {
    double top = -INFINITY;
    for (int64_t g = 0; g < nparts; ++g)
      if (lse_parts[g * nrows + r] > top) top = lse_parts[g * nrows + r];
    double* orow = o_out + r * D;
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    if (top == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int64_t g = 0; g < nparts; ++g) sum += exp(lse_parts[g * nrows + r] - top);
    const double lse = top + log(sum);
    for (int64_t g = 0; g < nparts; ++g) {
      const double w = exp(lse_parts[g * nrows + r] - lse);
      const double* og = o_parts + (g * nrows + r) * D;
      for (int64_t d = 0; d < D; ++d) orow[d] += w * og[d];
    }
    lse_out[r] = lse;
  }
  return 0;
}

/* Number of threads an OpenMP region of this library would use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
