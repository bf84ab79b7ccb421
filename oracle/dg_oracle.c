/*
 * dg_oracle.c - plain, slow CPU oracle for the FP8 (e4m3) block-scaled GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no code, header, table or constant generator with the HIP path.
 *
 * What it computes, and where the pages state it:
 *  - FP8 e4m3 with one fp32 scale per 128 consecutive activation elements of a row
 *    ("1x128") and one per 128x128 weight block: DeepGEMM article, section
 *    "FP8 and fine-grained scaling" (activations scaled per slice, weights per matrix
 *    block); DeepSeek-V3 repo review, "Innovations" item 4 (one scale per 128
 *    elements, quant / dequant / GEMM trio) and "Solution philosophy" (128x128 block
 *    scaling).
 *  - The quantisation bound 448: DeepSeek-V3 repo review, "Risks and shortcomings"
 *    item 6. 448 is the largest finite value of OCP E4M3FN (the "fn" variant), which
 *    fixes the format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 *    exponent 0 subnormal, no infinities, S.1111.111 is NaN.
 *  - Two-level accumulation: an FP8 product sum over a stretch of K, then promotion
 *    to fp32 and scaled accumulation: DeepGEMM launch write-up, sections
 *    "Built for modern AI compute" and "Deployment guide".
 *
 * Readings where the pages say nothing (each is listed in the design notes):
 *  - scale s = amax / 448 (the dequantisation factor), q = e4m3(x / s); the GEMM
 *    multiplies its block sums by s_a * s_b;
 *  - rounding: round to nearest, ties to the even code; saturation to +-448 (the
 *    format has no infinity);
 *  - division x / s is a correctly rounded fp32 division, not a reciprocal multiply;
 *  - an all-zero chunk (or one whose s underflows to 0) stores s = 0 and signed zeros;
 *  - the sign of zero is kept;
 *  - the promotion interval is one 128-wide K block (the scale changes every 128 K);
 *  - power-of-two (UE8M0) scales, the variant the DeepSeek-V3 repo review names under
 *    "Innovations" item 4 (scales rounded to powers of two so that scaling is a shift):
 *    s = the smallest power of two not below fp32(amax / 448), and at least 2^-126 (the
 *    smallest normal fp32, so that s is never 0); q = e4m3(x / s), where the division is
 *    exact.
 *
 * The GEMM result R = sum_kb (s_a * s_b) * P_kb is kept in fp64. Each block sum P_kb is
 * exact in fp64: every e4m3 value is a multiple of 2^-9, so each product is a multiple
 * of 2^-18 and at most 448^2 < 2^18, and 128 of them stay below 2^25 - 43 bits in all.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -fPIC -shared -fno-fast-math -ffp-contract=off
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define QBLK 128 /* scale granularity: 128 K elements; 128x128 weight blocks */

/* ------------------------------------------------------------------------- */
/* e4m3 decode table, from the OCP E4M3FN definition                          */
/* ------------------------------------------------------------------------- */
static double g_dec[256];

static void build_dec_table(void) {
  for (int b = 0; b < 256; ++b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15; /* biased exponent */
    int m = b & 7;         /* mantissa */
    double v;
    if (e == 15 && m == 7) {
      v = NAN; /* S.1111.111 is the only NaN; there is no infinity */
    } else if (e == 0) {
      v = ldexp((double)m / 8.0, -6); /* subnormal: (m/8) * 2^(1-7) */
    } else {
      v = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: (1+m/8) * 2^(e-7) */
    }
    g_dec[b] = sign ? -v : v;
  }
}

__attribute__((constructor)) static void dgo_init(void) { build_dec_table(); }

void dgo_decode_table(double* out /*[256]*/) { memcpy(out, g_dec, sizeof g_dec); }

double dgo_decode(uint8_t code) { return g_dec[code]; }

/* ------------------------------------------------------------------------- */
/* Encoder 1: nearest table value (the plain definition)                     */
/* ------------------------------------------------------------------------- */
/* Non-negative finite codes 0x00..0x7E are strictly increasing in value. Take
 * |y| clamped to 448, find the bracketing pair t[c] <= a < t[c+1] by bisection,
 * compare a with the exact midpoint, and on a tie take the even code. */
uint8_t dgo_enc_nearest(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (isnan(a)) return (uint8_t)(sign | 0x7F); /* outside the precondition */
  if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate */
  int lo = 0, hi = 0x7E; /* invariant: t[lo] <= a < t[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_dec[mid] <= a) lo = mid; else hi = mid;
  }
  double midpoint = 0.5 * (g_dec[lo] + g_dec[hi]); /* exact: both are short dyadics */
  int c;
  if (a < midpoint) c = lo;
  else if (a > midpoint) c = hi;
  else c = (lo & 1) ? hi : lo; /* tie: the code whose mantissa LSB is 0 */
  return (uint8_t)(sign | c);
}

/* ------------------------------------------------------------------------- */
/* Encoder 2: fp32 bit arithmetic (an independent formulation, for cross-check) */
/* ------------------------------------------------------------------------- */
uint8_t dgo_enc_bits(float y) {
  uint32_t u;
  memcpy(&u, &y, 4);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  u &= 0x7FFFFFFFu;
  if (u > 0x7F800000u) return (uint8_t)(sign | 0x7F); /* NaN: outside the precondition */
  if (u >= 0x43E00000u) return (uint8_t)(sign | 0x7E); /* |y| >= 448 (incl. inf): saturate */
  if (u < 0x3C800000u) {
    /* |y| < 2^-6: e4m3 subnormal range, code = RNE(|y| * 2^9) in 0..8 */
    uint32_t e = u >> 23;
    uint32_t sig = (e ? 0x800000u : 0u) | (u & 0x7FFFFFu);
    int exp2 = (int)(e ? e : 1) - 127 - 23; /* |y| = sig * 2^exp2 */
    int shift = -(exp2 + 9);                /* |y| * 2^9 = sig >> shift */
    if (shift >= 26) return sign;           /* below 2^-11: rounds to zero */
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return (uint8_t)(sign | q);
  }
  /* normal range: keep 3 of fp32's 23 mantissa bits with round-half-even */
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  r >>= 20;                        /* (biased exp << 3) | mantissa, fp32 bias */
  uint32_t code = r - ((127u - 7u) << 3); /* rebias the exponent from 127 to 7 */
  if (code > 0x7Eu) code = 0x7Eu;
  return (uint8_t)(sign | code);
}

/* Count fp32 bit patterns in [lo, hi] (inclusive, finite ones only) on which the two
 * encoders disagree. */
int64_t dgo_enc_crosscheck(uint32_t lo, uint32_t hi) {
  int64_t bad = 0;
  int64_t n = (int64_t)hi - (int64_t)lo + 1;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)(lo + i);
    if ((u & 0x7F800000u) == 0x7F800000u) continue; /* inf / NaN */
    float y;
    memcpy(&y, &u, 4);
    if (dgo_enc_nearest(y) != dgo_enc_bits(y)) ++bad;
  }
  return bad;
}

void dgo_encode_array(const float* y, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = dgo_enc_nearest(y[i]);
}

/* ------------------------------------------------------------------------- */
/* Casts                                                                      */
/* ------------------------------------------------------------------------- */
/* The power-of-two scale of a group: the smallest power of two >= v = fp32(amax/448),
 * and >= 2^-126. Written with frexp: v = f * 2^e with f in [0.5, 1), so v is a power of
 * two exactly when f == 0.5. */
static float pow2_scale(float v) {
  if (!(v > 0x1p-126f)) return 0x1p-126f;
  int e;
  float f = frexpf(v, &e);
  return f == 0.5f ? v : ldexpf(1.0f, e);
}

/* Quantise one group of values (a 1x128 chunk or a 128x128 block) that share a
 * scale. `idx` lists the positions of the group's elements; pow2 selects power-of-two
 * scales. */
static float quant_group(const float* x, const int64_t* idx, int count, uint8_t* q, int pow2) {
  float amax = 0.0f;
  for (int i = 0; i < count; ++i) {
    float v = fabsf(x[idx[i]]);
    if (v > amax) amax = v;
  }
  float s = amax / 448.0f; /* correctly rounded fp32 division */
  if (pow2) s = pow2_scale(s);
  for (int i = 0; i < count; ++i) {
    float v = x[idx[i]];
    if (s == 0.0f) {
      q[idx[i]] = signbit(v) ? 0x80 : 0x00;
    } else {
      float y = v / s; /* correctly rounded fp32 division, not v * (1/s) */
      q[idx[i]] = dgo_enc_nearest(y);
    }
  }
  return s;
}

/* Per-token cast: x [M,K] fp32 row-major -> q [M,K] e4m3, s [M,K/128] fp32. */
static void cast_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s, int pow2) {
  int64_t nkb = K / QBLK;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    int64_t idx[QBLK];
    for (int64_t j = 0; j < nkb; ++j) {
      for (int i = 0; i < QBLK; ++i) idx[i] = m * K + j * QBLK + i;
      s[m * nkb + j] = quant_group(x, idx, QBLK, q, pow2);
    }
  }
}
void dgo_cast_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s) {
  cast_per_token(x, M, K, q, s, 0);
}
void dgo_cast_per_token_pow2(const float* x, int64_t M, int64_t K, uint8_t* q, float* s) {
  cast_per_token(x, M, K, q, s, 1);
}

/* Weight block cast: w [N,K] fp32 -> q [N,K] e4m3, s [N/128, K/128] fp32. */
static void cast_per_block(const float* w, int64_t N, int64_t K, uint8_t* q, float* s, int pow2) {
  int64_t nnb = N / QBLK, nkb = K / QBLK;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bn = 0; bn < nnb; ++bn) {
    for (int64_t bk = 0; bk < nkb; ++bk) {
      int64_t idx[QBLK * QBLK];
      int c = 0;
      for (int64_t r = 0; r < QBLK; ++r)
        for (int64_t k = 0; k < QBLK; ++k) idx[c++] = (bn * QBLK + r) * K + bk * QBLK + k;
      s[bn * nkb + bk] = quant_group(w, idx, QBLK * QBLK, q, pow2);
    }
  }
}
void dgo_cast_per_block(const float* w, int64_t N, int64_t K, uint8_t* q, float* s) {
  cast_per_block(w, N, K, q, s, 0);
}
void dgo_cast_per_block_pow2(const float* w, int64_t N, int64_t K, uint8_t* q, float* s) {
  cast_per_block(w, N, K, q, s, 1);
}

/* bf16 bit patterns -> fp32 (exact widening). */
void dgo_bf16_to_f32(const uint16_t* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)x[i] << 16;
    memcpy(&out[i], &u, 4);
  }
}

/* ------------------------------------------------------------------------- */
/* GEMM                                                                       */
/* ------------------------------------------------------------------------- */
/* P_kb = sum over one 128-wide K block of dec(a) * dec(b), in fp64 (exact). */
static double block_sum(const uint8_t* arow, const uint8_t* brow, int64_t kb) {
  double p = 0.0;
  for (int64_t k = kb * QBLK; k < (kb + 1) * QBLK; ++k) p += g_dec[arow[k]] * g_dec[brow[k]];
  return p;
}

/* One output element: R[m,n] = sum_kb (sa[m,kb] * sb[n/128,kb]) * P_kb. */
static double gemm_element(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                           int64_t m, int64_t n, int64_t K) {
  int64_t nkb = K / QBLK;
  const uint8_t* arow = a + m * K;
  const uint8_t* brow = b + n * K;
  double r = 0.0;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    double scale = (double)sa[m * nkb + kb] * (double)sb[(n / QBLK) * nkb + kb];
    r += scale * block_sum(arow, brow, kb);
  }
  return r;
}

/* Dense "NT" GEMM: a [M,K], b [N,K] (both K-major) -> R [M,N] fp64 = A * B^T. */
void dgo_gemm(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int64_t M,
              int64_t N, int64_t K, double* R) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) R[m * N + n] = gemm_element(a, sa, b, sb, m, n, K);
}

/* Selected output elements. Row m of `a` uses group g = group_of_row[m] (or 0 when the
 * pointer is NULL): b and sb are [G,N,K] and [G,N/128,K/128]. A row whose group lies
 * outside [0, G) (a padding row, -1) gets NaN, as in dgo_grouped_contiguous. */
void dgo_gemm_pairs(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                    const int32_t* group_of_row, int32_t G, int64_t N, int64_t K,
                    const int64_t* rows, const int64_t* cols, int64_t count, double* out) {
  int64_t bstride = N * K, sbstride = (N / QBLK) * (K / QBLK);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < count; ++i) {
    int64_t m = rows[i];
    int64_t g = group_of_row ? group_of_row[m] : 0;
    out[i] = (g < 0 || g >= G)
                 ? NAN
                 : gemm_element(a, sa, b + g * bstride, sb + g * sbstride, m, cols[i], K);
  }
}

/* Contiguous grouped GEMM: row r of a [M_total,K] belongs to expert m_indices[r]
 * (-1 = padding). Rows of experts get the dense result with that expert's weights;
 * padding rows are set to NaN (they are not compared). */
void dgo_grouped_contiguous(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                            const int32_t* m_indices, int32_t G, int64_t M_total, int64_t N,
                            int64_t K, double* R) {
  int64_t bstride = N * K, sbstride = (N / QBLK) * (K / QBLK);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < M_total; ++r) {
    for (int64_t n = 0; n < N; ++n) {
      int32_t g = m_indices[r];
      R[r * N + n] = (g < 0 || g >= G)
                         ? NAN
                         : gemm_element(a, sa, b + g * bstride, sb + g * sbstride, r, n, K);
    }
  }
}

/* Masked grouped GEMM: a [G,M_max,K]; expert g has min(max(masked_m[g],0),M_max) valid
 * rows. Valid rows get the dense result with expert g's weights; other rows are NaN
 * (the kernel must leave them untouched). */
void dgo_grouped_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                        const int32_t* masked_m, int32_t G, int64_t M_max, int64_t N, int64_t K,
                        double* R) {
  int64_t bstride = N * K, sbstride = (N / QBLK) * (K / QBLK);
  int64_t nkb = K / QBLK;
#pragma omp parallel for collapse(3) schedule(static)
  for (int64_t g = 0; g < G; ++g) {
    for (int64_t r = 0; r < M_max; ++r) {
      for (int64_t n = 0; n < N; ++n) {
        int64_t valid = masked_m[g] < 0 ? 0 : (masked_m[g] > M_max ? M_max : masked_m[g]);
        int64_t row = g * M_max + r;
        R[row * N + n] = r >= valid ? NAN
                                    : gemm_element(a + g * M_max * K, sa + g * M_max * nkb,
                                                   b + g * bstride, sb + g * sbstride, r, n, K);
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Hooks used by the oracle's own pins                                        */
/* ------------------------------------------------------------------------- */
/* The fp64 block sums the GEMM uses: P [M,N,K/128]. */
void dgo_block_sums(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                    double* P) {
  int64_t nkb = K / QBLK;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t kb = 0; kb < nkb; ++kb)
        P[(m * N + n) * nkb + kb] = block_sum(a + m * K, b + n * K, kb);
}

int dgo_num_threads(void) { return omp_get_max_threads(); }
void dgo_set_num_threads(int n) { omp_set_num_threads(n); }
