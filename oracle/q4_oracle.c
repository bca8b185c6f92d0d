/*
 * q4f16_1 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library. The product path (the HIP library) never does, and
 * the two share no code, header, table or helper.
 *
 * What is computed (the plain definitions, written out; slow on purpose):
 *
 *   q4f16_1 format -- Zero TVM documentation, section "Q4F16 quantization
 *   format": eight 4-bit codes per uint32; nibble i of a word is
 *   (word >> 4i) & 0xF; one fp16 scale per group of 32 weights; a weight is
 *   (code - 7) * scale.  Layout (the plainest reading of an [out][in] weight
 *   packed along the input axis): words[n][k/8] holds element k of row n in
 *   bits [4*(k%8), 4*(k%8)+3]; scales[n][k/32].
 *
 *   GEMV -- for every input row m and output row n:
 *       y[m][n] = sum_k (q[n][k] - 7) * s[n][k/32] * x[m][k].
 *
 *   MLP glue (orc_silu_mul) -- fp16(silu(gate) * up), see below.
 *
 * Two independent evaluations of that sum are provided:
 *   orc_gemv_f64   -- fp64 accumulation in ascending k; every product is exact
 *                     in fp64 (at most 4 + 11 + 11 significant bits), only the
 *                     additions round.
 *   orc_gemv_exact -- every finite fp16 value is an integer multiple of 2^-24,
 *                     so every term is an integer multiple of 2^-48 below 2^84
 *                     in magnitude; the sum is formed exactly in __int128 and
 *                     rounded once, to fp64 and to fp16 (round to nearest even).
 *
 * fp16 <-> fp64 conversions are written from the IEEE 754 binary16 definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0 is
 * zero/subnormal, exponent 31 is inf/NaN), bf16 -> fp64 from the bfloat16
 * definition.  Codes above 15 given to orc_pack are reduced to their low nibble.
 *
 * The GEMV row loops may run on several host threads (orc_set_threads; OpenMP
 * when built with -fopenmp): an OpenMP "parallel for" over output rows, each row
 * computed by the same steps, so the results are those of one thread.
 *
 * parity pins: see the CPU tests (closed forms, exact brute force, numpy
 * float16 conversions, byte-view nibble decoding, hand-worked fixtures).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------- binary16 */

ORC_EXPORT double orc_half_to_f64(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                /* subnormal: f * 2^-24      */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);    /* (1 + f/1024) * 2^(e - 15) */
  return sign ? -v : v;
}

/* bfloat16 from its definition: 1 sign bit, 8 exponent bits with bias 127, 7
 * fraction bits (the upper half of an IEEE 754 binary32); exponent 0 is
 * zero/subnormal, exponent 255 is inf/NaN. */
ORC_EXPORT double orc_bf16_to_f64(uint16_t h) {
  int sign = h >> 15, e = (h >> 7) & 255, f = h & 127;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);               /* subnormal: f * 2^-133     */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);    /* (1 + f/128) * 2^(e - 127) */
  return sign ? -v : v;
}

static int bitlen_u128(unsigned __int128 v) {
  int n = 0;
  while (v) { v >>= 1; ++n; }
  return n;
}

/* Round mag * 2^e2 to an integer multiple of 2^qe, ties to even; returns the
 * multiple (exact when e2 >= qe). */
static unsigned __int128 round_to_quantum(unsigned __int128 mag, int e2, int qe) {
  if (e2 >= qe) return mag << (e2 - qe);
  int shift = qe - e2;
  if (shift > 128) return 0;                       /* below half a quantum */
  unsigned __int128 r, rem, half;
  if (shift == 128) {
    r = 0; rem = mag; half = (unsigned __int128)1 << 127;
  } else {
    r = mag >> shift;
    rem = mag - (r << shift);
    half = (unsigned __int128)1 << (shift - 1);
  }
  if (rem > half || (rem == half && (r & 1))) ++r;
  return r;
}

/* Exactly rounded binary16 of (-1)^neg * mag * 2^e2 (overflow gives +-inf). */
static uint16_t exact_to_half(int neg, unsigned __int128 mag, int e2) {
  uint16_t sbit = neg ? 0x8000 : 0;
  if (mag == 0) return sbit;
  int E = bitlen_u128(mag) - 1 + e2;               /* value in [2^E, 2^(E+1)) */
  int qe = E - 10 < -24 ? -24 : E - 10;            /* ulp of the result       */
  unsigned __int128 r = round_to_quantum(mag, e2, qe);
  if (r == 0) return sbit;
  if (r >= 2048) { r >>= 1; ++qe; }                /* rounding carried out    */
  if (r < 1024) return sbit | (uint16_t)r;         /* subnormal (qe == -24)   */
  int field = qe + 25;                             /* biased exponent         */
  if (field >= 31) return sbit | 0x7C00;
  return sbit | (uint16_t)(field << 10) | (uint16_t)(r - 1024);
}

/* Exactly rounded fp64 of (-1)^neg * mag * 2^e2. */
static double exact_to_f64(int neg, unsigned __int128 mag, int e2) {
  if (mag == 0) return neg ? -0.0 : 0.0;
  int E = bitlen_u128(mag) - 1 + e2;
  int qe = E - 52 < -1074 ? -1074 : E - 52;
  unsigned __int128 r = round_to_quantum(mag, e2, qe);
  double v = ldexp((double)(uint64_t)r, qe);       /* r <= 2^53: exact */
  return neg ? -v : v;
}

ORC_EXPORT uint16_t orc_f64_to_half(double v) {
  if (isnan(v)) return 0x7E00;
  int neg = signbit(v) ? 1 : 0;
  if (isinf(v)) return neg ? 0xFC00 : 0x7C00;
  double a = fabs(v);
  if (a == 0.0) return neg ? 0x8000 : 0;
  int ex;
  double fr = frexp(a, &ex);                       /* a = fr * 2^ex, fr in [0.5, 1) */
  uint64_t m = (uint64_t)ldexp(fr, 53);            /* exact 53-bit integer          */
  return exact_to_half(neg, (unsigned __int128)m, ex - 53);
}

/* fp16 value as an integer multiple of 2^-24; returns 0 for inf / NaN. */
static int half_to_fixed24(uint16_t h, int64_t* out) {
  int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  if (e == 31) return 0;
  int64_t v = e == 0 ? (int64_t)f : (int64_t)(1024 + f) << (e - 1);
  *out = sign ? -v : v;
  return 1;
}

/* ------------------------------------------------------------------- codec */

static inline unsigned code_at(const uint32_t* words, int64_t K, int64_t n, int64_t k) {
  uint32_t w = words[n * (K / 8) + k / 8];
  return (w >> (4 * (k % 8))) & 0xFu;
}

ORC_EXPORT void orc_unpack(const uint32_t* words, uint8_t* codes, int64_t N, int64_t K) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      codes[n * K + k] = (uint8_t)code_at(words, K, n, k);
}

ORC_EXPORT void orc_pack(const uint8_t* codes, uint32_t* words, int64_t N, int64_t K) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K / 8; ++j) {
      uint32_t w = 0;
      for (int i = 0; i < 8; ++i)
        w |= (uint32_t)(codes[n * K + 8 * j + i] & 0xFu) << (4 * i);
      words[n * (K / 8) + j] = w;
    }
}

/* Counts words w in [w0, w1) (w1 <= 2^32) for which pack(unpack(w)) != w. */
ORC_EXPORT int64_t orc_roundtrip_mismatches(uint64_t w0, uint64_t w1) {
  int64_t bad = 0;
  for (uint64_t v = w0; v < w1; ++v) {
    uint32_t w = (uint32_t)v, back;
    uint8_t c[8];
    orc_unpack(&w, c, 1, 8);
    orc_pack(c, &back, 1, 8);
    bad += back != w;
  }
  return bad;
}

/* -------------------------------------------------------------------- GEMV */

/* Threads the row loops below run on (OpenMP, when the library is built with it):
 * 1 by default, the plain single-threaded oracle.  Rows are independent and each
 * is computed by exactly the same steps whatever the thread count, so results
 * do not depend on it. */
static int g_threads = 1;

ORC_EXPORT void orc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
ORC_EXPORT int orc_get_threads(void) { return g_threads; }

/* Y[m][i] = sum_k (q[n][k] - 7) * s[n][k/32] * X[m][k], n = rows[i] (or i when
 * rows is NULL), accumulated in fp64 in ascending k.  X is [M][K], Y is
 * [M][n_rows].  Returns 0, or -1 on a bad shape. */
ORC_EXPORT int orc_gemv_f64(const uint32_t* words, const uint16_t* scales, const uint16_t* X,
                            int64_t M, int64_t N, int64_t K, const int64_t* rows,
                            int64_t n_rows, double* Y) {
  if (M < 1 || N < 1 || K < 32 || K % 32) return -1;
  for (int64_t i = 0; i < n_rows; ++i)
    if ((rows ? rows[i] : i) < 0 || (rows ? rows[i] : i) >= N) return -1;
  double* x = (double*)malloc(sizeof(double) * (size_t)K);
  if (!x) return -1;
  int bad = 0;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t k = 0; k < K; ++k) x[k] = orc_half_to_f64(X[m * K + k]);
#pragma omp parallel num_threads(g_threads) reduction(| : bad)
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)(K / 32));
      bad |= !s;
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < n_rows; ++i) {
        if (!s) continue;
        int64_t n = rows ? rows[i] : i;
        for (int64_t g = 0; g < K / 32; ++g) s[g] = orc_half_to_f64(scales[n * (K / 32) + g]);
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          int q = (int)code_at(words, K, n, k);
          acc += ((double)(q - 7) * s[k / 32]) * x[k];
        }
        Y[m * n_rows + i] = acc;
      }
      free(s);
    }
  }
  free(x);
  return bad ? -1 : 0;
}

/* Exact evaluation of the same sum in __int128 (units of 2^-48), rounded once
 * to fp64 (Y64) and to fp16 (Y16; either may be NULL).  Returns 0, -1 on a bad
 * shape, -2 if an input is inf or NaN. */
ORC_EXPORT int orc_gemv_exact(const uint32_t* words, const uint16_t* scales, const uint16_t* X,
                              int64_t M, int64_t N, int64_t K, const int64_t* rows,
                              int64_t n_rows, double* Y64, uint16_t* Y16) {
  if (M < 1 || N < 1 || K < 32 || K % 32 || K > (1 << 20)) return -1;
  for (int64_t i = 0; i < n_rows; ++i)
    if ((rows ? rows[i] : i) < 0 || (rows ? rows[i] : i) >= N) return -1;
  int bad = 0;
  for (int64_t m = 0; m < M; ++m) {
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 16) reduction(| : bad)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t n = rows ? rows[i] : i;
      __int128 acc = 0;
      int finite = 1;
      for (int64_t k = 0; k < K && finite; ++k) {
        int64_t sv, xv;
        finite = half_to_fixed24(scales[n * (K / 32) + k / 32], &sv) &&
                 half_to_fixed24(X[m * K + k], &xv);
        if (!finite) break;
        int q = (int)code_at(words, K, n, k);
        acc += (__int128)(q - 7) * (__int128)sv * (__int128)xv;
      }
      if (!finite) {
        bad = 1;
        continue;
      }
      int neg = acc < 0;
      unsigned __int128 mag = neg ? (unsigned __int128)(-acc) : (unsigned __int128)acc;
      if (Y64) Y64[m * n_rows + i] = exact_to_f64(neg, mag, -48);
      if (Y16) Y16[m * n_rows + i] = exact_to_half(neg, mag, -48);
    }
  }
  return bad ? -2 : 0;
}

/* ||W_n||_2 with W_n[k] = (q[n][k] - 7) * s[n][k/32], for n = rows[i]. */
ORC_EXPORT int orc_row_norms(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                             const int64_t* rows, int64_t n_rows, double* out) {
  if (N < 1 || K < 32 || K % 32) return -1;
  for (int64_t i = 0; i < n_rows; ++i)
    if ((rows ? rows[i] : i) < 0 || (rows ? rows[i] : i) >= N) return -1;
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 16)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t n = rows ? rows[i] : i;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double w = (double)((int)code_at(words, K, n, k) - 7) *
                 orc_half_to_f64(scales[n * (K / 32) + k / 32]);
      acc += w * w;
    }
    out[i] = sqrt(acc);
  }
  return 0;
}

/* ---------------------------------------------------------------- MLP glue */

/* The step between the gate/up projection and the down projection of the
 * decode loop's feed-forward block (Zero TVM documentation, section "Decode
 * loop": gate, up, SiLU, multiply and down form the FFN).  GU is [M][2H] fp16:
 * gate = GU[m][0 .. H), up = GU[m][H .. 2H) (the fp16 outputs of the gate/up
 * GEMV).  For every m, i:
 *     g = gate[m][i], u = up[m][i],
 *     silu(g) = g / (1 + exp(-g)),
 *     OUT[m][i] = fp16_rne(silu(g) * u),
 * evaluated in fp64 (the fp16 inputs are exact in fp64).  silu(+inf) = +inf,
 * silu(-inf) = -0 (its limits); NaN propagates. */
ORC_EXPORT void orc_silu_mul(const uint16_t* GU, uint16_t* OUT, int64_t M, int64_t H) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t i = 0; i < H; ++i) {
      double g = orc_half_to_f64(GU[m * 2 * H + i]);
      double u = orc_half_to_f64(GU[m * 2 * H + H + i]);
      double sg;
      if (isinf(g))
        sg = g > 0 ? g : -0.0;
      else
        sg = g / (1.0 + exp(-g));
      OUT[m * H + i] = orc_f64_to_half(sg * u);
    }
}

/* ---------------------------------------------------------- other formats */

/* The format variants of the everything-webgpu AI.md quantization table and of
 * the MLX checkpoints the Zero TVM documentation loads, each as a plain decode:
 *   format 1, q3f16_1: 12 bytes of codes + an fp16 scale per 32 weights; the
 *     group's 32 codes are the 3-bit fields [3i, 3i + 3) of its three
 *     little-endian words taken as one 96-bit value; weight = (q - 3) * s.
 *   format 2, q4f32_1: q4f16_1's codes with fp32 scales; x and y fp32.
 *   format 3, MLX affine 4-bit, group 64 (af4g64): q4f16_1's nibble order, a
 *     bf16 scale and a bf16 bias per 64 weights; weight = s * q + b (Splash
 *     docs/models.md, "MLX targets": an affine weight is s * q + z for its
 *     group's bf16 .scales and .biases, codes packed little-endian in 32-bit
 *     words; Zero TVM documentation: affine w = s*q + b, group 64).
 *   format 4, the same with fp16 scales and biases (an extra variant, not the
 *     pages' format).
 * W[n][k] for one element, in fp64. */
static double fmt_weight(int format, const uint32_t* words, const void* scales,
                         const void* biases, int64_t K, int64_t n, int64_t k) {
  if (format == 1) {
    const int64_t g = k / 32, i = k % 32;
    const uint32_t* w = words + n * (K / 32) * 3 + g * 3;
    unsigned q = 0;
    for (int b = 0; b < 3; ++b) {
      const int64_t bit = 3 * i + b;
      q |= ((w[bit / 32] >> (bit % 32)) & 1u) << b;
    }
    const double s = orc_half_to_f64(((const uint16_t*)scales)[n * (K / 32) + g]);
    return ((double)q - 3.0) * s;
  }
  const unsigned q = code_at(words, K, n, k);
  if (format == 2) {
    const float s = ((const float*)scales)[n * (K / 32) + k / 32];
    return ((double)q - 7.0) * (double)s;
  }
  const uint16_t sh = ((const uint16_t*)scales)[n * (K / 64) + k / 64];
  const uint16_t bh = ((const uint16_t*)biases)[n * (K / 64) + k / 64];
  const double s = format == 3 ? orc_bf16_to_f64(sh) : orc_half_to_f64(sh);
  const double b = format == 3 ? orc_bf16_to_f64(bh) : orc_half_to_f64(bh);
  return s * (double)q + b;
}

/* Y[i] = sum_k W[n][k] * x[k] (n = rows[i], or i when rows is NULL), fp64, k
 * ascending; x is fp16 bits (formats 1, 3, 4) or fp32 (format 2).  Also the row
 * norms ||W_n||_2 into NORMS when not NULL.  Returns 0, or -1 on a bad shape. */
ORC_EXPORT int orc_gemv_format(int format, const uint32_t* words, const void* scales,
                               const void* biases, const void* X, int64_t N, int64_t K,
                               const int64_t* rows, int64_t n_rows, double* Y, double* NORMS) {
  if (format < 1 || format > 4 || N < 1 || K < 32 || K % 32 || (format >= 3 && K % 64))
    return -1;
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t n = rows ? rows[i] : i;
    if (n < 0 || n >= N) return -1;
    double acc = 0.0, nn = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double w = fmt_weight(format, words, scales, biases, K, n, k);
      const double x = format == 2 ? (double)((const float*)X)[k]
                                   : orc_half_to_f64(((const uint16_t*)X)[k]);
      acc += w * x;
      nn += w * w;
    }
    Y[i] = acc;
    if (NORMS) NORMS[i] = sqrt(nn);
  }
  return 0;
}

/* ------------------------------------------------ the rest of a decode step */

/* The steps of the decode loop around its GEMVs (Zero TVM documentation,
 * "Decode loop"): the token's embedding row, RMSNorm, the residual add fused with
 * RMSNorm ("addNorm"), and the argmax over the LM head's logits. */

/* OUT[m][k] = fp16((q[t][k] - 7) * s[t][k/32]) with t = TOK[m], the embedding
 * table being a q4f16_1 matrix [N][K] (one row per token); a token outside
 * [0, N) gives a row of NaN. */
ORC_EXPORT void orc_embed_rows(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                               const int32_t* TOK, int64_t M, uint16_t* OUT) {
  for (int64_t m = 0; m < M; ++m) {
    const int64_t t = TOK[m];
    for (int64_t k = 0; k < K; ++k) {
      if (t < 0 || t >= N) {
        OUT[m * K + k] = 0x7E00;
        continue;
      }
      double w = (double)((int)code_at(words, K, t, k) - 7) *
                 orc_half_to_f64(scales[t * (K / 32) + k / 32]);
      OUT[m * K + k] = orc_f64_to_half(w);
    }
  }
}

/* RMSNorm of fp16 rows: OUT[m][k] = fp16(X[m][k] / sqrt(mean_k X[m][k]^2 + eps)
 * * GAMMA[k]), in fp64. */
ORC_EXPORT void orc_rmsnorm(const uint16_t* X, const uint16_t* GAMMA, double eps, int64_t M,
                            int64_t K, uint16_t* OUT) {
  for (int64_t m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double v = orc_half_to_f64(X[m * K + k]);
      ss += v * v;
    }
    double r = 1.0 / sqrt(ss / (double)K + eps);
    for (int64_t k = 0; k < K; ++k)
      OUT[m * K + k] = orc_f64_to_half(orc_half_to_f64(X[m * K + k]) * r *
                                       orc_half_to_f64(GAMMA[k]));
  }
}

/* The residual add and RMSNorm: RES_OUT = fp16(RES_IN + DELTA) (the exact sum
 * rounded once), OUT = RMSNorm(RES_OUT) as orc_rmsnorm. */
ORC_EXPORT void orc_add_rmsnorm(const uint16_t* DELTA, const uint16_t* RES_IN,
                                const uint16_t* GAMMA, double eps, int64_t M, int64_t K,
                                uint16_t* RES_OUT, uint16_t* OUT) {
  for (int64_t i = 0; i < M * K; ++i)
    RES_OUT[i] = orc_f64_to_half(orc_half_to_f64(RES_IN[i]) + orc_half_to_f64(DELTA[i]));
  orc_rmsnorm(RES_OUT, GAMMA, eps, M, K, OUT);
}

/* OUT[m] = the index of the largest value of row m of X [M][N] (fp16); ties go to
 * the lowest index; NaN entries are skipped (a row of NaN gives 0). */
ORC_EXPORT void orc_argmax(const uint16_t* X, int64_t M, int64_t N, int32_t* OUT) {
  for (int64_t m = 0; m < M; ++m) {
    int64_t best = -1;
    double bv = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double v = orc_half_to_f64(X[m * N + n]);
      if (isnan(v)) continue;
      if (best < 0 || v > bv) {
        best = n;
        bv = v;
      }
    }
    OUT[m] = (int32_t)(best < 0 ? 0 : best);
  }
}

/* ||x||_2 of an fp16 vector. */
ORC_EXPORT double orc_vec_norm(const uint16_t* x, int64_t K) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double v = orc_half_to_f64(x[k]);
    acc += v * v;
  }
  return sqrt(acc);
}
