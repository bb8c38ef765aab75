/*
 * oracle.c -- plain, slow CPU oracle for the ternary-weight linear layer.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library. The HIP
 * library never links it, and it includes no header, table or helper of the
 * HIP library: every definition below is restated from the sources cited.
 *
 * Sources (web pages; cited by title and section):
 *  [ART]  "NInfer sm_89 fork" article (2kiu.com news 5424991),
 *         section 7 "int8 artifact": prefill GEMM activations quantised to
 *         int8 so both operands feed an integer tensor-core contraction;
 *         section 9, item 2 "ternary weights (Bonsai)": weights in
 *         {-1,0,+1}, one fp16 scale per 128 weights, prefill as an int8
 *         contraction, decode bandwidth bound.
 *  [TUNE] "NINFER ternary perf-tuning" notes (markdownregistry diff page),
 *         section 2 rung-map table (s8 rung for T >= 17) and section 4
 *         numeric gate (s8 is the rung that changes numerics; the other
 *         rungs are numerics-inert).
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *  - the scale groups run along K (the input dimension) of each output row;
 *  - bf16-activation rungs: x is used as given (no quantisation), the
 *    reference result is accumulated in fp64;
 *  - s8 rung: per token, absmax over K, scale = fl32(absmax / 127) (IEEE
 *    single division), code = clamp(round-half-even(fl32(x / scale)),
 *    -127, 127), absmax == 0 gives scale 0 and all-zero codes;
 *  - s8 output: y = fl32(scale_t * sum_g s[n][g] * acc[t][n][g]) with the
 *    sum and product evaluated exactly and rounded once to fp32;
 *  - rotated quantisation: per 1024-wide block, (1/32) times the Sylvester
 *    Hadamard matrix, evaluated as fp32 fast Walsh-Hadamard butterflies with
 *    strides 1, 2, ..., 512 in that order, then the s8 rule above (see
 *    oracle_rotate_f32).
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off (see
 * oracle/__init__.py). float arithmetic must be IEEE single precision with
 * no excess precision (x86-64 SSE2: FLT_EVAL_METHOD == 0).
 */
#include <fenv.h>
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "oracle needs IEEE single-precision float evaluation (FLT_EVAL_METHOD == 0)"
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_WEIGHT (-2)
#define ORACLE_ERR_NONFINITE (-3)

int oracle_version(void) { return 1; }

/* ---------------------------------------------------------------- decoding */

/* bfloat16 bit pattern -> float: the top 16 bits of an IEEE binary32. Exact. */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* IEEE binary16 bit pattern -> double, exact (written out from the format:
 * 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits). */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* The same value split into an integer significand and a power of two:
 * h = sign * m * 2^e exactly, m in [0, 2047]. Finite inputs only. */
static void half_to_int_pow2(uint16_t h, int64_t* m, int* e) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  int64_t mm;
  int ee;
  if (ex == 0) {
    mm = f;
    ee = -24;
  } else {
    mm = 1024 + f;
    ee = ex - 25;
  }
  *m = sign ? -mm : mm;
  *e = ee;
}

/* IEEE binary32 value -> sign * m * 2^e exactly, m < 2^24. Finite only. */
static void float_to_int_pow2(float x, int64_t* m, int* e) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  int sign = (u >> 31) & 1;
  int ex = (u >> 23) & 0xff;
  int64_t f = u & 0x7fffff;
  int64_t mm;
  int ee;
  if (ex == 0) {
    mm = f;
    ee = -149;
  } else {
    mm = (1 << 23) + f;
    ee = ex - 150;
  }
  *m = sign ? -mm : mm;
  *e = ee;
}

static int weight_ok(int8_t w) { return w == -1 || w == 0 || w == 1; }

/* ------------------------------------------------- bf16-activation rungs */

/*
 * y[t][n] = sum_g s[n][g] * sum_{k in group g} w[n][k] * x[t][k]
 *
 * x: bf16 bits [T][K]; w: int8 [N][K] in {-1,0,+1}; s: fp16 bits
 * [N][K/G]; y: double [T][N]. Group g covers k in [g*G, (g+1)*G)
 * ([ART] section 9 item 2: one scale per 128 consecutive weights; G is a
 * parameter because the small test case uses 64). Accumulation in fp64.
 */
int oracle_linear_bf16(const uint16_t* x, int64_t T, int64_t K, const int8_t* w,
                       const uint16_t* s, int64_t N, int64_t G, double* y) {
  if (T < 0 || K <= 0 || N < 0 || G <= 0 || K % G != 0) return ORACLE_ERR_ARGS;
  const int64_t NG = K / G;
  for (int64_t i = 0; i < N * K; ++i)
    if (!weight_ok(w[i])) return ORACLE_ERR_WEIGHT;
  for (int64_t i = 0; i < T * K; ++i)
    if (!isfinite(bf16_to_float(x[i]))) return ORACLE_ERR_NONFINITE;
  for (int64_t i = 0; i < N * NG; ++i)
    if (!isfinite(half_to_double(s[i]))) return ORACLE_ERR_NONFINITE;

  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xt = x + t * K;
    for (int64_t n = 0; n < N; ++n) {
      const int8_t* wn = w + n * K;
      double total = 0.0;
      for (int64_t g = 0; g < NG; ++g) {
        double inner = 0.0;
        for (int64_t k = g * G; k < (g + 1) * G; ++k)
          inner += (double)wn[k] * (double)bf16_to_float(xt[k]);
        total += half_to_double(s[n * NG + g]) * inner;
      }
      y[t * N + n] = total;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------- s8 rung */

/*
 * Per-token symmetric int8 quantisation of the activations ([ART] section 7
 * and section 9 item 2; [TUNE] section 4: the s8 rung's numeric shift is the
 * int8 activation quantisation error).
 *
 *   a_t      = max_k |x[t][k]|                      (exact in float)
 *   scale_t  = fl32(a_t / 127)                      (IEEE single division)
 *   q[t][k]  = clamp(rne(fl32(x[t][k] / scale_t)), -127, 127)
 *   a_t == 0 -> scale_t = 0, q[t][:] = 0
 *
 * rne is round-to-nearest, ties to even (nearbyintf in FE_TONEAREST).
 */
int oracle_quant_s8(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale) {
  if (T < 0 || K <= 0) return ORACLE_ERR_ARGS;
  for (int64_t i = 0; i < T * K; ++i)
    if (!isfinite(bf16_to_float(x[i]))) return ORACLE_ERR_NONFINITE;
  const int saved = fegetround();
  fesetround(FE_TONEAREST);
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xt = x + t * K;
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float v = fabsf(bf16_to_float(xt[k]));
      if (v > a) a = v;
    }
    if (a == 0.0f) {
      scale[t] = 0.0f;
      for (int64_t k = 0; k < K; ++k) q[t * K + k] = 0;
      continue;
    }
    const float sc = a / 127.0f;
    scale[t] = sc;
    for (int64_t k = 0; k < K; ++k) {
      const float ratio = bf16_to_float(xt[k]) / sc;
      float r = nearbyintf(ratio);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[t * K + k] = (int8_t)r;
    }
  }
  fesetround(saved);
  return ORACLE_OK;
}

/* ------------------------------------------------------ rotated activations */

/*
 * Blockwise Hadamard rotation of the activations. [ART] section 9 item 2:
 * the Hadamard rotation of the original ternary model is done inside the
 * activation quantisation, with no kernel of its own. [TUNE] section 6,
 * constants table: the rotation works on 1024-wide blocks of a token.
 *
 * Readings (the pages give neither the matrix nor the arithmetic):
 *  - per token and 1024-wide block of K, xr = (1/32) H x, H the Sylvester
 *    Hadamard matrix of order 1024, H[i][j] = (-1)^popcount(i & j); the
 *    factor 1/32 = 1/sqrt(1024) makes the rotation orthonormal;
 *  - evaluated in IEEE single precision as the textbook in-place fast
 *    Walsh-Hadamard transform: strides h = 1, 2, 4, ..., 512 in that order,
 *    every pair (i, i + h) with (i & h) == 0 becoming (u + v, u - v), one
 *    rounding each; then one multiply by 1/32 per element.
 * K must be a multiple of 1024. xr: float [T][K].
 */
#define ROT_BLOCK 1024

int oracle_rotate_f32(const uint16_t* x, int64_t T, int64_t K, float* xr) {
  if (T < 0 || K <= 0 || K % ROT_BLOCK != 0) return ORACLE_ERR_ARGS;
  for (int64_t i = 0; i < T * K; ++i)
    if (!isfinite(bf16_to_float(x[i]))) return ORACLE_ERR_NONFINITE;
  const int saved = fegetround();
  fesetround(FE_TONEAREST);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t b = 0; b < K / ROT_BLOCK; ++b) {
      const uint16_t* xb = x + t * K + b * ROT_BLOCK;
      float* z = xr + t * K + b * ROT_BLOCK;
      for (int i = 0; i < ROT_BLOCK; ++i) z[i] = bf16_to_float(xb[i]);
      for (int h = 1; h < ROT_BLOCK; h <<= 1) {
        for (int i = 0; i < ROT_BLOCK; ++i) {
          if (i & h) continue;
          const float u = z[i], v = z[i + h];
          z[i] = u + v;
          z[i + h] = u - v;
        }
      }
      for (int i = 0; i < ROT_BLOCK; ++i) z[i] = z[i] * 0.03125f;
    }
  }
  fesetround(saved);
  return ORACLE_OK;
}

/*
 * Rotated per-token int8 quantisation: the steps of oracle_quant_s8 applied
 * to the rotated fp32 activations xr of oracle_rotate_f32:
 *   a_t = max_k |xr[t][k]|;  scale_t = fl32(a_t / 127);
 *   q[t][k] = clamp(round-half-even(fl32(xr[t][k] / scale_t)), -127, 127);
 *   a_t == 0 gives scale_t = 0 and q[t][:] = 0.
 */
int oracle_quant_s8_rot(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale) {
  if (T < 0 || K <= 0 || K % ROT_BLOCK != 0) return ORACLE_ERR_ARGS;
  float* xr = (float*)malloc(sizeof(float) * (size_t)(T > 0 ? T * K : 1));
  if (!xr) return ORACLE_ERR_ARGS;
  const int rc = oracle_rotate_f32(x, T, K, xr);
  if (rc != ORACLE_OK) {
    free(xr);
    return rc;
  }
  const int saved = fegetround();
  fesetround(FE_TONEAREST);
  for (int64_t t = 0; t < T; ++t) {
    const float* v = xr + t * K;
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k)
      if (fabsf(v[k]) > a) a = fabsf(v[k]);
    if (a == 0.0f) {
      scale[t] = 0.0f;
      for (int64_t k = 0; k < K; ++k) q[t * K + k] = 0;
      continue;
    }
    const float sc = a / 127.0f;
    scale[t] = sc;
    for (int64_t k = 0; k < K; ++k) {
      float r = nearbyintf(v[k] / sc);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[t * K + k] = (int8_t)r;
    }
  }
  fesetround(saved);
  free(xr);
  return ORACLE_OK;
}

/*
 * Integer group accumulators of the s8 contraction:
 *   acc[t][n][g] = sum_{k in group g} q[t][k] * w[n][k]      (int32, exact)
 * Layout of acc: [T][N][K/G].
 */
int oracle_s8_acc(const int8_t* q, int64_t T, int64_t K, const int8_t* w, int64_t N,
                  int64_t G, int32_t* acc) {
  if (T < 0 || K <= 0 || N < 0 || G <= 0 || K % G != 0) return ORACLE_ERR_ARGS;
  const int64_t NG = K / G;
  for (int64_t i = 0; i < N * K; ++i)
    if (!weight_ok(w[i])) return ORACLE_ERR_WEIGHT;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t g = 0; g < NG; ++g) {
        int64_t sum = 0;
        for (int64_t k = g * G; k < (g + 1) * G; ++k)
          sum += (int64_t)q[t * K + k] * (int64_t)w[n * K + k];
        acc[(t * N + n) * NG + g] = (int32_t)sum;
      }
  return ORACLE_OK;
}

/*
 * Round sign * mag * 2^e to the nearest IEEE binary32, ties to even, with
 * gradual underflow and overflow to infinity. mag is an exact unsigned
 * integer. This is the "rounded once" of the s8 output definition.
 */
static float round_scaled_int_to_float(int negative, unsigned __int128 mag, int e) {
  if (mag == 0) return negative ? -0.0f : 0.0f;
  int top = 127;
  while (!((mag >> top) & 1)) --top; /* mag in [2^top, 2^(top+1)) */
  /* value exponent: 2^(top + e). Binary32 keeps 24 significant bits for
   * normal numbers (exponent >= -126); below that the last kept bit has
   * weight 2^-149. */
  int lsb_exp = top + e - 23; /* weight of the 24th significant bit */
  if (lsb_exp < -149) lsb_exp = -149;
  int shift = lsb_exp - e; /* drop this many low bits of mag */
  unsigned __int128 kept;
  if (shift <= 0) {
    kept = mag << (-shift); /* exact, no rounding */
  } else if (shift > 128) {
    kept = 0; /* below half of the smallest subnormal: rounds to zero */
  } else if (shift == 128) {
    const unsigned __int128 half = (unsigned __int128)1 << 127;
    kept = mag > half ? 1 : 0; /* a tie rounds to the even value 0 */
  } else {
    kept = mag >> shift;
    unsigned __int128 rem = mag - (kept << shift);
    unsigned __int128 half = (unsigned __int128)1 << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) kept += 1;
  }
  /* kept * 2^lsb_exp is the rounded magnitude; kept < 2^25 here. */
  double d = ldexp((double)(uint64_t)kept, lsb_exp); /* exact in double */
  if (d > (double)FLT_MAX) return negative ? -INFINITY : INFINITY;
  float f = (float)d; /* exact: d is representable in binary32 */
  return negative ? -f : f;
}

/*
 * s8 rung output:
 *   y[t][n] = fl32( scale_t * sum_g s[n][g] * acc[t][n][g] )
 * evaluated exactly in integer arithmetic (every input is an integer times a
 * power of two) and rounded once. q: int8 [T][K]; scale: float [T];
 * w: int8 [N][K]; s: fp16 bits [N][K/G]; y: float [T][N].
 */
int oracle_linear_s8(const int8_t* q, const float* scale, int64_t T, int64_t K,
                     const int8_t* w, const uint16_t* s, int64_t N, int64_t G, float* y) {
  if (T < 0 || K <= 0 || N < 0 || G <= 0 || K % G != 0) return ORACLE_ERR_ARGS;
  const int64_t NG = K / G;
  for (int64_t i = 0; i < N * K; ++i)
    if (!weight_ok(w[i])) return ORACLE_ERR_WEIGHT;
  for (int64_t i = 0; i < N * NG; ++i)
    if (!isfinite(half_to_double(s[i]))) return ORACLE_ERR_NONFINITE;
  for (int64_t t = 0; t < T; ++t)
    if (!isfinite(scale[t])) return ORACLE_ERR_NONFINITE;

  for (int64_t t = 0; t < T; ++t) {
    int64_t mt;
    int et;
    float_to_int_pow2(scale[t], &mt, &et);
    for (int64_t n = 0; n < N; ++n) {
      /* Every term s*acc = ms * acc * 2^es with es in [-24, 5]; shift all
       * terms to the common exponent -24: sum = S * 2^-24 with S an exact
       * integer. |ms| < 2^11, |acc| <= 127*G, shift <= 29, so for any
       * G, NG < 2^31 the sum and its product with mt < 2^24 stay far below
       * 2^127 and fit a signed 128-bit integer. */
      __int128 S = 0;
      for (int64_t g = 0; g < NG; ++g) {
        int64_t acc = 0;
        for (int64_t k = g * G; k < (g + 1) * G; ++k)
          acc += (int64_t)q[t * K + k] * (int64_t)w[n * K + k];
        int64_t ms;
        int es;
        half_to_int_pow2(s[n * NG + g], &ms, &es);
        S += ((__int128)ms * (__int128)acc) * ((__int128)1 << (es + 24));  /* es + 24 >= 0 */
      }
      __int128 P = S * (__int128)mt; /* |P| < 2^97 */
      int negative = P < 0;
      unsigned __int128 mag = (unsigned __int128)(negative ? -P : P);
      y[t * N + n] = round_scaled_int_to_float(negative, mag, et - 24);
    }
  }
  return ORACLE_OK;
}

/*
 * The same output in one fixed fp32 order (the canonical epilogue order):
 *   acc_f = 0; for g ascending: acc_f = fmaf((float)acc_g, (float)s_g, acc_f);
 *   y = acc_f * scale_t
 * Every step is one IEEE single rounding (fmaf rounds acc*s + acc_f once).
 * A kernel that keeps this order reproduces it bit for bit, and the GPU
 * tests hold such kernels to it bitwise; the gate of the s8 rung itself is
 * the 1e-6 relative distance from oracle_linear_s8.
 */
int oracle_linear_s8_fp32_ordered(const int8_t* q, const float* scale, int64_t T, int64_t K,
                                  const int8_t* w, const uint16_t* s, int64_t N, int64_t G,
                                  float* y) {
  if (T < 0 || K <= 0 || N < 0 || G <= 0 || K % G != 0) return ORACLE_ERR_ARGS;
  const int64_t NG = K / G;
  for (int64_t i = 0; i < N * K; ++i)
    if (!weight_ok(w[i])) return ORACLE_ERR_WEIGHT;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      float total = 0.0f;
      for (int64_t g = 0; g < NG; ++g) {
        int32_t acc = 0;
        for (int64_t k = g * G; k < (g + 1) * G; ++k)
          acc += (int32_t)q[t * K + k] * (int32_t)w[n * K + k];
        total = fmaf((float)acc, (float)half_to_double(s[n * NG + g]), total);
      }
      y[t * N + n] = total * scale[t];
    }
  return ORACLE_OK;
}

/* ------------------------------------------- packed layout v1 (reader) */

/*
 * Independent reader of the 2-bit packed weight layout "v1" (the layout is
 * this library's own format, not the pages'; its written specification is
 * restated here from the public header's prose, sharing no code with it):
 *
 *  - needs N % 16 == 0, K % 256 == 0, G in {64, 128};
 *  - 2-bit code per weight: 00 -> 0, 01 -> +1, 11 -> -1 (10 is invalid);
 *  - strip s = rows [16s, 16s+16), k-tile kt = columns [256kt, 256kt+256);
 *    tile (s, kt) is 1024 bytes at byte offset (s*KT + kt)*1024, KT = K/256;
 *  - inside a tile, lane L in [0,64) owns bytes [16L, 16L+16) read as four
 *    little-endian 32-bit words P[0..3];
 *  - weight (row 16s + r, column 256kt + kk), kk = 32m + 8g + 2d + h with
 *    m in [0,8), g in [0,4), d in [0,4), h in {0,1}: lane L = 16g + r,
 *    word P[m >> 1], j = 4*(m & 1) + d, and its code occupies the two bits
 *    starting at bit b = (h ? 30 : 14) - 2j (bit b+1 is the code's high bit);
 *  - scales (fp16 bits) re-laid as [s][kt][r][gi], gi in [0, 256/G):
 *    element ((s*KT + kt)*16 + r)*(256/G) + gi is scale[16s + r][kt*(256/G) + gi].
 *
 * Outputs w int8 [N][K] and s fp16 bits [N][K/G]. Returns ORACLE_ERR_WEIGHT
 * if a code 10 is found.
 */
int oracle_unpack_layout_v1(const uint8_t* codes, const uint16_t* scales_packed, int64_t N,
                            int64_t K, int64_t G, int8_t* w, uint16_t* s) {
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 256 != 0 || (G != 64 && G != 128))
    return ORACLE_ERR_ARGS;
  const int64_t KT = K / 256;
  const int64_t NG = K / G;
  const int64_t GPT = 256 / G; /* groups per k-tile */
  for (int64_t n = 0; n < N; ++n) {
    const int64_t st = n / 16, r = n % 16;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t kt = k / 256, kk = k % 256;
      const int64_t m = kk / 32, g = (kk / 8) % 4, d = (kk / 2) % 4, h = kk % 2;
      const int64_t lane = 16 * g + r;
      const int64_t word = m >> 1;
      const int64_t j = 4 * (m & 1) + d;
      const int64_t b = (h ? 30 : 14) - 2 * j;
      const uint8_t* tile = codes + (st * KT + kt) * 1024;
      const uint8_t* wp = tile + lane * 16 + word * 4;
      const uint32_t P = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                         ((uint32_t)wp[3] << 24);
      const uint32_t code = (P >> b) & 3u;
      int8_t v;
      if (code == 0)
        v = 0;
      else if (code == 1)
        v = 1;
      else if (code == 3)
        v = -1;
      else
        return ORACLE_ERR_WEIGHT;
      w[n * K + k] = v;
    }
    for (int64_t g = 0; g < NG; ++g) {
      const int64_t kt = g / GPT, gi = g % GPT;
      s[n * NG + g] = scales_packed[((st * KT + kt) * 16 + r) * GPT + gi];
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------- packed layout t5 (reader) */

/*
 * Independent reader of the base-3 packed weight layout "t5": five weights
 * per byte, the format of the "NInfer sm_89 fork" article, section 9 item 2
 * ("t5" ternary: 5 trits per byte, one fp16 scale per 128 weights), laid out
 * by this library for the integer matrix core. Restated from the public
 * header's prose, sharing no code with the library:
 *
 *  - needs N % 16 == 0, K % 1024 == 0, G in {64, 128};
 *  - a weight w in {-1, 0, +1} is the trit t = w + 1 in {0, 1, 2};
 *  - strip s = rows [16s, 16s+16); k-quad Q = columns [1024Q, 1024Q+1024),
 *    four k-tiles j = 0..3 of 256 columns; block (s, Q) is 3328 bytes at
 *    byte offset (s*KQ + Q)*3328, KQ = K/1024;
 *  - inside a block, k-tile j's main part is bytes [768j, 768j+768): lane
 *    L in [0,64) owns bytes [768j + 12L, +12), three 4-byte words W0..W2;
 *    bytes [3072, 3328) are the tails: byte 3072 + 4L + j is lane L's tail
 *    byte for k-tile j;
 *  - weight (row 16s + r, column 1024Q + 256j + kk): with kk = 64q + u,
 *    u in [0,64), hi = u >= 32, u' = u - 32*hi, g = u' / 8, p = u' % 8,
 *    i = p / 2, e = hi ? (p odd ? 2 : 0) : (p odd ? 3 : 1): lane L = 16g + r,
 *    register R = 4q + i, byte e of the register;
 *  - R < 15: byte e of word W[R / 5] holds five trits t_0..t_4 (t_0 most
 *    significant) as the value v = sum_d t_d 3^(4-d) stored as the byte
 *    b = ceil(256 v / 243); the weight is digit d = R % 5. Here v is
 *    recovered as floor(243 b / 256) and split into base-3 digits;
 *  - R == 15: the tail byte holds the trit in bits [2e+1 : 2e] (value 3 is
 *    invalid);
 *  - scales as in layout v1: [s][kt][r][gi], kt = 4Q + j.
 *
 * Outputs w int8 [N][K] and s fp16 bits [N][K/G]. ORACLE_ERR_WEIGHT for a
 * byte that is not ceil(256 v / 243) of any v (never written) or a tail trit
 * of 3.
 */
int oracle_unpack_layout_t5(const uint8_t* codes, const uint16_t* scales_packed, int64_t N,
                            int64_t K, int64_t G, int8_t* w, uint16_t* s) {
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 1024 != 0 || (G != 64 && G != 128))
    return ORACLE_ERR_ARGS;
  const int64_t KQ = K / 1024, KT = K / 256, NG = K / G, GPT = 256 / G;
  static const int pow3[5] = {81, 27, 9, 3, 1};
  for (int64_t n = 0; n < N; ++n) {
    const int64_t st = n / 16, r = n % 16;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t Q = k / 1024, j = (k / 256) % 4, kk = k % 256;
      const int64_t q = kk / 64, u = kk % 64;
      const int64_t hi = u >= 32, up = u - 32 * hi;
      const int64_t g = up / 8, pp = up % 8, i = pp / 2, odd = pp % 2;
      const int64_t e = hi ? (odd ? 2 : 0) : (odd ? 3 : 1);
      const int64_t lane = 16 * g + r, R = 4 * q + i;
      const uint8_t* blk = codes + (st * KQ + Q) * 3328;
      int t;
      if (R < 15) {
        const int b = blk[768 * j + 12 * lane + 4 * (R / 5) + e];
        const int v = (243 * b) >> 8;
        if ((256 * v + 242) / 243 != b) return ORACLE_ERR_WEIGHT; /* not ceil(256 v / 243) */
        t = (v / pow3[R % 5]) % 3;
      } else {
        t = (blk[3072 + 4 * lane + j] >> (2 * e)) & 3;
        if (t == 3) return ORACLE_ERR_WEIGHT;
      }
      w[n * K + k] = (int8_t)(t - 1);
    }
    for (int64_t g = 0; g < NG; ++g) {
      const int64_t kt = g / GPT, gi = g % GPT;
      s[n * NG + g] = scales_packed[((st * KT + kt) * 16 + r) * GPT + gi];
    }
  }
  return ORACLE_OK;
}
