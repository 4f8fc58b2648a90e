/*
 * synth.c -- seeded synthetic inputs for the routed MoE layer.
 *
 * This module only draws numbers.  It holds none of the layer's arithmetic
 * (no routing, no projection, no activation, no combine); both the fp64 CPU
 * oracle and the HIP library receive the bytes it writes.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw n of stream (seed, tag) is mix64(key + (n + 1) * GAMMA),
 * key = mix64(seed) ^ mix64(tag ^ TAG_SALT).  Uniforms take the top 53 bits
 * as ((r >> 11) + 0.5) * 2^-53, strictly inside (0, 1).  Normals use the
 * Box-Muller transform (Box and Muller, 1958): the pair (2p, 2p+1) comes from
 * uniforms u1 = U(2p), u2 = U(2p+1) as r*cos(2*pi*u2), r*sin(2*pi*u2) with
 * r = sqrt(-2 ln u1), in double precision.
 *
 * Because every value depends only on (seed, tag, index), any slice can be
 * produced independently; the fill routines split work over pthreads and the
 * bytes do not depend on the thread count.
 *
 * Storage formats written here:
 *   - fp32: the double normal times std, rounded to float by a C cast (RNE).
 *   - bf16: that float rounded to bfloat16 by round-to-nearest-even on its
 *     bit pattern (upper 16 bits of an IEEE float).
 *   - fp8 e4m3 (OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF are NaN, max
 *     finite 448): per row of `cols` values, scale s = max|w| / 448 as float
 *     (s = 1 when the row is all zero), code = round-to-nearest-even of w / s,
 *     saturated at +-448.
 *   - MXFP4 (OCP Microscaling Formats v1.0): blocks of 32 consecutive values of
 *     a row share one E8M0 scale byte X (value 2^(X-127)), X - 127 =
 *     floor(log2(max|w| of the block)) - 2 (2 being the largest exponent of
 *     E2M1), or X = 0 for an all-zero block; each value is stored as the E2M1
 *     code (sign, 2 exponent bits, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5,
 *     2, 3, 4, 6) nearest w / 2^(X-127), ties to an even mantissa, saturating
 *     at 6.  Two codes per byte, the even-indexed value in the low nibble.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull
#define TAG_SALT 0x632BE59BD9B4E019ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return mix64(seed + GAMMA) ^ mix64((tag ^ TAG_SALT) + GAMMA);
}

static inline uint64_t draw_u64(uint64_t key, uint64_t n) {
  return mix64(key + (n + 1) * GAMMA);
}

static inline double draw_uniform(uint64_t key, uint64_t n) {
  return ((double)(draw_u64(key, n) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Normal number n of the stream (Box-Muller over the pair containing n). */
static inline double draw_normal(uint64_t key, uint64_t n) {
  uint64_t p = n >> 1;
  double u1 = draw_uniform(key, 2 * p);
  double u2 = draw_uniform(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (n & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP E4M3FN code of v by round-to-nearest-even, saturating at +-448. */
static uint8_t encode_e4m3fn(float v) {
  uint8_t sign = (v < 0.0f || (v == 0.0f && signbit(v))) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (isnan(v)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0.0009765625) { /* below half of the smallest subnormal 2^-9: rounds to 0 (ties to even 0) */
    return sign;
  }
  int e;
  frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) so the leading bit has weight 2^(e-1) */
  int E = e - 1;           /* unbiased exponent of a */
  if (E < -6) E = -6;      /* subnormal range shares the quantum 2^-9 */
  double quantum = ldexp(1.0, E - 3);
  double q = nearbyint(a / quantum); /* default rounding mode: nearest, ties to even */
  /* q in [8, 16] for normals (q == 16 carries into the next binade), [0, 8] for subnormals */
  if (q >= 16.0) { E += 1; q = 8.0; }
  if (E > 8 || (E == 8 && q > 14.0)) return sign | 0x7E; /* beyond 448 after rounding */
  if (q < 8.0) {            /* subnormal: exponent field 0, mantissa q */
    return sign | (uint8_t)q;
  }
  return sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8));
}

/* E2M1 code of v (already divided by its block scale): nearest magnitude, ties to the code
 * with an even mantissa bit, saturating at 6. */
static uint8_t encode_e2m1(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x8 : 0x0;
  double a = fabs(v);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double d = fabs(mag[c] - a), db = fabs(mag[best] - a);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------------ */
/* threaded fill                                                              */

typedef struct {
  int kind;            /* 0 f32, 1 bf16, 2 fp8 rows, 3 MXFP4 rows */
  uint64_t key;
  uint64_t first;      /* stream index of element 0 */
  int64_t lo, hi;      /* element range (rows for kind 2) */
  double std;
  int64_t cols;
  void *out;
  float *scales;
} fill_job;

static void *fill_worker(void *arg) {
  fill_job *j = (fill_job *)arg;
  if (j->kind == 0) {
    float *o = (float *)j->out;
    for (int64_t i = j->lo; i < j->hi; ++i) o[i] = (float)(draw_normal(j->key, j->first + (uint64_t)i) * j->std);
  } else if (j->kind == 1) {
    uint16_t *o = (uint16_t *)j->out;
    for (int64_t i = j->lo; i < j->hi; ++i)
      o[i] = float_to_bf16_rne((float)(draw_normal(j->key, j->first + (uint64_t)i) * j->std));
  } else if (j->kind == 3) {
    uint8_t *o = (uint8_t *)j->out, *sc = (uint8_t *)j->scales;
    const int64_t nb = j->cols / 32;
    float blk[32];
    for (int64_t r = j->lo; r < j->hi; ++r) {
      for (int64_t b = 0; b < nb; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
          uint64_t n = j->first + (uint64_t)(r * j->cols + b * 32 + i);
          blk[i] = (float)(draw_normal(j->key, n) * j->std);
          if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
        }
        int X = 0;
        if (amax > 0.0f) {
          int e;
          frexp((double)amax, &e); /* amax in [2^(e-1), 2^e) */
          X = (e - 1) - 2 + 127;
          if (X < 0) X = 0;
          if (X > 254) X = 254;
        }
        sc[r * nb + b] = (uint8_t)X;
        const double inv = ldexp(1.0, 127 - X);
        for (int i = 0; i < 32; i += 2)
          o[(r * j->cols + b * 32 + i) / 2] =
              (uint8_t)(encode_e2m1(blk[i] * inv) | (encode_e2m1(blk[i + 1] * inv) << 4));
      }
    }
  } else {
    uint8_t *o = (uint8_t *)j->out;
    float *row = (float *)malloc(sizeof(float) * (size_t)j->cols);
    for (int64_t r = j->lo; r < j->hi; ++r) {
      float amax = 0.0f;
      for (int64_t c = 0; c < j->cols; ++c) {
        uint64_t n = j->first + (uint64_t)(r * j->cols + c);
        row[c] = (float)(draw_normal(j->key, n) * j->std);
        float a = fabsf(row[c]);
        if (a > amax) amax = a;
      }
      float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      j->scales[r] = s;
      for (int64_t c = 0; c < j->cols; ++c) o[r * j->cols + c] = encode_e4m3fn(row[c] / s);
    }
    free(row);
  }
  return NULL;
}

static void run_fill(fill_job base, int64_t n_items, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (n_items < 65536 * (int64_t)threads && base.kind < 2) threads = (int)(n_items / 65536) + 1;
  if (base.kind >= 2 && n_items < threads) threads = (int)(n_items > 0 ? n_items : 1);
  pthread_t tid[64];
  fill_job jobs[64];
  for (int t = 0; t < threads; ++t) {
    jobs[t] = base;
    jobs[t].lo = n_items * t / threads;
    jobs[t].hi = n_items * (t + 1) / threads;
    if (threads == 1) { fill_worker(&jobs[t]); return; }
    pthread_create(&tid[t], NULL, fill_worker, &jobs[t]);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* exported                                                                   */

/* n normal draws of stream (seed, tag) starting at stream index `first`, times std, as fp32. */
void synth_normal_f32(uint64_t seed, uint64_t tag, uint64_t first, int64_t n, double std, float *out, int threads) {
  fill_job j = {0, stream_key(seed, tag), first, 0, n, std, 0, out, NULL};
  run_fill(j, n, threads);
}

/* Same draws rounded to bf16 (bit patterns). */
void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t first, int64_t n, double std, uint16_t *out, int threads) {
  fill_job j = {1, stream_key(seed, tag), first, 0, n, std, 0, out, NULL};
  run_fill(j, n, threads);
}

/* rows x cols normal draws times std, quantised per row to OCP E4M3FN codes plus one fp32 scale per row. */
void synth_normal_fp8_rows(uint64_t seed, uint64_t tag, uint64_t first, int64_t rows, int64_t cols, double std,
                           uint8_t *codes, float *scales, int threads) {
  fill_job j = {2, stream_key(seed, tag), first, 0, rows, std, cols, codes, scales};
  run_fill(j, rows, threads);
}

/* rows x cols normal draws times std as MXFP4: cols / 2 code bytes and cols / 32 E8M0
 * scale bytes per row (cols a multiple of 32). */
void synth_normal_mxfp4_rows(uint64_t seed, uint64_t tag, uint64_t first, int64_t rows, int64_t cols, double std,
                             uint8_t *codes, uint8_t *scales, int threads) {
  fill_job j = {3, stream_key(seed, tag), first, 0, rows, std, cols, codes, (float *)(void *)scales};
  run_fill(j, rows, threads);
}

/* n uniform draws in (0, 1) as doubles. */
void synth_uniform_f64(uint64_t seed, uint64_t tag, uint64_t first, int64_t n, double *out) {
  uint64_t key = stream_key(seed, tag);
  for (int64_t i = 0; i < n; ++i) out[i] = draw_uniform(key, first + (uint64_t)i);
}

/* A seeded permutation of 0..n-1 (Fisher-Yates driven by the stream's uniforms). */
void synth_permutation(uint64_t seed, uint64_t tag, int32_t n, int32_t *out) {
  uint64_t key = stream_key(seed, tag);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(draw_uniform(key, (uint64_t)(n - 1 - i)) * (double)(i + 1));
    if (j > i) j = i;
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* Raw 64-bit draws (for determinism checks of the generator itself). */
void synth_u64(uint64_t seed, uint64_t tag, uint64_t first, int64_t n, uint64_t *out) {
  uint64_t key = stream_key(seed, tag);
  for (int64_t i = 0; i < n; ++i) out[i] = draw_u64(key, first + (uint64_t)i);
}
