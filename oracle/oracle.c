/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the routed mixture-of-experts
 * FFN layer.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg use it; the library never does.  It shares no
 * code, header, table or helper with the HIP path.
 *
 * What is computed, and where it comes from.  The pages describe the layer
 * only by name; the arithmetic below is the standard Qwen-family sparse MoE
 * block, read as plainly as the pages allow:
 *   - veloGB10 README, "The model": routed experts per layer, a top-k choice
 *     per token (512 experts, top-10), plus one always-on shared expert.
 *   - Qwen3.6-35B-A3B for NInfer, "Artifact": routed experts have separate
 *     gate/up and down projections; the shared expert has the same form.
 *   - Qwen3.8 Flash-Next . GB10 UltraFast, first bullet ("verified-
 *     deterministic floor"): the token-to-expert alignment (the
 *     moe_align_block_size step) is made independent of thread arrival order,
 *     and the weighted combine avoids a float-atomicAdd epilogue.  Read here
 *     as: alignment lists each expert's slots in ascending slot order, and the
 *     combine sums a token's k expert outputs in slot order.
 *   - veloGB10 README, "Kernel work": router fold, grouped expert kernels
 *     that stream weights without rebuilding them, shared expert overlapped
 *     with the routed step.
 *
 * Readings fixed here (the pages are silent on all of them):
 *   R-route  logits l[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]; the k largest
 *            logits are chosen, ties to the lower expert index, -0 == +0, NaN
 *            below every number; slots j = 0..k-1 in that order; gate weights
 *            are the softmax over all E logits renormalised over the chosen k,
 *            which equals exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0).
 *   R-align  slot i = t*k + j; c_e = #slots routed to e; each expert's
 *            segment is padded to a multiple of BM (empty experts get none);
 *            segments are laid out in expert order; inside a segment slot ids
 *            ascend; padding and the tail up to the capacity hold the
 *            sentinel T*k; block_expert maps each BM block to its expert, -1
 *            past the padded total.
 *   R-ffn    SwiGLU expert: h_r = silu(g_r) * u_r with g = x.Wgu[r], u =
 *            x.Wgu[I + r] (rows [0, I) gate, [I, 2I) up); y_o = h . Wd[o].
 *            For fp8 weights, W = code * row_scale and the scale multiplies
 *            the finished row sum.
 *   R-shared shared expert with the same form; its output is scaled by
 *            sigmoid(x . w_sg).
 *   R-act8   wtype 2 (fp8 weights with fp8 activations, the matrix-core prefill
 *            reading of the pages' FP8 layers): each activation row entering
 *            an expert matrix -- the token x_t, and the bf16 h of a slot -- is
 *            quantised on its own: s = the smallest power of two with
 *            amax_i |a_i| <= 448 s (1 for an all-zero row) and code_i =
 *            E4M3FN(a_i / s), the nearest code, ties to an even mantissa (the
 *            quotient is exact: s is a power of two).  A power of two costs
 *            the e4m3 codes nothing -- they are floating point, every element
 *            keeps its three mantissa bits -- and it is the gfx950 matrix
 *            cores' own (E8M0) scale format.  Each dot product is the exact sum of
 *            decoded codes times decoded weights, multiplied by the weight's
 *            row scale and the activation row's scale.
 *   R-mx4    wtype 3 (MXFP4, OCP Microscaling Formats v1.0; 4-bit routed experts
 *            with 16-bit activations as in Qwen3.8 Flash-Next . GB10 UltraFast,
 *            "Target precision", in the gfx950-native form): weight (row, col) is
 *            the E2M1 code in nibble col & 1 (low nibble first) of byte
 *            col / 2 of the row, times 2^(X - 127) for the E8M0 byte X of
 *            block col / 32 of the row; no other scale.
 *   R-round  the HIP path stores h, each expert's output y and the layer
 *            output as bf16.  With `rounding` set, the oracle rounds at the
 *            same three points (fp64 -> bf16, round-to-nearest-even, single
 *            rounding); everything else stays fp64.
 */
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */

/* bfloat16 bits -> value: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Nearest bfloat16 (8 significant bits, binary32 exponent range), ties to
 * even, computed in one rounding from the double.  Returns the bit pattern. */
uint16_t oracle_bf16_round(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
  int E = e - 1;                     /* exponent of the leading bit */
  if (E < -126) E = -126;            /* bf16 subnormals: quantum 2^-133 */
  double quantum = ldexp(1.0, E - 7);
  double q = nearbyint(a / quantum); /* ties to even in the default mode */
  double r = q * quantum;            /* exact: q has at most 9 bits */
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow to infinity */
  float f = (float)r;                /* exact: r is representable in binary32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

double oracle_bf16_rounded(double v) { return oracle_bf16_value(oracle_bf16_round(v)); }

/* OCP 8-bit E4M3FN code -> value: sign s, exponent field E (bias 7), mantissa
 * m: E == 0 gives (-1)^s * 2^-6 * m/8, E == 15 with m == 7 is NaN, otherwise
 * (-1)^s * 2^(E-7) * (1 + m/8).  There are no infinities. */
double oracle_fp8_value(uint8_t q) {
  int s = (q >> 7) & 1, E = (q >> 3) & 15, m = q & 7;
  double mag;
  if (E == 15 && m == 7) return NAN;
  if (E == 0) mag = ldexp((double)m / 8.0, -6);
  else mag = ldexp(1.0 + (double)m / 8.0, E - 7);
  return s ? -mag : mag;
}

/* value -> OCP E4M3FN code: the nearest code, ties to the code with an even
 * mantissa; magnitudes of 448 and above give 448 (the largest finite code) and
 * NaN gives the NaN code.  Below 2^-6 the codes are the subnormal steps of 2^-9. */
uint8_t oracle_fp8_encode(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < 0.015625) return (uint8_t)(sign | (int)nearbyint(a * 512.0)); /* 8: the smallest normal */
  int ex;
  frexp(a, &ex); /* a = f * 2^ex with f in [0.5, 1) */
  int e = ex - 1;
  int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  return (uint8_t)(sign | ((e + 7) << 3) | m);
}

/* R-act8: one activation row (fp32-representable values) -> codes q[0..n) and the
 * row's scale, returned: s = 2^e for the least e with amax <= 448 * 2^e (e = 0 for
 * an all-zero row); q_i = oracle_fp8_encode(a_i * 2^-e), an exact product. */
double oracle_quantise_row(int n, const double *a, uint8_t *q) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) {
    double v = fabs((double)(float)a[i]);
    if (v > amax) amax = v;
  }
  int e = 0;
  if (amax > 0.0) {
    int ex;
    double f = frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1); 448 / 512 = 0.875 */
    e = f <= 0.875 ? ex - 9 : ex - 8;
  }
  for (int i = 0; i < n; ++i) q[i] = oracle_fp8_encode((float)ldexp((double)(float)a[i], -e));
  return ldexp(1.0, e);
}

/* E2M1 code (low 4 bits): sign bit 3, exponent field E = bits 2..1 (bias 1), mantissa m =
 * bit 0; E == 0 gives (-1)^s * m / 2, otherwise (-1)^s * 2^(E-1) * (1 + m/2). */
double oracle_fp4_value(uint8_t c) {
  int s = (c >> 3) & 1, E = (c >> 1) & 3, m = c & 1;
  double mag = E == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
  return s ? -mag : mag;
}

/* E8M0 scale byte: 2^(X - 127); 0xFF is NaN. */
double oracle_e8m0_value(uint8_t X) { return X == 0xFF ? NAN : ldexp(1.0, (int)X - 127); }

/* weight (row, col) of a matrix with `cols` columns: bf16 (wtype 0), fp8 codes (1, 2), or
 * MXFP4 (3: codes two per byte, with the E8M0 block scales `sc`) -- R-mx4 above */
static double weight(const void *w, const void *sc, int wtype, size_t row, size_t col, size_t cols) {
  if (wtype == 0) return oracle_bf16_value(((const uint16_t *)w)[row * cols + col]);
  if (wtype != 3) return oracle_fp8_value(((const uint8_t *)w)[row * cols + col]);
  uint8_t b = ((const uint8_t *)w)[(row * cols + col) / 2];
  uint8_t code = (col & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
  return oracle_fp4_value(code) * oracle_e8m0_value(((const uint8_t *)sc)[row * (cols / 32) + col / 32]);
}

static double silu(double g) { return g / (1.0 + exp(-g)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------ */
/* routing                                                                   */

/* Router logits in fp64: l[t][e] = sum_h x[t][h] * Wr[e][h] + b[e] (b may be
 * NULL).  veloGB10 README, "Kernel work" (router fold); R-route above. */
void oracle_router_logits(int T, int H, int E, const uint16_t *x, const float *w_r, const float *b_r,
                          double *logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += oracle_bf16_value(x[(size_t)t * H + h]) * (double)w_r[(size_t)e * H + h];
      if (b_r) acc += (double)b_r[e];
      logits[(size_t)t * E + e] = acc;
    }
}

/* The shared expert's gate logit z[t] = sum_h x[t][h] * w_sg[h], fp64. */
void oracle_shared_gate_logits(int T, int H, const uint16_t *x, const float *w_sg, double *z) {
  for (int t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int h = 0; h < H; ++h) acc += oracle_bf16_value(x[(size_t)t * H + h]) * (double)w_sg[h];
    z[t] = acc;
  }
}

/* Is (a, ea) ranked before (b, eb)?  Larger logit first; equal logits (IEEE
 * equality, so -0 == +0) by lower expert index; NaN after every number. */
static int ranks_before(float a, int ea, float b, int eb) {
  int na = isnan(a), nb = isnan(b);
  if (na != nb) return nb;
  if (!na && a != b) return a > b;
  return ea < eb;
}

/* Top-k routing from given fp32 logits [T][E] (R-route): ids [T][k] int32 in
 * rank order and gate weights [T][k] in fp64.  renormalize != 0: softmax over
 * all experts renormalised over the chosen k; renormalize == 0: the plain
 * softmax probability of each chosen expert.  veloGB10 README, "The model"
 * (top-k per token); Qwen3.8 Flash-Next . GB10 UltraFast, "How it works"
 * (sort-free verify-path top-k is the selection being mirrored). */
void oracle_route_topk(int T, int E, int k, int renormalize, const float *logits, int32_t *ids, double *w) {
  char *taken = (char *)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    double top = (double)l[ids[(size_t)t * k]];
    double denom = 0.0;
    if (renormalize) {
      for (int j = 0; j < k; ++j) denom += exp((double)l[ids[(size_t)t * k + j]] - top);
    } else {
      for (int e = 0; e < E; ++e) denom += exp((double)l[e] - top);
    }
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - top) / denom;
  }
  free(taken);
}

/* ------------------------------------------------------------------------ */
/* alignment                                                                 */

/* Capacity of the padded slot list: every slot, plus at most BM-1 padding for
 * each expert that can be touched, rounded up to BM. */
int64_t oracle_align_capacity(int T, int k, int E, int BM) {
  int64_t n = (int64_t)T * k;
  int64_t touched = n < E ? n : E;
  int64_t c = n + touched * (BM - 1);
  return (c + BM - 1) / BM * BM;
}

/* Token-to-expert alignment (R-align): histogram, padded exclusive scan and a
 * stable scatter of slot ids.  Qwen3.8 Flash-Next . GB10 UltraFast, first
 * bullet and "Configuration reference" (moe_align_block_size with the
 * arrival-order shim).  Returns 0, or -1 when cap is too small. */
int oracle_align(int T, int k, int E, int BM, int64_t cap, const int32_t *ids, int32_t *sorted,
                 int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *num_padded) {
  int64_t n = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n; ++i) counts[ids[i]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int32_t padded = (counts[e] + BM - 1) / BM * BM;
    offsets[e + 1] = offsets[e] + padded;
  }
  *num_padded = offsets[E];
  if (offsets[E] > cap) return -1;
  for (int64_t p = 0; p < cap; ++p) sorted[p] = (int32_t)n;
  for (int e = 0; e < E; ++e) {
    int32_t r = 0;
    for (int64_t i = 0; i < n; ++i)
      if (ids[i] == e) sorted[offsets[e] + r++] = (int32_t)i;
  }
  for (int64_t b = 0; b < cap / BM; ++b) block_expert[b] = -1;
  for (int e = 0; e < E; ++e)
    for (int32_t p = offsets[e]; p < offsets[e + 1]; p += BM) block_expert[p / BM] = e;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* experts and the layer                                                     */

/* One token through one SwiGLU expert of a bank (R-ffn, R-round).
 * Qwen3.6-35B-A3B for NInfer, "Artifact" (gate/up and down projections).
 *   x [H] bf16 bits; w_gu [2I][H], w_d [H][I] (this expert's slices);
 *   s_gu [2I], s_d [H] row scales for fp8 (ignored for bf16); for MXFP4 the E8M0 block
 *   scales, [2I][H/32] and [H][I/32] bytes;
 *   y [H] output in fp64 (bf16-rounded values when rounding != 0).
 * wtype 2 quantises x before the gate/up sums and h before the down sums (R-act8). */
static void expert_ffn(int H, int I, int wtype, const uint16_t *x, const void *w_gu, const void *w_d,
                       const void *sgu, const void *sd, int rounding, double *hbuf, double *y) {
  const float *s_gu = (const float *)sgu, *s_d = (const float *)sd; /* fp8 row scales */
  double *xa = (double *)calloc((size_t)H, sizeof(double));
  uint8_t *q = (uint8_t *)malloc((size_t)(H > I ? H : I));
  for (int h = 0; h < H; ++h) xa[h] = oracle_bf16_value(x[h]);
  double sx = 1.0, sh = 1.0;
  if (wtype == 2) {
    sx = oracle_quantise_row(H, xa, q);
    for (int h = 0; h < H; ++h) xa[h] = oracle_fp8_value(q[h]);
  }
  for (int r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += xa[h] * weight(w_gu, sgu, wtype, (size_t)r, (size_t)h, (size_t)H);
      u += xa[h] * weight(w_gu, sgu, wtype, (size_t)(I + r), (size_t)h, (size_t)H);
    }
    if (wtype == 1 || wtype == 2) {
      g *= (double)s_gu[r];
      u *= (double)s_gu[I + r];
    }
    if (wtype == 2) {
      g *= sx;
      u *= sx;
    }
    double a = silu(g) * u;
    hbuf[r] = rounding ? oracle_bf16_rounded(a) : a;
  }
  if (wtype == 2) {
    sh = oracle_quantise_row(I, hbuf, q);
    for (int r = 0; r < I; ++r) hbuf[r] = oracle_fp8_value(q[r]);
  }
  for (int o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int r = 0; r < I; ++r) acc += hbuf[r] * weight(w_d, sd, wtype, (size_t)o, (size_t)r, (size_t)I);
    if (wtype == 1 || wtype == 2) acc *= (double)s_d[o];
    if (wtype == 2) acc *= sh;
    y[o] = rounding ? oracle_bf16_rounded(acc) : acc;
  }
  free(xa);
  free(q);
}

/* bytes of an n-element matrix, and of its scales (per-row fp32 for fp8; one E8M0 byte per
 * 32 elements for MXFP4) for `rows` rows */
static size_t matrix_bytes(int wtype, size_t n) { return wtype == 0 ? 2 * n : wtype == 3 ? n / 2 : n; }
static size_t scale_bytes(int wtype, size_t rows, size_t n) {
  return wtype == 3 ? n / 32 : (wtype == 1 || wtype == 2) ? 4 * rows : 0;
}

/* The layer for a list of tokens, routed by the given ids and gate weights:
 *   out[t] = sum_{j<k} w[t][j] * y_{e(t,j)}(x_t) + sigmoid(x_t . w_sg) * y_shared(x_t)
 * summed in slot order j = 0..k-1, then the shared term (R-shared), rounded to
 * bf16 when rounding != 0 (R-round).  The shared expert is absent when I_s == 0.
 * Qwen3.8 Flash-Next . GB10 UltraFast, first bullet (combine without float
 * atomics: a fixed order); veloGB10 README, "The model" (shared expert).
 *   x [T][H] bf16; w_gu [E][2I][H]; w_d [E][H][I]; s_gu [E][2I]; s_d [E][H] (MXFP4:
 *   [E][2I][H/32], [E][H][I/32] scale bytes);
 *   ids [T][k]; w [T][k] fp64; shared: ws_gu [2I_s][H], ws_d [H][I_s],
 *   ss_gu [2I_s], ss_d [H], w_sg [H] fp32;
 *   tokens [n_tok] (token indices to compute); out [n_tok][H] fp64. */
void oracle_moe_layer(int T, int H, int E, int k, int I, int wtype, const uint16_t *x, const void *w_gu,
                      const void *w_d, const void *s_gu, const void *s_d, const int32_t *ids, const double *w,
                      int I_s, const void *ws_gu, const void *ws_d, const void *ss_gu, const void *ss_d,
                      const float *w_sg, int n_tok, const int32_t *tokens, int rounding, double *out) {
  (void)T;
  (void)E;
  int Imax = I > I_s ? I : I_s;
  double *hbuf = (double *)malloc(sizeof(double) * (size_t)Imax);
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  double *acc = (double *)malloc(sizeof(double) * (size_t)H);
  const size_t ngu = (size_t)2 * I * H, nd = (size_t)H * I;
  for (int q = 0; q < n_tok; ++q) {
    int t = tokens[q];
    const uint16_t *xt = x + (size_t)t * H;
    for (int o = 0; o < H; ++o) acc[o] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      const char *gu = (const char *)w_gu + (size_t)e * matrix_bytes(wtype, ngu);
      const char *dn = (const char *)w_d + (size_t)e * matrix_bytes(wtype, nd);
      const char *sg = wtype != 0 ? (const char *)s_gu + (size_t)e * scale_bytes(wtype, 2 * (size_t)I, ngu) : NULL;
      const char *sd = wtype != 0 ? (const char *)s_d + (size_t)e * scale_bytes(wtype, (size_t)H, nd) : NULL;
      expert_ffn(H, I, wtype, xt, gu, dn, sg, sd, rounding, hbuf, y);
      double wj = w[(size_t)t * k + j];
      for (int o = 0; o < H; ++o) acc[o] += wj * y[o];
    }
    if (I_s > 0) {
      double z = 0.0;
      for (int h = 0; h < H; ++h) z += oracle_bf16_value(xt[h]) * (double)w_sg[h];
      double gamma = sigmoid(z);
      expert_ffn(H, I_s, wtype, xt, ws_gu, ws_d, ss_gu, ss_d, rounding, hbuf, y);
      for (int o = 0; o < H; ++o) acc[o] += gamma * y[o];
    }
    for (int o = 0; o < H; ++o) out[(size_t)q * H + o] = rounding ? oracle_bf16_rounded(acc[o]) : acc[o];
  }
  free(hbuf);
  free(y);
  free(acc);
}

/* One expert applied to one token, exposed for the pins (y [H] fp64). */
void oracle_expert(int H, int I, int wtype, const uint16_t *x, const void *w_gu, const void *w_d,
                   const void *s_gu, const void *s_d, int rounding, double *y) {
  double *hbuf = (double *)malloc(sizeof(double) * (size_t)I);
  expert_ffn(H, I, wtype, x, w_gu, w_d, s_gu, s_d, rounding, hbuf, y);
  free(hbuf);
}

/* ------------------------------------------------------------------------ */
/* the layer over several host threads                                       */

typedef struct {
  int T, H, E, k, I, wtype;
  const uint16_t *x;
  const void *w_gu, *w_d, *s_gu, *s_d;
  const int32_t *ids;
  const double *w;
  int I_s;
  const void *ws_gu, *ws_d, *ss_gu, *ss_d;
  const float *w_sg;
  const int32_t *tokens;
  int rounding;
  double *out;
  int first, count; /* this thread's range of the token list */
} layer_job;

static void *layer_worker(void *p) {
  const layer_job *j = (const layer_job *)p;
  if (j->count > 0)
    oracle_moe_layer(j->T, j->H, j->E, j->k, j->I, j->wtype, j->x, j->w_gu, j->w_d, j->s_gu, j->s_d, j->ids, j->w,
                     j->I_s, j->ws_gu, j->ws_d, j->ss_gu, j->ss_d, j->w_sg, j->count, j->tokens + j->first,
                     j->rounding, j->out + (size_t)j->first * j->H);
  return NULL;
}

/* oracle_moe_layer with the token list split into nthreads contiguous ranges, one host
 * thread each.  Every token is computed by exactly the code above, on its own buffers, so
 * the output is bitwise that of oracle_moe_layer for any thread count.  Returns the number
 * of threads used (1 when nthreads <= 1 or a thread cannot be started). */
int oracle_moe_layer_mt(int T, int H, int E, int k, int I, int wtype, const uint16_t *x, const void *w_gu,
                        const void *w_d, const void *s_gu, const void *s_d, const int32_t *ids, const double *w,
                        int I_s, const void *ws_gu, const void *ws_d, const void *ss_gu, const void *ss_d,
                        const float *w_sg, int n_tok, const int32_t *tokens, int rounding, double *out,
                        int nthreads) {
  if (nthreads > n_tok) nthreads = n_tok;
  if (nthreads < 1) nthreads = 1;
  layer_job *jobs = (layer_job *)calloc((size_t)nthreads, sizeof(layer_job));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    layer_job *j = &jobs[i];
    j->T = T; j->H = H; j->E = E; j->k = k; j->I = I; j->wtype = wtype;
    j->x = x; j->w_gu = w_gu; j->w_d = w_d; j->s_gu = s_gu; j->s_d = s_d;
    j->ids = ids; j->w = w; j->I_s = I_s;
    j->ws_gu = ws_gu; j->ws_d = ws_d; j->ss_gu = ss_gu; j->ss_d = ss_d; j->w_sg = w_sg;
    j->tokens = tokens; j->rounding = rounding; j->out = out;
    j->first = (int)((int64_t)n_tok * i / nthreads);
    j->count = (int)((int64_t)n_tok * (i + 1) / nthreads) - j->first;
  }
  /* thread 0's range runs on the calling thread; a range whose thread cannot be started
   * runs here too */
  int used = 1;
  char *live = (char *)calloc((size_t)nthreads, 1);
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, layer_worker, &jobs[i]) == 0) {
      live[i] = 1;
      ++used;
    } else {
      layer_worker(&jobs[i]);
    }
  }
  layer_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i)
    if (live[i]) pthread_join(th[i], NULL);
  free(live);
  free(jobs);
  free(th);
  return used;
}
