/*
 * kvq_oracle.c -- CPU oracle for the rotated 4-bit KV cache and for decode
 * attention over it.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, deliberately unoptimised
 * restatement of what the method computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the HIP library (bit_quantized_kv_rotate_amd),
 * and the HIP library never calls it.
 *
 * Source of the method: the AMD ROCm blog post "UltraQuant on AMD Instinct"
 * (read from a machine-translated copy).
 *   - section "What is UltraQuant?": keys and values are stored on the FP4
 *     grid that MI355X supports natively (E2M1), each 32-channel group shares
 *     one power-of-two scale, a group costs 17 bytes against 32 for an 8-bit
 *     cache; before quantisation every head vector goes through a
 *     Walsh-Hadamard rotation that spreads outlier channels.
 *   - section "Why UltraQuant beats 8-bit KV": the scales are UE8M0 bytes and
 *     the FP4 codes are consumed natively; every decode step re-reads the
 *     whole cache.
 *   - section "Throughput vs latency trade-off": an MTP verify step carries
 *     several query positions per sequence over one paged cache.
 * Where the page is silent (normalisation and order of the Hadamard
 * transform, the exact shared-exponent rule, rounding, nibble order, the
 * causal rule between verify positions) the oracle takes one plain reading;
 * every such reading is listed in the design notes of the repository.
 *
 * Precision: the rotation and the quantisation run in fp32 in a fixed order
 * (radix-2 butterfly stages h = 1, 2, 4, ..., d/2, then one multiply by the
 * fp32-rounded 1/sqrt(d)); attention (scores, softmax, weighted sum and the
 * inverse rotation of the output) runs in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 *
 * Every exported function is pinned by tests against closed forms,
 * independent library routines or brute force; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

/* ------------------------------------------------------------------ */
/* bf16 input                                                          */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper half of an fp32; widening is exact. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

float orc_bf16_to_f32(uint16_t b) { return bf16_to_f32(b); }

/* ------------------------------------------------------------------ */
/* Walsh-Hadamard rotation ("What is UltraQuant?")                     */
/* ------------------------------------------------------------------ */

/* In-place orthonormal Walsh-Hadamard transform in natural (Sylvester)
 * order, fp32: for h = 1, 2, ..., d/2 and each pair (j, j+h) inside a block
 * of 2h entries, x[j] <- x[j] + x[j+h] and x[j+h] <- x[j] - x[j+h] (both
 * computed from the old values, one rounding each); afterwards every entry is
 * multiplied once by fp32(1/sqrt(d)).  d must be a power of two. */
void orc_fwht_f32(float *x, int d) {
  for (int h = 1; h < d; h *= 2) {
    for (int i = 0; i < d; i += 2 * h) {
      for (int j = i; j < i + h; ++j) {
        float a = x[j];
        float b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
  const float c = (float)(1.0 / sqrt((double)d));
  for (int k = 0; k < d; ++k) x[k] = x[k] * c;
}

/* The same transform in fp64 (used to take attention outputs back from the
 * rotated basis; H is symmetric and orthogonal, so it is its own inverse). */
void orc_fwht_f64(double *x, int d) {
  for (int h = 1; h < d; h *= 2) {
    for (int i = 0; i < d; i += 2 * h) {
      for (int j = i; j < i + h; ++j) {
        double a = x[j];
        double b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
  const double c = 1.0 / sqrt((double)d);
  for (int k = 0; k < d; ++k) x[k] = x[k] * c;
}

/* ------------------------------------------------------------------ */
/* Shared power-of-two scale (UE8M0)                                   */
/* ------------------------------------------------------------------ */

/* Scale exponent for one 32-value group: e_s = floor(log2(amax)) - emax_elem,
 * where emax_elem is the exponent of the element format's largest value
 * (2 for E2M1, whose largest value is 6 = 1.5 * 2^2; 8 for E4M3, largest
 * 448 = 1.75 * 2^8).  floor(log2(amax)) comes from frexp, exactly.  amax = 0
 * and anything that would go below -127 clamp to -127.  The stored byte is
 * e_s + 127 and stands for 2^(byte - 127). */
int orc_scale_exponent(float amax, int emax_elem) {
  if (!(amax > 0.0f)) return -127;
  int E;
  (void)frexp((double)amax, &E); /* amax = m * 2^E, m in [0.5, 1) */
  int e = (E - 1) - emax_elem;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

int orc_scale_byte(float amax, int emax_elem) {
  return orc_scale_exponent(amax, emax_elem) + 127;
}

double orc_scale_value(int byte) { return ldexp(1.0, byte - 127); }

/* ------------------------------------------------------------------ */
/* FP4 E2M1 element codes                                              */
/* ------------------------------------------------------------------ */

/* Magnitudes of the eight E2M1 codes 0..7 (sign is bit 3). */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double v = E2M1_GRID[code & 7];
  return (code & 8) ? -v : v;
}

/* Code of y in a group whose scale exponent is e_s: r = y * 2^-e_s (exact in
 * fp64); the magnitude code is the grid point nearest to |r|, a tie going to
 * the even code; anything beyond 6 takes 6; the sign bit is y's sign bit (so
 * a negative value that rounds to zero is stored as 0x8). */
int orc_e2m1_encode(float y, int e_s) {
  double r = fabs(ldexp((double)y, -e_s));
  int best = 0;
  double best_d = fabs(r - E2M1_GRID[0]);
  for (int k = 1; k < 8; ++k) {
    double dk = fabs(r - E2M1_GRID[k]);
    if (dk < best_d || (dk == best_d && (k % 2) == 0)) {
      best = k;
      best_d = dk;
    }
  }
  return best | (signbit(y) ? 8 : 0);
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 element codes (8-bit comparator)                           */
/* ------------------------------------------------------------------ */

/* OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, 0x7F/0xFF are NaN, subnormals m * 2^-9, largest 448. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest finite E4M3 value to |y * 2^-e_s|, a tie going to the even code;
 * magnitudes past 448 therefore take 448; sign copied from y. */
int orc_e4m3_encode(float y, int e_s) {
  double r = fabs(ldexp((double)y, -e_s));
  int best = 0;
  double best_d = fabs(r - 0.0);
  for (int k = 1; k < 127; ++k) { /* 0x7F is NaN */
    double dk = fabs(r - orc_e4m3_value(k));
    if (dk < best_d || (dk == best_d && (k % 2) == 0)) {
      best = k;
      best_d = dk;
    }
  }
  return best | (signbit(y) ? 0x80 : 0);
}

/* The two encoders over n values at one scale exponent (a loop of the
 * single-value functions above, for sweeps over many inputs): out[i] is the
 * code of y[i]. */
void orc_e2m1_encode_n(const float *y, int64_t n, int e_s, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_encode(y[i], e_s);
}

void orc_e4m3_encode_n(const float *y, int64_t n, int e_s, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(y[i], e_s);
}

/* ------------------------------------------------------------------ */
/* One head vector: rotate, then quantise group by group               */
/* ------------------------------------------------------------------ */

/* FP4: x is d bf16 values.  Output: d/2 code bytes (channel 2i in the low
 * nibble of byte i, channel 2i+1 in the high nibble) and d/32 scale bytes.
 * Each 32-channel group therefore occupies 16 code bytes + 1 scale byte. */
void orc_quantize_fp4(const uint16_t *x, int d, int rotate, uint8_t *codes,
                      uint8_t *scales) {
  float *y = (float *)malloc(sizeof(float) * (size_t)d);
  for (int c = 0; c < d; ++c) y[c] = bf16_to_f32(x[c]);
  if (rotate) orc_fwht_f32(y, d);
  for (int g = 0; g < d / 32; ++g) {
    float amax = 0.0f;
    for (int c = 32 * g; c < 32 * g + 32; ++c)
      if (fabsf(y[c]) > amax) amax = fabsf(y[c]);
    int e_s = orc_scale_exponent(amax, 2);
    scales[g] = (uint8_t)(e_s + 127);
    for (int i = 0; i < 16; ++i) {
      int lo = orc_e2m1_encode(y[32 * g + 2 * i], e_s);
      int hi = orc_e2m1_encode(y[32 * g + 2 * i + 1], e_s);
      codes[16 * g + i] = (uint8_t)(lo | (hi << 4));
    }
  }
  free(y);
}

/* FP8 comparator: d code bytes (channel c in byte c) and d/32 scale bytes. */
void orc_quantize_fp8(const uint16_t *x, int d, int rotate, uint8_t *codes,
                      uint8_t *scales) {
  float *y = (float *)malloc(sizeof(float) * (size_t)d);
  for (int c = 0; c < d; ++c) y[c] = bf16_to_f32(x[c]);
  if (rotate) orc_fwht_f32(y, d);
  for (int g = 0; g < d / 32; ++g) {
    float amax = 0.0f;
    for (int c = 32 * g; c < 32 * g + 32; ++c)
      if (fabsf(y[c]) > amax) amax = fabsf(y[c]);
    int e_s = orc_scale_exponent(amax, 8);
    scales[g] = (uint8_t)(e_s + 127);
    for (int c = 32 * g; c < 32 * g + 32; ++c)
      codes[c] = (uint8_t)orc_e4m3_encode(y[c], e_s);
  }
  free(y);
}

/* Dequantise one vector: value = code value * 2^(scale byte - 127), exact. */
void orc_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int d,
                     float *out) {
  for (int c = 0; c < d; ++c) {
    int byte = codes[c / 2];
    int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
    out[c] = (float)ldexp(orc_e2m1_value(code), scales[c / 32] - 127);
  }
}

void orc_dequant_fp8(const uint8_t *codes, const uint8_t *scales, int d,
                     float *out) {
  for (int c = 0; c < d; ++c)
    out[c] = (float)ldexp(orc_e4m3_value(codes[c]), scales[c / 32] - 127);
}

/* Many vectors, one after the other (n vectors of d values each). */
void orc_quantize_fp4_n(const uint16_t *x, int64_t n, int d, int rotate,
                        uint8_t *codes, uint8_t *scales) {
  for (int64_t v = 0; v < n; ++v)
    orc_quantize_fp4(x + v * d, d, rotate, codes + v * (d / 2),
                     scales + v * (d / 32));
}

void orc_quantize_fp8_n(const uint16_t *x, int64_t n, int d, int rotate,
                        uint8_t *codes, uint8_t *scales) {
  for (int64_t v = 0; v < n; ++v)
    orc_quantize_fp8(x + v * d, d, rotate, codes + v * d, scales + v * (d / 32));
}

void orc_dequant_fp4_n(const uint8_t *codes, const uint8_t *scales, int64_t n,
                       int d, float *out) {
  for (int64_t v = 0; v < n; ++v)
    orc_dequant_fp4(codes + v * (d / 2), scales + v * (d / 32), d, out + v * d);
}

void orc_dequant_fp8_n(const uint8_t *codes, const uint8_t *scales, int64_t n,
                       int d, float *out) {
  for (int64_t v = 0; v < n; ++v)
    orc_dequant_fp8(codes + v * d, scales + v * (d / 32), d, out + v * d);
}

/* ------------------------------------------------------------------ */
/* Decode attention for one sequence                                   */
/* ------------------------------------------------------------------ */

/* Textbook softmax attention in fp64 for one sequence, all in one basis.
 *   q    : [n_q][hq][d] fp64 queries
 *   khat : [L][hkv][d] fp32 keys (already dequantised)
 *   vhat : [L][hkv][d] fp32 values, or NULL when values equal keys
 *   out  : [n_q][hq][d] fp64
 * Query head h reads KV head h / (hq / hkv).  Query position j (of n_q, the
 * last n_q tokens of the L cached ones being the verify positions) sees
 * tokens 0 .. L - n_q + j.  Scores are sm_scale * <q, k> accumulated in fp64;
 * softmax is the two-pass max-subtracted form. */
void orc_attend(const double *q, int n_q, int hq, int hkv, int d, int L,
                const float *khat, const float *vhat, double sm_scale,
                double *out) {
  const int g = hq / hkv;
  const float *V = vhat ? vhat : khat;
  double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  for (int j = 0; j < n_q; ++j) {
    for (int h = 0; h < hq; ++h) {
      const int kv = h / g;
      const double *qv = q + ((size_t)j * hq + h) * d;
      double *o = out + ((size_t)j * hq + h) * d;
      const int last = L - n_q + j; /* inclusive */
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (last < 0) continue;
      double M = -INFINITY;
      for (int t = 0; t <= last; ++t) {
        const float *k = khat + ((size_t)t * hkv + kv) * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qv[c] * (double)k[c];
        s[t] = sm_scale * acc;
        if (s[t] > M) M = s[t];
      }
      double Z = 0.0;
      for (int t = 0; t <= last; ++t) {
        s[t] = exp(s[t] - M);
        Z += s[t];
      }
      for (int t = 0; t <= last; ++t) {
        const double p = s[t] / Z;
        const float *v = V + ((size_t)t * hkv + kv) * d;
        for (int c = 0; c < d; ++c) o[c] += p * (double)v[c];
      }
    }
  }
  free(s);
}

/* Decode attention as the cache user sees it, for one sequence:
 *   q_bf16 : [n_q][hq][d] bf16 queries in the caller's basis
 *   khat, vhat : the dequantised cache (rotated basis when rotate = 1)
 *   out    : [n_q][hq][d] fp64 in the caller's basis
 * With rotate = 1 the query is rotated by the fp32 transform (the same one
 * the cache went through) before the scores, and the weighted sum of values
 * is taken back by the fp64 transform at the end.  Rotation does not change
 * the attention itself because H is orthogonal. */
void orc_decode(const uint16_t *q_bf16, int n_q, int hq, int hkv, int d, int L,
                const float *khat, const float *vhat, int rotate,
                double sm_scale, double *out) {
  const size_t nq = (size_t)n_q * hq * d;
  double *q = (double *)calloc(nq ? nq : 1, sizeof(double));
  float *tmp = (float *)malloc(sizeof(float) * (size_t)d);
  for (size_t r = 0; r < (size_t)n_q * hq; ++r) {
    for (int c = 0; c < d; ++c) tmp[c] = bf16_to_f32(q_bf16[r * d + c]);
    if (rotate) orc_fwht_f32(tmp, d);
    for (int c = 0; c < d; ++c) q[r * d + c] = (double)tmp[c];
  }
  orc_attend(q, n_q, hq, hkv, d, L, khat, vhat, sm_scale, out);
  if (rotate)
    for (size_t r = 0; r < (size_t)n_q * hq; ++r) orc_fwht_f64(out + r * d, d);
  free(tmp);
  free(q);
}

int orc_version(void) { return 1; }
