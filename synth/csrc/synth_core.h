/* Seeded synthetic-input generator: the per-element arithmetic shared by the
 * host (C, synth_host.c) and device (HIP, synth_dev.hip) fill routines, so that
 * both produce the same bytes for the same (seed, tensor id, element index).
 *
 * This file holds no part of the MoE layer's arithmetic. It only turns counters
 * into input values:
 *   - Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 *     Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): 10 rounds
 *     of two 32x32->64-bit multiplies with a Weyl-sequence key schedule.
 *   - inverse-transform sampling of N(0,1) through a table of normal quantiles
 *     (filled by the caller) with linear interpolation in fp32;
 *   - round-to-nearest-even narrowing of fp32 to bf16, OCP E4M3FN, OCP MX E2M1 and
 *     symmetric INT8, used to store generated weights in the layer's storage formats.
 *
 * Every floating-point step is a single IEEE-754 binary32 operation (multiply,
 * add, divide) or exact integer work, so host and device agree bit for bit as
 * long as both are compiled without FMA contraction (-ffp-contract=off).
 *
 * The including file defines SYN_FN (function qualifiers) before including.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYN_FN
#error "define SYN_FN before including synth_core.h"
#endif

#define SYN_PHILOX_M0 0xD2511F53u
#define SYN_PHILOX_M1 0xCD9E8D57u
#define SYN_PHILOX_W0 0x9E3779B9u
#define SYN_PHILOX_W1 0xBB67AE85u

/* Number of intervals of the quantile table; the table holds SYN_QN + 1 points. */
#define SYN_QBITS 16
#define SYN_QN (1u << SYN_QBITS)

typedef struct { uint32_t v[4]; } syn_u32x4;

SYN_FN void syn_mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

/* Philox4x32 with 10 rounds on counter c and key (k0, k1). */
SYN_FN syn_u32x4 syn_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                   uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    syn_mulhilo(SYN_PHILOX_M0, c0, &hi0, &lo0);
    syn_mulhilo(SYN_PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += SYN_PHILOX_W0;
    k1 += SYN_PHILOX_W1;
  }
  syn_u32x4 out;
  out.v[0] = c0; out.v[1] = c1; out.v[2] = c2; out.v[3] = c3;
  return out;
}

/* The raw 32-bit word for element i of tensor `tid` under `seed`.
 * Element i takes word (i mod 4) of the block at counter (i/4, tid, 0). */
SYN_FN uint32_t syn_word(uint64_t seed, uint32_t tid, uint64_t i) {
  uint64_t blk = i >> 2;
  syn_u32x4 r = syn_philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), tid, 0u,
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
  return r.v[i & 3u];
}

SYN_FN float syn_bits_f32(uint32_t u) {
  union { uint32_t u; float f; } c; c.u = u; return c.f;
}
SYN_FN uint32_t syn_f32_bits(float f) {
  union { uint32_t u; float f; } c; c.f = f; return c.u;
}

/* Standard normal by inverse transform: the top SYN_QBITS bits of the word pick
 * an interval of the quantile table q[0..SYN_QN], the low 16 bits place the
 * point inside it. f = low16 * 2^-16 is exact; the two fp32 operations below are
 * each rounded once. */
SYN_FN float syn_std_normal(uint32_t u, const float* q) {
  uint32_t idx = u >> (32 - SYN_QBITS);
  float f = (float)(u & 0xFFFFu) * (1.0f / 65536.0f);
  float a = q[idx];
  float b = q[idx + 1];
  float d = b - a;
  float t = f * d;
  return a + t;
}

/* N(0, std^2) as one more rounded fp32 multiply. */
SYN_FN float syn_normal(uint64_t seed, uint32_t tid, uint64_t i, float std, const float* q) {
  float z = syn_std_normal(syn_word(seed, tid, i), q);
  return z * std;
}

/* Elements 4b .. 4b+3 of N(0, std^2): the four words of one Philox block, each turned into
 * a value exactly as syn_normal does (the same values, a quarter of the Philox work). */
SYN_FN void syn_normal4(uint64_t seed, uint32_t tid, uint64_t b, float std, const float* q,
                        float out[4]) {
  syn_u32x4 r = syn_philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), tid, 0u, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
  for (int j = 0; j < 4; ++j) out[j] = syn_std_normal(r.v[j], q) * std;
}

/* U(lo, hi): 24 random bits give an exact fp32 in [0,1); then lo + (hi-lo)*f,
 * with span = hi - lo precomputed by the caller in fp32. */
SYN_FN float syn_uniform(uint64_t seed, uint32_t tid, uint64_t i, float lo, float span) {
  float f = (float)(syn_word(seed, tid, i) >> 8) * (1.0f / 16777216.0f);
  float t = span * f;
  return lo + t;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
SYN_FN uint16_t syn_bf16_rne(float x) {
  uint32_t u = syn_f32_bits(x);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448.
 * E4M3FN: bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF are NaN. */
SYN_FN uint8_t syn_e4m3_rne_sat(float x) {
  uint32_t u = syn_f32_bits(x);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu);         /* NaN */
  float ax = syn_bits_f32(a);
  if (ax >= 464.0f) return (uint8_t)(sign | 0x7Eu);            /* rounds above 448 */
  if (ax < 0.015625f) {                                         /* below 2^-6: subnormal grid 2^-9 */
    float s = ax * 512.0f;                                      /* exact */
    uint32_t m = (uint32_t)s;
    float fr = s - (float)m;                                    /* exact */
    if (fr > 0.5f || (fr == 0.5f && (m & 1u))) m += 1u;
    return (uint8_t)(sign | m);                                 /* m == 8 is the min normal */
  }
  int e = (int)(a >> 23) - 127;                                 /* -6 .. 8 */
  uint32_t mant = a & 0x7FFFFFu;
  uint32_t m = mant >> 20;
  uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) m += 1u;
  if (m == 8u) { m = 0u; e += 1; }
  if (e > 8 || (e == 8 && m == 7u)) return (uint8_t)(sign | 0x7Eu);
  return (uint8_t)(sign | (uint32_t)((e + 7) << 3) | m);
}

/* fp32 (already divided by the block scale) -> symmetric INT8 code: the nearest integer,
 * ties to even (rintf under the default rounding mode), clamped to [-127, 127]. */
SYN_FN int8_t syn_int8_rne_sat(float x) {
  float r = __builtin_rintf(x);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* |x| -> OCP MX E2M1 magnitude code (0..7), round to nearest even, saturating
 * at 6. Representable magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
SYN_FN uint8_t syn_e2m1_rne_sat(float x) {
  uint32_t u = syn_f32_bits(x);
  uint8_t sign = (uint8_t)((u >> 28) & 0x8u);
  float a = syn_bits_f32(u & 0x7FFFFFFFu);
  uint8_t m;
  if (a <= 0.25f) m = 0;
  else if (a < 0.75f) m = 1;
  else if (a <= 1.25f) m = 2;
  else if (a < 1.75f) m = 3;
  else if (a <= 2.5f) m = 4;
  else if (a < 3.5f) m = 5;
  else if (a <= 5.0f) m = 6;
  else m = 7;
  return (uint8_t)(sign | m);
}

/* OCP MX shared scale for a block with max magnitude amax: the e8m0 code of
 * 2^(floor(log2 amax) - 2), where 2 is the largest E2M1 exponent. A zero block
 * gets code 127 (scale 1). */
SYN_FN uint8_t syn_mx_scale_code(float amax) {
  uint32_t a = syn_f32_bits(amax) & 0x7FFFFFFFu;
  if (a == 0u) return 127u;
  int e;
  if ((a >> 23) == 0u) {                 /* fp32 subnormal: find the top bit */
    int top = 22;
    while (top > 0 && !((a >> top) & 1u)) --top;
    e = top - 149;
  } else {
    e = (int)(a >> 23) - 127;
  }
  int x = e - 2 + 127;
  if (x < 0) x = 0;
  if (x > 254) x = 254;
  return (uint8_t)x;
}

/* Multiply by 2^(code-127) exactly (fp32 normal range only, as used here). */
SYN_FN float syn_scale_pow2(float v, int code) {
  int e = code - 127;
  float s = syn_bits_f32((uint32_t)(e + 127) << 23);
  return v * s;
}

#endif
