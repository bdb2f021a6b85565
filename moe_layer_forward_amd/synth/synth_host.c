/*
 * Seeded synthetic inputs for the MoE layer workloads, host side.
 *
 * This module holds no arithmetic of the MoE layer itself: it only turns
 * (seed, stream, index, element) into a number.  The device twin
 * (synth_dev.hip) implements the same definition independently so that a
 * tensor generated on the GPU and the same tensor regenerated here on the
 * host are bit-identical.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
 * ten rounds of two 32x32->64 multiplies (constants 0xD2511F53 and
 * 0xCD9E8D57), with the key advanced by the Weyl constants 0x9E3779B9 and
 * 0xBB67AE85 between rounds.
 *
 * Element definition (used identically on both sides):
 *   key     = (seed, stream)
 *   counter = (elem & 0xffffffff, elem >> 32, index, 0)
 *   r[0..3] = philox4x32_10(counter, key)
 *   d       = sum of the eight 16-bit halves of r[0..3]      (0 .. 524280)
 *   c       = 2*d - 524280                                   (even, |c| <= 524280)
 *   value   = (float)c * scale      one correctly rounded fp32 multiply
 * where scale = fl32(sigma / sqrt(8/3 * (2^32 - 1))) is supplied by the
 * caller, so that value has mean 0 and standard deviation sigma.  The sum of
 * eight uniforms (Irwin-Hall, n = 8) is an approximately normal variate with
 * support +-4.9 sigma; it uses only exact integer arithmetic plus one IEEE
 * multiply, so host and device agree bit for bit.  bf16 output rounds the
 * fp32 value to nearest-even.
 *
 * 4-bit weight storage (synth_quantize_q4) prepares quantized copies of bf16
 * weights, the way a checkpoint is prepared offline; it is input preparation,
 * and its device twin computes the same fp32 operations:
 *   per group of 32 consecutive inputs of a row,
 *     s = f16_rne(max|w| / 7)                 (one IEEE division, then f32->f16)
 *     q = clamp(rint(w / s), -8, 7)           (q = 0 when s == 0)
 *   codes: 8 per 32-bit word, input k of the row in bits 4*(k % 8) of word k / 8,
 *          as 4-bit two's complement; scales: f16 bits, one per group.
 *
 * 8-bit weight storage (synth_quantize_fp8), input preparation of the same kind: per 128 x 128
 * block of a matrix,
 *     s = max|w| / 448                        (one IEEE division; fp32 scale)
 *     c = e4m3(w / s)                         (one IEEE division, then round to nearest even,
 *                                              saturating at +-448; c = 0 when s == 0)
 *   codes: one byte per weight in the matrix's layout, OCP E4M3 (sign, 4 exponent bits with
 *   bias 7, 3 mantissa bits; largest 448); scales: fp32 [rows/128, cols/128].
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
    mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline float synth_value(uint32_t seed, uint32_t stream, uint32_t index, uint64_t elem,
                                float scale) {
  uint32_t ctr[4] = {(uint32_t)elem, (uint32_t)(elem >> 32), index, 0u};
  uint32_t key[2] = {seed, stream};
  uint32_t r[4];
  synth_philox4x32_10(ctr, key, r);
  int32_t d = 0;
  for (int i = 0; i < 4; ++i) d += (int32_t)(r[i] & 0xffffu) + (int32_t)(r[i] >> 16);
  int32_t c = 2 * d - 524280;
  return (float)c * scale;  /* (float)c is exact: |c| < 2^24 */
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7fffu + lsb) >> 16);
}

/* Fill out[i] for i in [0, n): element (elem0 + i) of tensor (seed, stream, index). */
void synth_fill_f32(uint32_t seed, uint32_t stream, uint32_t index, uint64_t elem0, int64_t n,
                    float scale, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_value(seed, stream, index, elem0 + (uint64_t)i, scale);
}

void synth_fill_bf16(uint32_t seed, uint32_t stream, uint32_t index, uint64_t elem0, int64_t n,
                     float scale, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne(synth_value(seed, stream, index, elem0 + (uint64_t)i, scale));
}

/* Rows of a [rows, cols] tensor: row_ids[j] selects the row; out is [n_rows, cols]. */
void synth_fill_rows_bf16(uint32_t seed, uint32_t stream, uint32_t index, int64_t cols,
                          const int64_t *row_ids, int64_t n_rows, float scale, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n_rows; ++j)
    for (int64_t c = 0; c < cols; ++c)
      out[j * cols + c] = f32_to_bf16_rne(
          synth_value(seed, stream, index, (uint64_t)(row_ids[j] * cols + c), scale));
}

void synth_fill_rows_f32(uint32_t seed, uint32_t stream, uint32_t index, int64_t cols,
                         const int64_t *row_ids, int64_t n_rows, float scale, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n_rows; ++j)
    for (int64_t c = 0; c < cols; ++c)
      out[j * cols + c] = synth_value(seed, stream, index, (uint64_t)(row_ids[j] * cols + c), scale);
}

/* IEEE binary32 -> binary16, round to nearest even (overflow to infinity). */
static inline uint16_t f32_to_f16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  const uint32_t sign = (v.u >> 16) & 0x8000u, a = v.u & 0x7fffffffu;
  if (a >= 0x7f800000u) return (uint16_t)(sign | (a > 0x7f800000u ? 0x7e00u : 0x7c00u));
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);      /* >= 65520 rounds to infinity */
  if (a >= 0x38800000u) {                                       /* normal binary16 */
    uint32_t m = a - 0x38000000u;                               /* exponent bias 127 -> 15 */
    m += 0x0fffu + ((m >> 13) & 1u);
    return (uint16_t)(sign | (m >> 13));
  }
  const uint32_t e = a >> 23;                                   /* subnormal binary16 or zero */
  if (e < 102) return (uint16_t)sign;                           /* below half the smallest step */
  const uint32_t mant = (a & 0x7fffffu) | 0x800000u;
  const uint32_t shift = 126u - e;                              /* value * 2^24 = mant >> shift */
  uint32_t n = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (n & 1u))) ++n;
  return (uint16_t)(sign | n);
}

static inline float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  union { float f; uint32_t u; } v;
  if (e == 0x1f) {
    v.u = sign | 0x7f800000u | (m << 13);
  } else if (e) {
    v.u = sign | ((e + 112u) << 23) | (m << 13);
  } else {
    v.f = (float)m * 5.9604644775390625e-08f;                   /* m * 2^-24, exact */
    v.u |= sign;
  }
  return v.f;
}

/* w: [rows, cols] bf16 bits, cols a multiple of 32 -> codes [rows, cols/8], scales [rows, cols/32]. */
void synth_quantize_q4(const uint16_t *w, int64_t n_groups, uint32_t *codes, uint16_t *scales) {
#pragma omp parallel for schedule(static)
  for (int64_t gi = 0; gi < n_groups; ++gi) {
    float v[32], amax = 0.f;
    for (int k = 0; k < 32; ++k) {
      union { uint32_t u; float f; } b;
      b.u = (uint32_t)w[gi * 32 + k] << 16;
      v[k] = b.f;
      const float av = fabsf(v[k]);
      if (av > amax) amax = av;
    }
    const uint16_t s16 = f32_to_f16_rne(amax / 7.0f);
    const float s = f16_to_f32(s16);
    scales[gi] = s16;
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t word = 0;
      for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s > 0.f) {
          const float t = rintf(v[8 * wd + i] / s);
          q = t > 7.f ? 7 : (t < -8.f ? -8 : (int)t);
        }
        word |= ((uint32_t)q & 0xfu) << (4 * i);
      }
      codes[gi * 4 + wd] = word;
    }
  }
}

/* OCP E4M3 code of an fp32 value: round to nearest even, saturating at +-448 (the format has no
 * infinities; S.1111.111 is NaN and never produced).  Every step is exact except the rintf. */
static uint8_t f32_to_e4m3_rne(float t) {
  union { float f; uint32_t u; } b;
  b.f = t;
  const uint8_t sign = (uint8_t)((b.u >> 24) & 0x80u);
  b.u &= 0x7fffffffu;
  const float a = b.f;
  if (!(a < 448.0f)) return sign | 0x7e;
  if (a < 0.015625f) return sign | (uint8_t)rintf(a * 512.0f); /* quantum 2^-9; 8 -> 0x08 = 2^-6 */
  int e = (int)(b.u >> 23) - 127;                                 /* 2^e <= a < 2^(e+1), -6 <= e <= 8 */
  union { float f; uint32_t u; } p;
  p.u = (uint32_t)(127 + 3 - e) << 23;                            /* 2^(3 - e) */
  float q = rintf(a * p.f);                                       /* 8 .. 16 */
  if (q == 16.0f) {
    q = 8.0f;
    ++e;
  }
  return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* w: n_mats matrices [rows, cols] of bf16 bits (rows, cols multiples of 128) ->
 * codes [n_mats, rows, cols] bytes, scales [n_mats, rows/128, cols/128] fp32. */
void synth_quantize_fp8(const uint16_t *w, int64_t n_mats, int64_t rows, int64_t cols, uint8_t *codes,
                        float *scales) {
  const int64_t br = rows / 128, bc = cols / 128, n_blocks = n_mats * br * bc;
#pragma omp parallel for schedule(static)
  for (int64_t bi = 0; bi < n_blocks; ++bi) {
    const int64_t m = bi / (br * bc), r0 = (bi / bc) % br * 128, c0 = bi % bc * 128;
    const int64_t base = m * rows * cols;
    float amax = 0.f;
    for (int64_t r = r0; r < r0 + 128; ++r)
      for (int64_t c = c0; c < c0 + 128; ++c) {
        union { uint32_t u; float f; } b;
        b.u = (uint32_t)w[base + r * cols + c] << 16;
        const float av = fabsf(b.f);
        if (av > amax) amax = av;
      }
    const float s = amax / 448.0f;
    scales[bi] = s;
    for (int64_t r = r0; r < r0 + 128; ++r)
      for (int64_t c = c0; c < c0 + 128; ++c) {
        union { uint32_t u; float f; } b;
        b.u = (uint32_t)w[base + r * cols + c] << 16;
        codes[base + r * cols + c] = s > 0.f ? f32_to_e4m3_rne(b.f / s) : 0;
      }
  }
}
