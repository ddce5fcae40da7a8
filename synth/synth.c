/*
 * Seeded synthetic inputs for the batched decode step: weights, prompts, KV
 * contents, lengths and traces.  This module holds none of the decode
 * arithmetic; it only turns (seed, stream, index) into numbers, and converts
 * them into the storage formats the inputs are handed over in (f32, bf16,
 * Q8_0 planes).  Both the CPU oracle and the GPU path consume its output.
 *
 * Generator: Philox4x32-10, the counter-based generator published by Salmon,
 * Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3",
 * SC'11).  Element i of stream s under seed k uses counter
 * (i/4 low word, i/4 high word, s low word, s high word) and key
 * (k low word, k high word); the output word i%4 is element i's draw.
 * Normal draws use the Box-Muller transform on the word pairs (0,1), (2,3),
 * computed in double precision.  Everything is a pure function of the
 * element index, so the OpenMP split does not change any value.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(const uint32_t in[4], uint64_t seed, uint32_t out[4]) {
  uint32_t x0 = in[0], x1 = in[1], x2 = in[2], x3 = in[3];
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * x0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

static inline void block_words(uint64_t seed, uint64_t stream, uint64_t blk, uint32_t w[4]) {
  uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  philox4x32_10(c, seed, w);
}

/* Four standard normals from one Philox block (Box-Muller, double precision). */
static inline void block_normals(uint64_t seed, uint64_t stream, uint64_t blk, double z[4]) {
  uint32_t w[4];
  block_words(seed, stream, blk, w);
  const double two_pi = 6.283185307179586476925286766559;
  for (int p = 0; p < 2; ++p) {
    double u1 = ((double)w[2 * p] + 1.0) * (1.0 / 4294967296.0); /* (0, 1] */
    double u2 = (double)w[2 * p + 1] * (1.0 / 4294967296.0);     /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double s, c;
    sincos(two_pi * u2, &s, &c);
    z[2 * p] = r * c;
    z[2 * p + 1] = r * s;
  }
}

/* f32 -> bf16 bits, round to nearest even (NaN kept quiet). */
static inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static inline float bf16_bits_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* f32 -> IEEE binary16 bits, round to nearest even, with subnormals and
 * overflow to infinity. */
static inline uint16_t f32_to_f16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t ex = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (ex == 0xffu) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
  int e = (int)ex - 127 + 15;
  if (e >= 31) return (uint16_t)(sign | 0x7c00u);
  if (e <= 0) {
    if (e < -10) return (uint16_t)sign;
    man |= 0x800000u;
    int shift = 14 - e; /* 24-bit significand -> (11 + e - 1) bits */
    uint32_t half = man >> shift;
    uint32_t rem = man & ((1u << shift) - 1u);
    uint32_t mid = 1u << (shift - 1);
    if (rem > mid || (rem == mid && (half & 1u))) half += 1u;
    return (uint16_t)(sign | half);
  }
  uint32_t half = (uint32_t)(e << 10) | (man >> 13);
  uint32_t rem = man & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (half & 1u))) half += 1u; /* may carry into exponent: correct */
  return (uint16_t)(sign | half);
}

static inline float f16_bits_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t ex = (h >> 10) & 0x1fu;
  uint32_t man = h & 0x3ffu;
  uint32_t u;
  if (ex == 0) {
    if (man == 0) {
      u = sign;
    } else {
      int e = -1;
      do { man <<= 1; ++e; } while (!(man & 0x400u));
      u = sign | ((uint32_t)(127 - 15 - e) << 23) | ((man & 0x3ffu) << 13);
    }
  } else if (ex == 31) {
    u = sign | 0x7f800000u | (man << 13);
  } else {
    u = sign | ((ex - 15 + 127) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ---- exported API --------------------------------------------------------- */

/* Blocks of four draws cover elements [first, first + n); each block is computed once. */
#define FOR_BLOCKS(first, n, BODY)                                                   \
  do {                                                                               \
    uint64_t b0_ = (first) >> 2, b1_ = ((first) + (uint64_t)(n) + 3) >> 2;           \
    _Pragma("omp parallel for schedule(static)")                                     \
    for (int64_t bb_ = (int64_t)b0_; bb_ < (int64_t)b1_; ++bb_) {                    \
      uint64_t blk = (uint64_t)bb_;                                                  \
      BODY                                                                           \
    }                                                                                \
  } while (0)

/* out[j] = (float)(scale * N_{first+j}) */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, double scale, float* out) {
  if (n <= 0) return;
  FOR_BLOCKS(first, n, {
    double z[4];
    block_normals(seed, stream, blk, z);
    for (int c = 0; c < 4; ++c) {
      uint64_t i = 4 * blk + (uint64_t)c;
      if (i >= first && i < first + (uint64_t)n) out[i - first] = (float)(scale * z[c]);
    }
  });
}

/* out[j] = bf16_rne((float)(scale * N_{first+j})) — the f32 draw, then rounded. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, double scale, uint16_t* out) {
  if (n <= 0) return;
  FOR_BLOCKS(first, n, {
    double z[4];
    block_normals(seed, stream, blk, z);
    for (int c = 0; c < 4; ++c) {
      uint64_t i = 4 * blk + (uint64_t)c;
      if (i >= first && i < first + (uint64_t)n) out[i - first] = f32_to_bf16_bits((float)(scale * z[c]));
    }
  });
}

/* Raw 32-bit words: out[j] = word_{first+j}. */
void synth_words(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = first + (uint64_t)j;
    uint32_t w[4];
    block_words(seed, stream, i >> 2, w);
    out[j] = w[i & 3];
  }
}

/* Uniform integers in [lo, lo + span) by the multiply-shift map of one word. */
void synth_uniform_int(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, int64_t lo, uint32_t span,
                       int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = first + (uint64_t)j;
    uint32_t w[4];
    block_words(seed, stream, i >> 2, w);
    out[j] = (int32_t)(lo + (int64_t)(((uint64_t)w[i & 3] * span) >> 32));
  }
}

/* Uniform doubles in (0, 1): (word + 0.5) / 2^32. */
void synth_uniform_open01(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, double* out) {
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = first + (uint64_t)j;
    uint32_t w[4];
    block_words(seed, stream, i >> 2, w);
    out[j] = ((double)w[i & 3] + 0.5) * (1.0 / 4294967296.0);
  }
}

void synth_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_bits(in[j]);
}

void synth_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = bf16_bits_to_f32(in[j]);
}

void synth_f32_to_f16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_f16_bits(in[j]);
}

void synth_f16_to_f32(const uint16_t* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f16_bits_to_f32(in[j]);
}

/*
 * Q8_0 storage of a [rows, k] f32 matrix, blocks of 32 along k (k % 32 == 0):
 *   d = max|w| / 127 (f32);  q_i = clamp(round-half-away(w_i / d), -127, 127);
 *   stored scale = f16_rne(d); an all-zero block stores d = 0 and q = 0.
 * Two planes: q [rows, k] int8 and scale [rows, k/32] binary16 bits.
 */
void synth_q8_0_quantize(const float* w, int64_t rows, int64_t k, int8_t* q, uint16_t* scale) {
  int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* src = w + r * k + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(src[i]);
        if (a > amax) amax = a;
      }
      float d = amax / 127.0f;
      int8_t* dst = q + r * k + b * 32;
      if (d == 0.0f) {
        for (int i = 0; i < 32; ++i) dst[i] = 0;
      } else {
        for (int i = 0; i < 32; ++i) {
          float v = roundf(src[i] / d); /* roundf: half away from zero */
          if (v > 127.0f) v = 127.0f;
          if (v < -127.0f) v = -127.0f;
          dst[i] = (int8_t)v;
        }
      }
      scale[r * nb + b] = f32_to_f16_bits(d);
    }
  }
}
