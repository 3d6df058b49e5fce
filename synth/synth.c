/*
 * synth.c -- seeded synthetic inputs for the quantized decode path.
 *
 * Test and benchmark infrastructure.  This file only produces input bytes:
 * it holds none of the decode arithmetic (no dequantization, no dot
 * products, no normalisation).  Both the fp64 oracle and the HIP path are fed
 * from the buffers it fills, so neither side generates its own inputs.
 *
 * Random numbers: a counter-based SplitMix64 stream (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  Word i of
 * the stream with key k is mix(k + (i + 1) * 0x9E3779B97F4A7C15), the
 * (i+1)-th output of a SplitMix64 generator whose state starts at k.  Any
 * tensor, block or element can therefore be regenerated independently and
 * in parallel.
 *
 * Block byte layouts written here (fields in order, little endian):
 *   Q8_0  34 B / 32 weights : f16 d, 32 x int8 q        (q uniform in -127..127)
 *   Q4_0  18 B / 32 weights : f16 d, 16 B of nibbles    (bytes uniform)
 *   Q4_K 144 B / 256 weights: f16 d, f16 dmin, 12 B packed 6-bit scales/mins,
 *                             128 B of nibbles          (bytes uniform)
 *   Q6_K 210 B / 256 weights: 128 B low nibbles, 64 B high 2-bit fields,
 *                             16 x int8 scales, f16 d   (bytes uniform)
 * Every f16 scale (d, dmin) is drawn uniform in [1e-3, 1e-2] in double and
 * rounded to the nearest f16 (ties to even); the stored f16 is the truth.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t sm_word(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * SM_GAMMA);
}

/* Uniform double in [0, 1) with 53 random bits. */
static inline double sm_u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

/* Key of a sub-stream: hash of (seed, a, b, c). */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = sm_mix(seed + SM_GAMMA);
  k = sm_mix(k ^ sm_mix(a + 2 * SM_GAMMA));
  k = sm_mix(k ^ sm_mix(b + 3 * SM_GAMMA));
  k = sm_mix(k ^ sm_mix(c + 4 * SM_GAMMA));
  return k;
}

uint64_t synth_word(uint64_t key, uint64_t i) { return sm_word(key, i); }

/* double -> IEEE binary16 bits, round to nearest, ties to even. */
uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7e00u;
  if (a >= 65520.0) return sign | 0x7c00u; /* rounds to infinity */
  if (a < 0x1p-14) {                        /* subnormal: units of 2^-24 */
    double m = nearbyint(a * 0x1p24);       /* 1024 becomes the smallest normal */
    return sign | (uint16_t)m;
  }
  int e;
  double f = frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
  double m = nearbyint(ldexp(f, 11)); /* 11 significant bits, in [1024, 2048] */
  int E = e - 1 + 15;
  if (m == 2048.0) { m = 1024.0; E += 1; }
  if (E >= 31) return sign | 0x7c00u;
  return sign | (uint16_t)(E << 10) | (uint16_t)((int)m - 1024);
}

/* Standard normal number i of a stream (Box-Muller, cosine branch), using
 * words 2i and 2i+1. */
static inline double sm_normal(uint64_t key, uint64_t i) {
  double u1 = 1.0 - sm_u01(sm_word(key, 2 * i)); /* (0, 1] */
  double u2 = sm_u01(sm_word(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline void put16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }

static inline void put_word_bytes(uint8_t* p, uint64_t w, int n) {
  for (int i = 0; i < n; ++i) p[i] = (uint8_t)(w >> (8 * i));
}

static inline uint16_t scale_f16(uint64_t w, double lo, double hi) {
  return synth_f64_to_f16(lo + (hi - lo) * sm_u01(w));
}

enum { SY_Q8_0 = 0, SY_Q4_0 = 1, SY_Q4_K = 2, SY_Q6_K = 3, SY_Q5_K = 4, SY_F16 = 5, SY_F32 = 6 };
#define SY_WORDS_PER_BLOCK 32u

int synth_block_elems(int fmt) {
  switch (fmt) {
    case SY_Q8_0: case SY_Q4_0: return 32;
    case SY_Q4_K: case SY_Q6_K: case SY_Q5_K: return 256;
    case SY_F16: case SY_F32: return 1;
  }
  return 0;
}

int synth_block_bytes(int fmt) {
  switch (fmt) {
    case SY_Q8_0: return 34;
    case SY_Q4_0: return 18;
    case SY_Q4_K: return 144;
    case SY_Q6_K: return 210;
    case SY_Q5_K: return 176;
    case SY_F16: return 2;
    case SY_F32: return 4;
  }
  return 0;
}

/* One block of format fmt from words [b*32, b*32+32) of the stream. */
static void fill_block(int fmt, uint64_t key, uint64_t b, double dlo, double dhi, uint8_t* out) {
  const uint64_t w0 = b * SY_WORDS_PER_BLOCK;
  switch (fmt) {
    case SY_Q8_0: {
      put16(out, scale_f16(sm_word(key, w0), dlo, dhi));
      for (int j = 0; j < 16; ++j) {
        uint64_t w = sm_word(key, w0 + 1 + j);
        for (int h = 0; h < 2; ++h) {
          uint64_t u = (w >> (32 * h)) & 0xffffffffULL;
          int q = (int)((u * 255ULL) >> 32) - 127; /* -127..127 */
          out[2 + 2 * j + h] = (uint8_t)(int8_t)q;
        }
      }
      break;
    }
    case SY_Q4_0:
      put16(out, scale_f16(sm_word(key, w0), dlo, dhi));
      put_word_bytes(out + 2, sm_word(key, w0 + 1), 8);
      put_word_bytes(out + 10, sm_word(key, w0 + 2), 8);
      break;
    case SY_Q4_K:
      put16(out, scale_f16(sm_word(key, w0), dlo, dhi));
      put16(out + 2, scale_f16(sm_word(key, w0 + 1), dlo, dhi));
      put_word_bytes(out + 4, sm_word(key, w0 + 2), 8);
      put_word_bytes(out + 12, sm_word(key, w0 + 3), 4);
      for (int j = 0; j < 16; ++j) put_word_bytes(out + 16 + 8 * j, sm_word(key, w0 + 4 + j), 8);
      break;
    case SY_Q5_K:
      put16(out, scale_f16(sm_word(key, w0), dlo, dhi));
      put16(out + 2, scale_f16(sm_word(key, w0 + 1), dlo, dhi));
      put_word_bytes(out + 4, sm_word(key, w0 + 2), 8);                                  /* scales */
      put_word_bytes(out + 12, sm_word(key, w0 + 3), 4);
      for (int j = 0; j < 20; ++j) put_word_bytes(out + 16 + 8 * j, sm_word(key, w0 + 4 + j), 8); /* qh, qs */
      break;
    case SY_F16: /* unquantized weights: N(0, (10 dhi)^2), i.e. std 0.1 at the default scale range */
      put16(out, synth_f64_to_f16(10.0 * dhi * sm_normal(key, b)));
      break;
    case SY_F32: {
      float f = (float)(10.0 * dhi * sm_normal(key, b));
      uint32_t u;
      memcpy(&u, &f, 4);
      put_word_bytes(out, u, 4);
      break;
    }
    case SY_Q6_K:
      for (int j = 0; j < 24; ++j) put_word_bytes(out + 8 * j, sm_word(key, w0 + j), 8); /* ql, qh */
      put_word_bytes(out + 192, sm_word(key, w0 + 24), 8);                              /* scales */
      put_word_bytes(out + 200, sm_word(key, w0 + 25), 8);
      put16(out + 208, scale_f16(sm_word(key, w0 + 26), dlo, dhi));
      break;
  }
}

/* Fill blocks [b0, b0 + nblocks) of a quantized tensor; block b lands at
 * out + (b - b0) * block_bytes.  Returns 0, or -1 for an unknown format. */
int synth_quant(int fmt, uint64_t key, int64_t b0, int64_t nblocks, double dlo, double dhi, uint8_t* out) {
  int bb = synth_block_bytes(fmt);
  if (bb == 0 || nblocks < 0 || b0 < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nblocks; ++i) fill_block(fmt, key, (uint64_t)(b0 + i), dlo, dhi, out + i * bb);
  return 0;
}

/* out[i] = float(mean + std * N_i), elements [i0, i0 + n) of the stream. */
void synth_normal_f32(uint64_t key, int64_t i0, int64_t n, double mean, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * sm_normal(key, (uint64_t)(i0 + i)));
}

/* out[i] = f16 bits of N_i (round to nearest even). */
void synth_normal_f16(uint64_t key, int64_t i0, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f64_to_f16(sm_normal(key, (uint64_t)(i0 + i)));
}

/* out[i] uniform integer in [0, bound). */
void synth_uint_below(uint64_t key, int64_t n, uint32_t bound, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint64_t u = sm_word(key, (uint64_t)i) >> 32;
    out[i] = (int32_t)((u * (uint64_t)bound) >> 32);
  }
}
