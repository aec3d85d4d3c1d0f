/*
 * Seeded synthetic inputs for the skinny quantized product (weights and
 * activations). This module is shared by the oracle side and the HIP side as
 * their common input source; it holds none of the product's arithmetic: it
 * does not decode or dequantize anything.
 *
 * Distributions (the workload the pages describe, as synthetic stand-ins for
 * the Q4_K_M GGUF weights of the 27B model of "sixi-asi 0.9", section
 * "Numbers"):
 *   - every 144-byte super-block: bytes 4..143 are uniform random bytes. Because
 *     the 6-bit scales, the 6-bit mins and the 4-bit quants occupy disjoint bit
 *     fields of those bytes, each of them is then uniform over its range
 *     (0..63, 0..63, 0..15) whatever the packing, so the generator needs no
 *     knowledge of the packing.
 *   - bytes 0..1 and 2..3: the little-endian binary16 encodings of
 *     d = f16_rne(|z1| * 1e-2) and dmin = f16_rne(|z2| * 1e-2), z ~ N(0,1).
 *   - activations: x = f32_rne(scale * z), z ~ N(0,1).
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: word i of stream (seed, tensor, field) is the (i+1)-th output of
 * SplitMix64 started from a key mixed from (seed, tensor, field). Normals come
 * from the Box-Muller transform on two 53-bit uniforms, in double precision.
 * Every value is a pure function of (seed, tensor, field, index), so the output
 * does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

enum {
  FIELD_BYTES = 1, FIELD_D = 2, FIELD_DMIN = 3, FIELD_X = 4, FIELD_FP4_ELEMS = 5,
  FIELD_FP4_SCALES = 6, FIELD_INT4_CODES = 7, FIELD_INT4_SCALES = 8
};

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t sm_key(uint64_t seed, uint64_t tensor, uint64_t field) {
  return sm_mix(sm_mix(seed + SM_GAMMA) ^ (tensor * 0xD1B54A32D192ED03ULL) ^
                (field * 0x8CB92BA72F3D8DD7ULL));
}

static inline uint64_t sm_word(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * SM_GAMMA);
}

/* Standard normal number i of a stream: Box-Muller on words 2i and 2i+1. */
static inline double sm_normal(uint64_t key, uint64_t i) {
  const double two53 = 9007199254740992.0;
  double u1 = ((double)(sm_word(key, 2 * i) >> 11) + 1.0) / two53; /* (0, 1] */
  double u2 = (double)(sm_word(key, 2 * i + 1) >> 11) / two53;      /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* IEEE 754 binary64 -> binary16, round to nearest, ties to even. */
uint16_t synth_f64_to_f16(double v) {
  uint64_t b;
  memcpy(&b, &v, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t man = b & 0xFFFFFFFFFFFFFULL;
  if (ex == 0x7FF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
  if (ex == 0) return sign; /* zero or binary64 subnormal: rounds to zero */
  int e = ex - 1023;
  uint64_t sig = man | (1ULL << 52); /* value = sig * 2^(e-52) */
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  if (shift >= 64) return sign;
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ULL << shift) - 1);
  uint64_t half = 1ULL << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  if (e >= -14) {
    int E = e + 15;
    if (q == 2048) { q = 1024; E++; }
    if (E >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (E << 10) | (uint16_t)(q - 1024));
  }
  return (uint16_t)(sign | q); /* subnormal; q == 1024 is the smallest normal */
}

/* W: n_rows x (K/256) super-blocks of 144 bytes, row-major, blocks along K. */
int synth_weights(uint64_t seed, uint64_t tensor, int64_t n_rows, int64_t K,
                  uint8_t* out) {
  if (K <= 0 || K % 256 != 0 || n_rows < 0 || !out) return -1;
  const int64_t nblk = n_rows * (K / 256);
  const uint64_t kb = sm_key(seed, tensor, FIELD_BYTES);
  const uint64_t kd = sm_key(seed, tensor, FIELD_D);
  const uint64_t km = sm_key(seed, tensor, FIELD_DMIN);
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < nblk; ++blk) {
    uint8_t* p = out + blk * 144;
    for (int w = 0; w < 18; ++w) {
      uint64_t r = sm_word(kb, (uint64_t)blk * 18 + (uint64_t)w);
      for (int t = 0; t < 8; ++t) p[8 * w + t] = (uint8_t)(r >> (8 * t));
    }
    uint16_t d = synth_f64_to_f16(fabs(sm_normal(kd, (uint64_t)blk)) * 1e-2);
    uint16_t dm = synth_f64_to_f16(fabs(sm_normal(km, (uint64_t)blk)) * 1e-2);
    p[0] = (uint8_t)(d & 0xFF);
    p[1] = (uint8_t)(d >> 8);
    p[2] = (uint8_t)(dm & 0xFF);
    p[3] = (uint8_t)(dm >> 8);
  }
  return 0;
}

/* Block-scaled FP4 weights in the usual two-array layout: elems n_rows x K/2
   bytes of 4-bit codes (uniform random bytes, two codes per byte), scales
   n_rows x K/16 bytes, one 8-bit scale code per 16 elements with a uniform
   exponent field 0..14 and mantissa field 0..7 and the sign bit clear (so no
   code is NaN; zero and subnormal scales occur). Only random bit fields: the
   values these codes stand for are not computed here. */
int synth_nvfp4(uint64_t seed, uint64_t tensor, int64_t n_rows, int64_t K, uint8_t* elems,
                uint8_t* scales) {
  if (K <= 0 || K % 16 != 0 || n_rows < 0 || !elems || !scales) return -1;
  const int64_t ne = n_rows * (K / 2), ns = n_rows * (K / 16);
  const uint64_t ke = sm_key(seed, tensor, FIELD_FP4_ELEMS);
  const uint64_t ks = sm_key(seed, tensor, FIELD_FP4_SCALES);
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < (ne + 7) / 8; ++w) {
    const uint64_t r = sm_word(ke, (uint64_t)w);
    for (int t = 0; t < 8 && 8 * w + t < ne; ++t) elems[8 * w + t] = (uint8_t)(r >> (8 * t));
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < ns; ++i) {
    const uint64_t r = sm_word(ks, (uint64_t)i);
    scales[i] = (uint8_t)(((r % 15u) << 3) | ((r >> 8) & 7u));
  }
  return 0;
}

/* Plain 4-bit integer weights in the usual two-array layout: codes n_rows x
   K/2 bytes (uniform random bytes, two 4-bit codes per byte), scales n_rows x
   K/128 binary16 bit patterns, one per 128 elements, f16_rne(|z| * 1e-2) like
   the super-blocks' d and dmin. Only random fields: the values the codes
   stand for are not computed here. */
int synth_int4(uint64_t seed, uint64_t tensor, int64_t n_rows, int64_t K, uint8_t* codes,
               uint16_t* scales) {
  if (K <= 0 || K % 128 != 0 || n_rows < 0 || !codes || !scales) return -1;
  const int64_t nc = n_rows * (K / 2), ns = n_rows * (K / 128);
  const uint64_t kc = sm_key(seed, tensor, FIELD_INT4_CODES);
  const uint64_t ks = sm_key(seed, tensor, FIELD_INT4_SCALES);
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < (nc + 7) / 8; ++w) {
    const uint64_t r = sm_word(kc, (uint64_t)w);
    for (int t = 0; t < 8 && 8 * w + t < nc; ++t) codes[8 * w + t] = (uint8_t)(r >> (8 * t));
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < ns; ++i)
    scales[i] = synth_f64_to_f16(fabs(sm_normal(ks, (uint64_t)i)) * 1e-2);
  return 0;
}

/* x: M x K fp32, row-major, x[m][k] = f32_rne(scale * z). */
int synth_acts(uint64_t seed, uint64_t tensor, int64_t M, int64_t K, double scale,
               float* out) {
  if (M < 0 || K < 0 || !out) return -1;
  const uint64_t kx = sm_key(seed, tensor, FIELD_X);
  const int64_t n = M * K;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(scale * sm_normal(kx, (uint64_t)i));
  return 0;
}

/* n values f32_rne(scale * z), z ~ N(0,1), of stream `field` (generic inputs). */
int synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t field, int64_t n, double scale,
                     float* out) {
  if (n < 0 || (n && !out)) return -1;
  const uint64_t key = sm_key(seed, tensor, field);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(scale * sm_normal(key, (uint64_t)i));
  return 0;
}

/* n values f32_rne(lo + (hi - lo) * w), w = (53 high bits of the word) / 2^53 in [0, 1). */
int synth_uniform_f32(uint64_t seed, uint64_t tensor, uint64_t field, int64_t n, double lo,
                      double hi, float* out) {
  if (n < 0 || (n && !out)) return -1;
  const uint64_t key = sm_key(seed, tensor, field);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double w = (double)(sm_word(key, (uint64_t)i) >> 11) * 0x1.0p-53;
    out[i] = (float)(lo + (hi - lo) * w);
  }
  return 0;
}

/* Raw stream access, used by the tests of the generator itself. */
uint64_t synth_word(uint64_t seed, uint64_t tensor, uint64_t field, uint64_t i) {
  return sm_word(sm_key(seed, tensor, field), i);
}

double synth_normal(uint64_t seed, uint64_t tensor, uint64_t field, uint64_t i) {
  return sm_normal(sm_key(seed, tensor, field), i);
}

int synth_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
