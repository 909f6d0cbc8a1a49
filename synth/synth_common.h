/*
 * synth_common.h -- seeded synthetic expert-blob generator, shared by the
 * host build (gen_host.c, gcc) and the device build (gen_dev.hip, hipcc).
 *
 * This is test and benchmark input generation only: it holds none of the
 * MoE method's arithmetic (no dequantisation, no dot products).  It writes
 * random bytes in the expert-blob format that include/moe.h documents:
 * codes are uniform random bits, every (scale, bias) word holds a bf16 scale
 * drawn from U(s_lo, s_hi) and a bf16 bias from U(z_lo, z_hi).
 *
 * Generator: SplitMix64 in counter mode (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014): the stream key
 * of (seed, layer, expert) is mix(seed ^ mix(layer << 32 | expert)); word i of
 * the blob uses mix(key + (i + 1) * golden_gamma).
 * Every operation below is an exact integer operation or a single
 * IEEE-754 round-to-nearest fp32 operation, so the host and device builds
 * produce identical bytes (the callers forbid FMA contraction).
 */
#ifndef SYNTH_COMMON_H_
#define SYNTH_COMMON_H_

#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t expert) {
  return synth_mix64(seed ^ synth_mix64(((uint64_t)layer << 32) | expert));
}

SYNTH_FN uint64_t synth_word64(uint64_t key, uint64_t i) {
  return synth_mix64(key + (i + 1) * SYNTH_GAMMA);
}

/* fp32 -> bf16 bit pattern, round to nearest even (finite inputs only). */
SYNTH_FN uint16_t synth_f32_to_bf16(uint32_t f) {
  uint32_t lsb = (f >> 16) & 1u;
  return (uint16_t)((f + 0x7FFFu + lsb) >> 16);
}

/* Blob geometry of the format in include/moe.h, written out here on its own
 * (the generator shares no code with the library or the oracle).
 * Returns the number of 32-bit words in the blob and fills the word offsets
 * of the six sections. */
SYNTH_FN uint64_t synth_layout(int H, int I, int bits, uint64_t off[7]) {
  const uint64_t cpw = 32u / (uint32_t)bits;
  const uint64_t g = 64;
  uint64_t sz[6];
  sz[0] = (uint64_t)I * (H / cpw);    /* gate codes */
  sz[1] = (uint64_t)I * (H / cpw);    /* up codes */
  sz[2] = (uint64_t)H * (I / cpw);    /* down codes */
  sz[3] = (uint64_t)I * (H / g);      /* gate (scale, bias) */
  sz[4] = (uint64_t)I * (H / g);      /* up (scale, bias) */
  sz[5] = (uint64_t)H * (I / g);      /* down (scale, bias) */
  uint64_t o = 0;
  for (int s = 0; s < 6; ++s) {
    off[s] = o;
    o += sz[s];
    o = (o + 63) & ~(uint64_t)63; /* 256-byte alignment = 64 words */
  }
  off[6] = o;
  return o;
}


/* Uniform draw in [lo, hi) from 24 random bits, as bf16: u = k * 2^-24 (exact),
 * v = lo + (hi - lo) * u with three individually rounded fp32 operations. */
#ifdef __HIP_DEVICE_COMPILE__
#define SYNTH_FSUB(a, b) __fsub_rn((a), (b))
#define SYNTH_FMUL(a, b) __fmul_rn((a), (b))
#define SYNTH_FADD(a, b) __fadd_rn((a), (b))
#else
#define SYNTH_FSUB(a, b) ((a) - (b))
#define SYNTH_FMUL(a, b) ((a) * (b))
#define SYNTH_FADD(a, b) ((a) + (b))
#endif

SYNTH_FN uint16_t synth_uniform_bf16(uint32_t k24, float lo, float hi) {
  float u = (float)k24 * 5.9604644775390625e-08f; /* 2^-24 */
  float d = SYNTH_FSUB(hi, lo);
  float t = SYNTH_FMUL(d, u);
  float v = SYNTH_FADD(lo, t);
  union { float f; uint32_t u; } c;
  c.f = v;
  return synth_f32_to_bf16(c.u);
}

/* Parameters of one synthetic blob family. */
typedef struct {
  uint64_t seed;
  int32_t H, I, bits;
  float s_lo, s_hi, z_lo, z_hi;
} synth_params;

/* Word i of the blob of (layer, expert); `off` from synth_layout. */
SYNTH_FN uint32_t synth_blob_word(const synth_params *p, uint64_t key,
                                  const uint64_t off[7], uint64_t i) {
  if (i >= off[6]) return 0u;
  uint64_t v = synth_word64(key, i);
  int sec = 0;
  while (sec < 5 && i >= off[sec + 1]) ++sec;
  /* words between a section's end and the next aligned start are padding */
  uint64_t sz;
  {
    const uint64_t cpw = 32u / (uint32_t)p->bits;
    uint64_t rows = (sec == 2 || sec == 5) ? (uint64_t)p->H : (uint64_t)p->I;
    uint64_t cols = (sec == 2 || sec == 5) ? (uint64_t)p->I : (uint64_t)p->H;
    sz = rows * (sec < 3 ? cols / cpw : cols / 64);
  }
  if (i - off[sec] >= sz) return 0u;
  if (sec < 3) return (uint32_t)(v >> 32);
  uint16_t s = synth_uniform_bf16((uint32_t)(v >> 40), p->s_lo, p->s_hi);
  uint16_t z = synth_uniform_bf16((uint32_t)((v >> 8) & 0xFFFFFFu), p->z_lo, p->z_hi);
  return (uint32_t)s | ((uint32_t)z << 16);
}

#endif /* SYNTH_COMMON_H_ */
