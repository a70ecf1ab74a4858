/*
 * synth_core.h -- seeded, counter-based synthetic input generator.
 *
 * This module produces the inputs of the MoE decode layer (activations, bf16
 * weight matrices, MXFP4-quantised expert blobs, the Zipf-like router bias).
 * It is shared by the CPU oracle and the GPU library alike, and therefore
 * holds none of the layer's arithmetic: there is no decode of an MXFP4 value,
 * no dot product, no routing and no activation function in here.  The only
 * numeric formats it touches are the ones it has to *write*: bf16 (round to
 * nearest even of an fp32 value) and the MXFP4 encoding (OCP Microscaling
 * Formats v1.0: E2M1 element codes with one E8M0 shared scale per block of 32).
 *
 * The same functions are compiled for the host (gcc, libsynth_host.so) and for
 * the device (hipcc, libsynth_dev.so) so that a tensor of any size can be
 * generated in HBM in milliseconds and any slice of it regenerated on the
 * host, byte for byte.  Every step is integer arithmetic or a single
 * correctly rounded fp32 multiply, so both builds produce identical bytes.
 *
 * Definitions
 *   mix64(z)           SplitMix64 finaliser (Steele, Lea, Flood: "Fast
 *                      splittable pseudorandom number generators", OOPSLA 2014):
 *                      z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                      z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key(seed, tag)     = mix64(seed * GAMMA + tag), GAMMA = 0x9E3779B97F4A7C15.
 *   draw(key, i)       = mix64(key + (i + 1) * GAMMA)    (counter-based stream).
 *   gauss_int(key, i)  = 2 * S - 8 * 65535, where S is the sum of the eight
 *                      16-bit fields of draw(key, 2i) and draw(key, 2i+1)
 *                      (Irwin-Hall sum of 8 uniforms: mean 0, standard
 *                      deviation 65536 * sqrt(8/3) up to O(2^-32)).
 *   normal(key, i, m)  = (float)gauss_int * m with m = (float)(sigma /
 *                      (65536 * sqrt(8/3))): approximately N(0, sigma^2),
 *                      truncated at 4.9 sigma.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

/* Tensor kinds used to build tags. A tag names one tensor of one layer. */
enum {
  SYN_KIND_X = 1,        /* activations, bf16 [B][H]                         */
  SYN_KIND_ROUTER = 2,   /* router weight, bf16 [E][H]                       */
  SYN_KIND_BIASPERM = 3, /* permutation behind the Zipf-like router bias     */
  SYN_KIND_SHARED = 4,   /* shared expert, matrix 0 gate, 1 up, 2 down       */
  SYN_KIND_EXPERT = 5,   /* routed expert e, matrix 0 gate, 1 up, 2 down     */
  SYN_KIND_DENSE = 6,    /* dense bf16 block matrix j of a layer             */
  SYN_KIND_H0 = 7        /* fp32 residual stream entering a layer stack      */
};

SYN_FN uint64_t syn_tag(uint32_t layer, uint32_t kind, uint32_t expert, uint32_t matrix) {
  return ((uint64_t)(layer & 0xFFFFu) << 48) | ((uint64_t)(kind & 0xFFu) << 40) |
         ((uint64_t)(expert & 0xFFFFFFFu) << 8) | (uint64_t)(matrix & 0xFFu);
}

SYN_FN uint64_t syn_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYN_FN uint64_t syn_key(uint64_t seed, uint64_t tag) { return syn_mix64(seed * SYN_GAMMA + tag); }

SYN_FN uint64_t syn_draw(uint64_t key, uint64_t i) { return syn_mix64(key + (i + 1) * SYN_GAMMA); }

SYN_FN int32_t syn_gauss_int(uint64_t key, uint64_t i) {
  uint64_t a = syn_draw(key, 2 * i), b = syn_draw(key, 2 * i + 1);
  int32_t s = (int32_t)(a & 0xFFFF) + (int32_t)((a >> 16) & 0xFFFF) + (int32_t)((a >> 32) & 0xFFFF) +
              (int32_t)(a >> 48) + (int32_t)(b & 0xFFFF) + (int32_t)((b >> 16) & 0xFFFF) +
              (int32_t)((b >> 32) & 0xFFFF) + (int32_t)(b >> 48);
  return 2 * s - 8 * 65535;
}

SYN_FN float syn_normal(uint64_t key, uint64_t i, float mult) { return (float)syn_gauss_int(key, i) * mult; }

SYN_FN uint32_t syn_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

SYN_FN float syn_bits_f32(uint32_t u) {
  union { float f; uint32_t u; } c;
  c.u = u;
  return c.f;
}

/* fp32 -> bf16, round to nearest, ties to even (inputs here are finite). */
SYN_FN uint16_t syn_bf16_rne(float f) {
  uint32_t u = syn_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/*
 * MXFP4 encoding of one block of 32 fp32 values (OCP MX v1.0, E2M1 elements).
 * Shared exponent: floor(log2(amax)) - 2 (2 = largest E2M1 exponent), clamped
 * to [-127, 127]; the scale byte is that exponent + 127.  An all-zero block
 * gets scale byte 127 and zero codes.  Each value divided by the scale (an
 * exact power-of-two multiply) is rounded to nearest-even on the E2M1
 * magnitude grid {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.  Rounding is
 * done by comparing against the midpoints of the grid: a value strictly above
 * a midpoint moves up, a value equal to it moves to the code whose mantissa
 * bit is 0.  Sign is bit 3 of the code.  Element 2i goes to bits 3:0 of byte
 * i, element 2i+1 to bits 7:4.  Values here are normal floats well inside the
 * fp32 range; the generator never emits scale byte 0xFF.
 */
SYN_FN uint8_t syn_e2m1_round(float a /* |v| / scale, >= 0 */) {
  uint8_t c = 0;
  c += (a > 0.25f);  /* 0   | 0.5 : tie goes to code 0 (even)  */
  c += (a >= 0.75f); /* 0.5 | 1   : tie goes to code 2         */
  c += (a > 1.25f);  /* 1   | 1.5 : tie goes to code 2         */
  c += (a >= 1.75f); /* 1.5 | 2   : tie goes to code 4         */
  c += (a > 2.5f);   /* 2   | 3   : tie goes to code 4         */
  c += (a >= 3.5f);  /* 3   | 4   : tie goes to code 6         */
  c += (a > 5.0f);   /* 4   | 6   : tie goes to code 6         */
  return c;
}

SYN_FN void syn_mxfp4_block(const float* v, uint8_t* codes16, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = v[i] < 0.0f ? -v[i] : v[i];
    amax = a > amax ? a : amax;
  }
  if (amax == 0.0f) {
    for (int i = 0; i < 16; ++i) codes16[i] = 0;
    *scale = 127;
    return;
  }
  int e = (int)((syn_f32_bits(amax) >> 23) & 0xFFu) - 127; /* floor(log2 amax) */
  int se = e - 2;
  if (se < -127) se = -127;
  if (se > 127) se = 127;
  *scale = (uint8_t)(se + 127);
  /* multiply by 2^-se: an exact power of two while 127 - se stays in [1, 254] */
  float inv = syn_bits_f32((uint32_t)(127 - se) << 23);
  for (int i = 0; i < 16; ++i) {
    uint8_t nib[2];
    for (int h = 0; h < 2; ++h) {
      float x = v[2 * i + h];
      float a = (x < 0.0f ? -x : x) * inv;
      nib[h] = (uint8_t)(syn_e2m1_round(a) | (x < 0.0f ? 8u : 0u));
    }
    codes16[i] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
}

/*
 * Expert blob layout (bytes), for hidden H and expert intermediate I, both
 * multiples of 32.  Each sub-array is row-major and starts at a multiple of
 * 256 bytes; the blob size is rounded up to 256.
 *   gate codes  [I][H/2]   up codes [I][H/2]   down codes [H][I/2]
 *   gate scales [I][H/32]  up scales [I][H/32] down scales [H][I/32]
 */
SYN_FN uint64_t syn_round256(uint64_t n) { return (n + 255u) & ~(uint64_t)255u; }

SYN_FN void syn_blob_offsets(uint64_t H, uint64_t I, uint64_t off[6], uint64_t* total) {
  uint64_t sz[6] = {I * H / 2, I * H / 2, H * I / 2, I * H / 32, I * H / 32, H * I / 32};
  uint64_t o = 0;
  for (int m = 0; m < 6; ++m) {
    off[m] = o;
    o += syn_round256(sz[m]);
  }
  *total = o;
}

#endif /* SYNTH_CORE_H */
