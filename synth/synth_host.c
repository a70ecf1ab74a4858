/*
 * synth_host.c -- host build of the seeded input generator (see synth_core.h
 * for the definitions).  Built with gcc + OpenMP into libsynth_host.so.  The
 * oracle's tests and the benchmark use it to regenerate any tensor of a
 * layer on the host; the device build (synth_dev.hip) writes the same bytes
 * straight into HBM.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "synth_core.h"

/* Multiplier that turns gauss_int into N(0, sigma^2) samples (fp32). */
float synth_mult(double sigma) { return (float)(sigma / (65536.0 * 1.6329931618554521 /* sqrt(8/3) */)); }

uint64_t synth_tag(uint32_t layer, uint32_t kind, uint32_t expert, uint32_t matrix) {
  return syn_tag(layer, kind, expert, matrix);
}

uint64_t synth_draw(uint64_t seed, uint64_t tag, uint64_t i) { return syn_draw(syn_key(seed, tag), i); }

int32_t synth_gauss_int(uint64_t seed, uint64_t tag, uint64_t i) { return syn_gauss_int(syn_key(seed, tag), i); }

/* out[i] = normal(i) as fp32, i in [0, n) */
void synth_fill_f32(uint64_t seed, uint64_t tag, double sigma, float* out, uint64_t n) {
  uint64_t key = syn_key(seed, tag);
  float m = synth_mult(sigma);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = syn_normal(key, (uint64_t)i, m);
}

/* out[i] = bf16_rne(normal(i)), i in [0, n) */
void synth_fill_bf16(uint64_t seed, uint64_t tag, double sigma, uint16_t* out, uint64_t n) {
  uint64_t key = syn_key(seed, tag);
  float m = synth_mult(sigma);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = syn_bf16_rne(syn_normal(key, (uint64_t)i, m));
}

/* rows [r0, r0+nr) of a bf16 [N][K] matrix whose element (n,k) is index n*K+k */
void synth_fill_bf16_rows(uint64_t seed, uint64_t tag, double sigma, uint64_t K, uint64_t r0, uint64_t nr,
                          uint16_t* out) {
  uint64_t key = syn_key(seed, tag);
  float m = synth_mult(sigma);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)nr; ++r)
    for (uint64_t k = 0; k < K; ++k) out[r * K + k] = syn_bf16_rne(syn_normal(key, (r0 + r) * K + k, m));
}

uint64_t synth_expert_bytes(uint64_t H, uint64_t I) {
  uint64_t off[6], total;
  syn_blob_offsets(H, I, off, &total);
  return total;
}

void synth_expert_offsets(uint64_t H, uint64_t I, uint64_t* off6) {
  uint64_t total;
  syn_blob_offsets(H, I, off6, &total);
}

/* Quantise matrix m of expert e (rows N, contraction K) into codes/scales. */
static void quantise_matrix(uint64_t key, float mult, uint64_t N, uint64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < (int64_t)N; ++n) {
    float v[32];
    for (uint64_t kb = 0; kb < K / 32; ++kb) {
      for (int t = 0; t < 32; ++t) v[t] = syn_normal(key, (uint64_t)n * K + kb * 32 + (uint64_t)t, mult);
      syn_mxfp4_block(v, codes + (uint64_t)n * (K / 2) + kb * 16, scales + (uint64_t)n * (K / 32) + kb);
    }
  }
}

/* Writes the full blob of expert `expert` of layer `layer` (weights ~N(0, sigma^2)). */
void synth_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, uint64_t H, uint64_t I, double sigma,
                       uint8_t* out) {
  uint64_t off[6], total;
  syn_blob_offsets(H, I, off, &total);
  memset(out, 0, total);
  float m = synth_mult(sigma);
  quantise_matrix(syn_key(seed, syn_tag(layer, SYN_KIND_EXPERT, expert, 0)), m, I, H, out + off[0], out + off[3]);
  quantise_matrix(syn_key(seed, syn_tag(layer, SYN_KIND_EXPERT, expert, 1)), m, I, H, out + off[1], out + off[4]);
  quantise_matrix(syn_key(seed, syn_tag(layer, SYN_KIND_EXPERT, expert, 2)), m, H, I, out + off[2], out + off[5]);
}

/* Quantise an arbitrary fp32 [N][K] matrix (K % 32 == 0) with the generator's encoder. */
void synth_quantise(const float* w, uint64_t N, uint64_t K, uint8_t* codes, uint8_t* scales) {
  for (uint64_t n = 0; n < N; ++n)
    for (uint64_t kb = 0; kb < K / 32; ++kb)
      syn_mxfp4_block(w + n * K + kb * 32, codes + n * (K / 2) + kb * 16, scales + n * (K / 32) + kb);
}

/*
 * Zipf-like router bias: b_e = -s * ln(rank_e), where rank is a seeded
 * permutation of 1..E (Fisher-Yates driven by the counter stream).
 */
void synth_zipf_bias(uint64_t seed, uint32_t layer, uint32_t E, double s, float* out) {
  uint64_t key = syn_key(seed, syn_tag(layer, SYN_KIND_BIASPERM, 0, 0));
  uint32_t* rank = (uint32_t*)malloc(sizeof(uint32_t) * E);
  for (uint32_t e = 0; e < E; ++e) rank[e] = e + 1;
  for (uint32_t i = E - 1; i >= 1; --i) {
    uint32_t j = (uint32_t)(syn_draw(key, i) % (uint64_t)(i + 1));
    uint32_t t = rank[i];
    rank[i] = rank[j];
    rank[j] = t;
  }
  for (uint32_t e = 0; e < E; ++e) out[e] = (float)(-s * log((double)rank[e]));
  free(rank);
}
