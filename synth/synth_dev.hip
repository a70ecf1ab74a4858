// synth_dev.hip -- device build of the seeded input generator (definitions in
// synth_core.h).  Fills HBM with exactly the bytes that synth_host.c produces,
// so that a layer's 15.7 GB of experts can be made in milliseconds while the
// oracle regenerates only the experts it needs.  Built into libsynth_dev.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

__global__ void syn_k_fill_bf16(uint64_t key, float mult, uint16_t* __restrict__ out, uint64_t n) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = syn_bf16_rne(syn_normal(key, i, mult));
}

__global__ void syn_k_fill_f32(uint64_t key, float mult, float* __restrict__ out, uint64_t n) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = syn_normal(key, i, mult);
}

// One thread per 32-element block.  Blocks are enumerated expert-major, then
// matrix (gate, up, down), then row, then block within the row.
__global__ void syn_k_expert_blobs(uint64_t seed, uint32_t layer, uint32_t e0, uint32_t ne, uint64_t H, uint64_t I,
                                   float mult, uint8_t* __restrict__ base, uint64_t blob_bytes) {
  uint64_t off[6], total;
  syn_blob_offsets(H, I, off, &total);
  const uint64_t nb_gu = I * (H / 32);  // blocks per gate (or up) matrix
  const uint64_t nb_d = H * (I / 32);   // blocks per down matrix
  const uint64_t per_expert = 2 * nb_gu + nb_d;
  const uint64_t nblocks = per_expert * ne;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblocks; t += stride) {
    uint32_t el = (uint32_t)(t / per_expert);
    uint64_t r = t - (uint64_t)el * per_expert;
    uint32_t m;
    uint64_t K, b;
    if (r < nb_gu) { m = 0; b = r; K = H; }
    else if (r < 2 * nb_gu) { m = 1; b = r - nb_gu; K = H; }
    else { m = 2; b = r - 2 * nb_gu; K = I; }
    uint64_t bpr = K / 32;
    uint64_t row = b / bpr, kb = b - row * bpr;
    uint64_t key = syn_key(seed, syn_tag(layer, SYN_KIND_EXPERT, e0 + el, m));
    float v[32];
    for (int i = 0; i < 32; ++i) v[i] = syn_normal(key, row * K + kb * 32 + (uint64_t)i, mult);
    uint8_t* blob = base + (uint64_t)el * blob_bytes;
    uint8_t codes[16];
    uint8_t sc;
    syn_mxfp4_block(v, codes, &sc);
    uint8_t* cdst = blob + off[m] + row * (K / 2) + kb * 16;
    for (int i = 0; i < 16; ++i) cdst[i] = codes[i];
    blob[off[3 + m] + row * bpr + kb] = sc;
  }
}

static int launch_grid(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (int)(g > 65536 ? 65536 : (g == 0 ? 1 : g));
}

extern "C" {

int synth_dev_fill_bf16(uint64_t key, float mult, uint16_t* out, uint64_t n, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(syn_k_fill_bf16, dim3(launch_grid(n)), dim3(256), 0, (hipStream_t)stream, key, mult, out, n);
  return (int)hipGetLastError();
}

int synth_dev_fill_f32(uint64_t key, float mult, float* out, uint64_t n, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(syn_k_fill_f32, dim3(launch_grid(n)), dim3(256), 0, (hipStream_t)stream, key, mult, out, n);
  return (int)hipGetLastError();
}

// Writes experts e0 .. e0+ne-1 of `layer` into base (expert el at el * blob_bytes).
// Padding bytes of each blob are not written; the caller zeroes the buffer first.
int synth_dev_expert_blobs(uint64_t seed, uint32_t layer, uint32_t e0, uint32_t ne, uint64_t H, uint64_t I, float mult,
                           uint8_t* base, uint64_t blob_bytes, void* stream) {
  uint64_t off[6], total;
  syn_blob_offsets(H, I, off, &total);
  if (blob_bytes < total || H % 32 || I % 32) return -1;
  uint64_t nblocks = (2 * I * (H / 32) + H * (I / 32)) * (uint64_t)ne;
  if (nblocks == 0) return 0;
  hipLaunchKernelGGL(syn_k_expert_blobs, dim3(launch_grid(nblocks)), dim3(256), 0, (hipStream_t)stream, seed, layer,
                     e0, ne, H, I, mult, base, blob_bytes);
  return (int)hipGetLastError();
}

}  // extern "C"
