// pack.hip -- one-time, in-place rewrite of MXFP4 expert blobs between the
// canonical layout (row-major codes and scales, documented in moe_mxfp4.h)
// and the packed layout that moe_decode_layer streams.
//
// Packed layout of one MXFP4 matrix [N][K] (N a multiple of 16, K of 32, so
// a row has C = K/32 blocks of 32 elements, each 16 bytes of codes + 1 scale
// byte): rows are taken 16 at a time (a "row group" g), and each row group's
// blocks 16 at a time (a "segment" s of SC = min(16, C - 16 s) blocks).  One
// (g, s) tile holds
//     codes  [SC][16 rows] x 16 bytes   (block 16s+c of row 16g+r at c*256 + r*16)
//     scales [16 rows][SC] bytes; in a full tile (SC = 16) a row's 16 scale
//            bytes are ordered so that its dword q holds blocks q, 4+q, 8+q,
//            12+q (block 4 kb + q at byte 4 q + kb): the lane that decodes
//            blocks 4 kb + q of the row loads its four scales as one dword
// i.e. SC * 272 bytes, with every tile of a row group before the next group.
// A wave reading tile (g, s) in 1 KB slabs gives lane l = 16 q + r the block
// 16 s + 4 kb + q of row r in slab kb -- a contiguous 1 KB per load
// instruction, with the tile's scales right behind its codes, instead of
// sixteen separate 3.5 KB rows plus a scale stream in another region.
//
// Packed expert blob (same size as the canonical one): the gate and up tiles
// of each (g, s) side by side -- [gate tile][up tile] -- for every row group g
// of I and segment s of H; then the down tiles (g over H, s over I); then the
// canonical blob's alignment padding, zeroed.  Both directions are exact byte
// permutations (a bijection on the used bytes).
#include "internal.h"
#include "mx_common.h"

namespace moe {

// Byte offset, inside a matrix's packed region, of tile (g, s): the row
// groups before g hold 16 * C * 17 bytes each; the segments before s of
// group g are full (16 blocks, 4352 bytes).
__host__ __device__ inline size_t tile_offset(int g, int s, int C) {
  return (size_t)g * 16 * C * 17 + (size_t)s * 16 * 272;
}

// One thread per (matrix m, row n, block c).  m 0/1/2 = gate/up/down.
// to_packed: canonical src -> packed dst, else packed src -> canonical dst.
__global__ __launch_bounds__(256) void k_pack(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int H,
                                              int I, BlobLayout cb, bool to_packed) {
  const int C1 = H / 32, C2 = I / 32;
  const size_t n1 = (size_t)2 * I * C1, n2 = (size_t)H * C2;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n1 + n2) return;
  int m, n, c, C;
  size_t pbase;  // packed offset of this (row group, segment) tile pair / tile
  if (t < n1) {
    m = (int)(t / ((size_t)I * C1));
    const size_t r = t - (size_t)m * I * C1;
    n = (int)(r / C1);
    c = (int)(r - (size_t)n * C1);
    C = C1;
  } else {
    m = 2;
    const size_t r = t - n1;
    n = (int)(r / C2);
    c = (int)(r - (size_t)n * C2);
    C = C2;
  }
  const int g = n >> 4, rr = n & 15, s = c >> 4, cc = c & 15;
  const int SC = min(16, C - 16 * s);
  if (m < 2) {
    // gate and up tiles of (g, s) side by side: region holds 2 tiles per (g, s)
    pbase = 2 * tile_offset(g, s, C1) + (size_t)m * SC * 272;
  } else {
    pbase = (size_t)2 * I * C1 * 17 + tile_offset(g, s, C2);
  }
  const size_t p_code = pbase + (size_t)cc * 256 + rr * 16;
  const size_t p_scale = pbase + (size_t)SC * 256 + (SC == 16 ? rr * 16 + (cc & 3) * 4 + (cc >> 2) : rr * SC + cc);
  const size_t row_bytes = (size_t)C * 16;
  const size_t c_code = cb.off[m] + (size_t)n * row_bytes + (size_t)c * 16;
  const size_t c_scale = cb.off[3 + m] + (size_t)n * C + c;
  if (to_packed) {
    *reinterpret_cast<u32x4*>(dst + p_code) = *reinterpret_cast<const u32x4*>(src + c_code);
    dst[p_scale] = src[c_scale];
  } else {
    *reinterpret_cast<u32x4*>(dst + c_code) = *reinterpret_cast<const u32x4*>(src + p_code);
    dst[c_scale] = src[p_scale];
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(uint8_t* __restrict__ p, size_t n) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = 0;
}

// Rewrites experts [0, E) in place, one expert at a time through `scratch`
// (a copy of the expert, then the permutation back into its place).
hipError_t launch_pack_experts(uint8_t* experts, int E, int H, int I, uint8_t* scratch, bool to_packed,
                               hipStream_t s) {
  const BlobLayout cb = blob_layout(H, I);
  const size_t used = (size_t)2 * I * (H / 32) * 17 + (size_t)H * (I / 32) * 17;
  const size_t n = (size_t)2 * I * (H / 32) + (size_t)H * (I / 32);
  const unsigned grid = (unsigned)((n + 255) / 256);
  for (int e = 0; e < E; ++e) {
    uint8_t* blob = experts + (size_t)e * cb.bytes;
    hipError_t err = hipMemcpyAsync(scratch, blob, cb.bytes, hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return err;
    if (to_packed && used < cb.bytes) {
      hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((cb.bytes - used + 255) / 256)), dim3(256), 0, s, blob + used,
                         cb.bytes - used);
    }
    if (!to_packed && used < cb.bytes) {  // canonical padding between sub-arrays: zero
      hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((cb.bytes + 255) / 256)), dim3(256), 0, s, blob, cb.bytes);
    }
    hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, s, scratch, blob, H, I, cb, to_packed);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
