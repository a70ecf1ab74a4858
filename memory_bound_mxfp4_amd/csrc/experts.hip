// experts.hip -- shared and routed SwiGLU experts (FC1 + SwiGLU, FC2), the
// weighted combine into the residual, and the standalone MXFP4 GEMV.
//
// Every matmul here is one or a few activation rows against a weight matrix
// -- about one FLOP per weight byte, so the kernels are HBM-bound ("Kimi K3 on
// GB300: 13 kernels a layer", section "What one decode step of Kimi K3
// does").  The design streams each weight byte once with coalesced 16-byte
// non-temporal loads, dequantises MXFP4 in registers with the gfx950 scaled
// FP4 conversions (exact into bf16 / fp32), and reduces over K with wave
// butterflies; activations sit in LDS.
//
// The layer's own expert streams live in layer.hip; this file holds the
// standalone GEMV entry point and the workspace clearing kernel.
#include "internal.h"
#include "mx_common.h"

namespace moe {

constexpr int LDS_BUDGET = 65536;

// ---------------------------------------------------------------------------
// Dot-product building blocks.  A "row" is one weight row; LPR lanes share it
// (lane l handles 16-byte chunks l, l+LPR, ...).  Chunks are loaded 8 at a
// time per lane before any math, so 8 x 16 bytes per lane are in flight.
// acc[r] accumulates the partial dot product with activation row r (LDS).
// ---------------------------------------------------------------------------

// MXFP4 weights x bf16 activations (chunk = 32 elements = 1 scale block).
template <int RG, int LPR>
__device__ __forceinline__ void dot_mx_bf16(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                            int C, const uint16_t* xs, int K, int nr, int l, float (&acc)[RG]) {
  for (int c0 = l; c0 < C; c0 += LPR * 8) {
    u32x4 q[8];
    uint32_t sb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C) {
        q[i] = ld_weight16(codes + 16 * (size_t)c);
        sb[i] = scales[c];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C) {
        float s = e8m0_scale(sb[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bf16x2 w[4];
          dq4_bf16(q[i][d], s, w);
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            if (r < nr) {
              u32x4 xv = *reinterpret_cast<const u32x4*>(xs + (size_t)r * K + 32 * c + 8 * d);
              float a = acc[r];
              a = dot2_bf16(w[0], xv[0], a);
              a = dot2_bf16(w[1], xv[1], a);
              a = dot2_bf16(w[2], xv[2], a);
              a = dot2_bf16(w[3], xv[3], a);
              acc[r] = a;
            }
          }
        }
      }
    }
  }
}

// MXFP4 weights x fp32 activations.
template <int RG, int LPR>
__device__ __forceinline__ void dot_mx_f32(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                           int C, const float* xs, int K, int nr, int l, float (&acc)[RG]) {
  for (int c0 = l; c0 < C; c0 += LPR * 8) {
    u32x4 q[8];
    uint32_t sb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C) {
        q[i] = ld_weight16(codes + 16 * (size_t)c);
        sb[i] = scales[c];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C) {
        float s = e8m0_scale(sb[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          f32x2 w[4];
          dq4_f32(q[i][d], s, w);
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            if (r < nr) {
              const float* xp = xs + (size_t)r * K + 32 * c + 8 * d;
              f32x4 x0 = *reinterpret_cast<const f32x4*>(xp);
              f32x4 x1 = *reinterpret_cast<const f32x4*>(xp + 4);
              float a = acc[r];
              a = fmaf(w[0].x, x0.x, a);
              a = fmaf(w[0].y, x0.y, a);
              a = fmaf(w[1].x, x0.z, a);
              a = fmaf(w[1].y, x0.w, a);
              a = fmaf(w[2].x, x1.x, a);
              a = fmaf(w[2].y, x1.y, a);
              a = fmaf(w[3].x, x1.z, a);
              a = fmaf(w[3].y, x1.w, a);
              acc[r] = a;
            }
          }
        }
      }
    }
  }
}

int pick_rg(int B, size_t row_bytes) {
  int rg = B <= 1 ? 1 : (B <= 8 ? 2 : 4);
  while (rg > 1 && (size_t)rg * row_bytes > (size_t)LDS_BUDGET) rg >>= 1;
  return rg;
}

__global__ __launch_bounds__(256) void k_zero(u32x4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t g = (n16 + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)g), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone MXFP4 GEMV: y[b][n] = dequant(W)[n] . x[b].  16 lanes per weight
// row, 16 rows per block pass; x rows staged in LDS RG at a time.
// grid: ceil(N/16) blocks of 256 threads.
// ---------------------------------------------------------------------------
template <int RG, bool XF32>
__global__ __launch_bounds__(256) void k_gemv_mx(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                 int N, int K, const void* __restrict__ x, int B, float* __restrict__ y) {
  extern __shared__ u32x4 lds_raw[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sub = lane >> 4, l16 = lane & 15;
  const int n = blockIdx.x * 16 + wave * 4 + sub;
  const int xsz = XF32 ? 4 : 2;
  const int per_row = K * xsz / 16;
  for (int g0 = 0; g0 < B; g0 += RG) {
    const int nr = min(RG, B - g0);
    __syncthreads();
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(x) + (size_t)g0 * K * xsz);
    for (int i = threadIdx.x; i < nr * per_row; i += 256) lds_raw[i] = src[i];
    __syncthreads();
    float acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = 0.0f;
    if (n < N) {
      const uint8_t* cr = codes + (size_t)n * (K / 2);
      const uint8_t* sr = scales + (size_t)n * (K / 32);
      if (XF32) dot_mx_f32<RG, 16>(cr, sr, K / 32, reinterpret_cast<const float*>(lds_raw), K, nr, l16, acc);
      else dot_mx_bf16<RG, 16>(cr, sr, K / 32, reinterpret_cast<const uint16_t*>(lds_raw), K, nr, l16, acc);
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (r < nr) {
        float v = sum_lanes<16>(acc[r]);
        if (l16 == 0 && n < N) y[(size_t)(g0 + r) * N + n] = v;
      }
    }
  }
}

hipError_t launch_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, const void* x, bool x_f32,
                             int B, float* y, hipStream_t s) {
  size_t row_bytes = (size_t)K * (x_f32 ? 4 : 2);
  int rg = pick_rg(B >= 4 ? 16 : B, row_bytes);
  size_t lds = (size_t)rg * row_bytes;
  dim3 grid((N + 15) / 16), block(256);
#define GEMV_CASE(R)                                                                                   \
  if (rg == R) {                                                                                       \
    if (x_f32) hipLaunchKernelGGL((k_gemv_mx<R, true>), grid, block, lds, s, codes, scales, N, K, x, B, y); \
    else hipLaunchKernelGGL((k_gemv_mx<R, false>), grid, block, lds, s, codes, scales, N, K, x, B, y);      \
  }
  GEMV_CASE(1)
  GEMV_CASE(2)
  GEMV_CASE(4)
#undef GEMV_CASE
  return hipGetLastError();
}

}  // namespace moe
