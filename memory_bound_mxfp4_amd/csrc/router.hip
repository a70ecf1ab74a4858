// router.hip -- the standalone router_topk entry point: router GEMV with
// exact fp64 accumulation, then wave-level top-k with renormalised gates.
// (The layer kernel runs the same device functions inside its work queue.)
//
// The router, top-16 selection and shared/routed experts are the per-layer
// work of "Kimi K3 on GB300: 13 kernels a layer" (section "What one decode
// step of Kimi K3 does"); the same page's section "Why batch 1 on a rack is
// not only a bandwidth problem" names router scores and top-16 selection as
// short, dependent, bandwidth-idle work -- so these kernels aim at latency:
// every expert row is streamed once by one wave, and selection is a handful
// of wave-wide butterfly reductions with no host round trip.
#include "internal.h"
#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits.  Two waves per expert row (one half each); block (e-pair,
// row-block) stages RB activation rows in LDS (swizzled 16-byte granules, row
// stride xstride).  bf16 x bf16 products are exact in fp32; they are summed in
// fp64 (exact for this data up to 2^-52 relative), the bias is added in fp64
// and the result is rounded to fp32 once.
// grid: (ceil(E/2), ceil(B/RB)) blocks of 256 threads; LDS: RB * xstride * 16 bytes.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x, int B, int H,
                                                       const uint16_t* __restrict__ wr, const float* __restrict__ bias,
                                                       int E, int xstride, float* __restrict__ logits) {
  extern __shared__ u32x4 xs[];
  __shared__ double part[4][RB];
  const int w = threadIdx.x >> 6, half = w & 1;
  const int e = blockIdx.x * 2 + (w >> 1);
  const int b0 = blockIdx.y * RB, nb = min(RB, B - b0);
  const int C = H / 8, gh = (C + 1) / 2;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)b0 * H);
  for (int i = threadIdx.x; i < nb * C; i += 256) {
    const int r = i / C, c = i - r * C;
    xs[r * xstride + swz(c)] = src[i];
  }
  __syncthreads();
  double acc[RB];
  router_dot<RB>(wr + (size_t)min(e, E - 1) * H, half * gh, half ? C : gh, xs, xstride, nb, acc);
  if (half && (threadIdx.x & 63) == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) part[w][r] = acc[r];
  }
  __syncthreads();
  if (!half && e < E && (threadIdx.x & 63) == 0) {
    const double bb = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < nb) logits[(size_t)(b0 + r) * E + e] = (float)(acc[r] + part[w + 1][r] + bb);
  }
}

hipError_t launch_router_logits(const uint16_t* x, int B, int H, const uint16_t* wr, const float* bias, int E,
                                float* logits, hipStream_t s) {
  const int xstride = ((H / 8 + 7) / 8) * 8;
  dim3 grid((E + 1) / 2, B);
  if (B == 1) {
    hipLaunchKernelGGL(k_router_logits<1>, grid, dim3(256), (size_t)xstride * 16, s, x, B, H, wr, bias, E, xstride,
                       logits);
  } else {
    grid.y = (B + 3) / 4;
    hipLaunchKernelGGL(k_router_logits<4>, grid, dim3(256), (size_t)4 * xstride * 16, s, x, B, H, wr, bias, E,
                       xstride, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k + renormalised gates: one wave per row (topk_row in moe_device.h).
// grid: B blocks of 64 threads.
// ---------------------------------------------------------------------------
template <int KPL>
__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ logits, int E, int k, int32_t* __restrict__ idx,
                                             float* __restrict__ gate) {
  const int b = blockIdx.x;
  topk_row<KPL>(logits + (size_t)b * E, E, k, idx + (size_t)b * k, gate + (size_t)b * k);
}

hipError_t launch_topk(const float* logits, int B, int E, int k, int32_t* idx, float* gate, hipStream_t s) {
  int kpl = (E + 63) / 64;
  dim3 grid(B), block(64);
  if (kpl <= 1) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, logits, E, k, idx, gate);
  else if (kpl <= 2) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, logits, E, k, idx, gate);
  else if (kpl <= 4) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, logits, E, k, idx, gate);
  else if (kpl <= 8) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, logits, E, k, idx, gate);
  else if (kpl <= 16) hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, logits, E, k, idx, gate);
  else if (kpl <= 32) hipLaunchKernelGGL(k_topk<32>, grid, block, 0, s, logits, E, k, idx, gate);
  else hipLaunchKernelGGL(k_topk<64>, grid, block, 0, s, logits, E, k, idx, gate);
  return hipGetLastError();
}

}  // namespace moe
