// dense.hip -- the bf16 dense block between MoE layers of a decode-step
// stack: RMSNorm (gain 1) to bf16, a bf16 GEMV with fp32 accumulation rounded
// to bf16, and the residual add.  The dense bf16 trunk that every token reads
// is described in "Kimi K3 on GB300: 13 kernels a layer" (section "What one
// decode step of Kimi K3 does"); like the experts it is one row against a
// weight matrix, so the GEMV streams each weight byte once with 16-byte
// non-temporal loads.
#include "internal.h"
#include "mx_common.h"

namespace moe {

// out[b] = bf16( in[b] * rsqrt(mean(in[b]^2) + eps) ).  grid: B blocks x 256.
// Each thread requests its whole share of the row (16-byte chunks, up to
// RN of them: all of a 7168-element row) before summing, and keeps it in
// registers for the output pass, so a row costs one memory round trip.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ in, int H, float eps,
                                                 uint16_t* __restrict__ out) {
  constexpr int RN = 8;
  __shared__ float part[4];
  const int b = blockIdx.x;
  const float* row = in + (size_t)b * H;
  const int H4 = H / 4;  // H is a multiple of 4 and the rows are 16-byte aligned on this path
  f32x4 v[RN];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = threadIdx.x + 256 * i;
    v[i] = c < H4 ? reinterpret_cast<const f32x4*>(row)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  for (int c = threadIdx.x + 256 * RN; c < H4; c += 256) {  // rows longer than 256 * RN * 4
    const f32x4 u = reinterpret_cast<const f32x4*>(row)[c];
    ss = fmaf(u.x, u.x, fmaf(u.y, u.y, fmaf(u.z, u.z, fmaf(u.w, u.w, ss))));
  }
  ss = sum_lanes<64>(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* o = out + (size_t)b * H;
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < H4) {
      const uint32_t lo = (uint32_t)f32_to_bf16(v[i].x * r) | ((uint32_t)f32_to_bf16(v[i].y * r) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v[i].z * r) | ((uint32_t)f32_to_bf16(v[i].w * r) << 16);
      reinterpret_cast<u32x2*>(o)[c] = u32x2{lo, hi};
    }
  }
  for (int c = threadIdx.x + 256 * RN; c < H4; c += 256) {
    const f32x4 u = reinterpret_cast<const f32x4*>(row)[c];
    const uint32_t lo = (uint32_t)f32_to_bf16(u.x * r) | ((uint32_t)f32_to_bf16(u.y * r) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(u.z * r) | ((uint32_t)f32_to_bf16(u.w * r) << 16);
    reinterpret_cast<u32x2*>(o)[c] = u32x2{lo, hi};
  }
}

// The same for rows that are not 16-byte aligned (hidden % 4 != 0 or an
// unaligned buffer): scalar loads, two passes.
__global__ __launch_bounds__(256) void k_rmsnorm_scalar(const float* __restrict__ in, int H, float eps,
                                                        uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int b = blockIdx.x;
  const float* row = in + (size_t)b * H;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += 256) ss = fmaf(row[i], row[i], ss);
  ss = sum_lanes<64>(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) out[(size_t)b * H + i] = f32_to_bf16(row[i] * r);
}

hipError_t launch_rmsnorm(const float* in, int B, int H, float eps, uint16_t* out, hipStream_t s) {
  if (H % 4 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0)
    hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(256), 0, s, in, H, eps, out);
  else
    hipLaunchKernelGGL(k_rmsnorm_scalar, dim3(B), dim3(256), 0, s, in, H, eps, out);
  return hipGetLastError();
}

// y[b][n] = bf16( sum_k W[n][k] x[b][k] ).  Half a wave per weight row (two
// rows per wave, eight per block); x rows staged in LDS RG at a time.
template <int RG>
__global__ __launch_bounds__(256) void k_dense_gemv(const uint16_t* __restrict__ w, int N, int K,
                                                    const uint16_t* __restrict__ x, int B, uint16_t* __restrict__ y) {
  extern __shared__ u32x4 lds_raw[];
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(lds_raw);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int n = blockIdx.x * 8 + wave * 2 + half;
  const int C8 = K / 8;
  for (int g0 = 0; g0 < B; g0 += RG) {
    const int nr = min(RG, B - g0);
    __syncthreads();
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)g0 * K);
    for (int i = threadIdx.x; i < nr * C8; i += 256) lds_raw[i] = src[i];
    __syncthreads();
    float acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = 0.0f;
    if (n < N) {
      const uint16_t* wr = w + (size_t)n * K;
      for (int c0 = l32; c0 < C8; c0 += 32 * 8) {
        u32x4 q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int c = c0 + 32 * i;
          if (c < C8) q[i] = ld_weight16(wr + 8 * (size_t)c);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int c = c0 + 32 * i;
          if (c < C8) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
              if (r < nr) {
                u32x4 xv = reinterpret_cast<const u32x4*>(xs + (size_t)r * K)[c];
                float a = acc[r];
                a = dot2_bf16(q[i][0], xv[0], a);
                a = dot2_bf16(q[i][1], xv[1], a);
                a = dot2_bf16(q[i][2], xv[2], a);
                a = dot2_bf16(q[i][3], xv[3], a);
                acc[r] = a;
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (r < nr) {
        float v = sum_lanes<32>(acc[r]);
        if (l32 == 0 && n < N) y[(size_t)(g0 + r) * N + n] = f32_to_bf16(v);
      }
    }
  }
}

// One activation row (batch 1): a wave per weight row, two waves per block
// (3584 blocks at 7168 rows, so the stream runs on without lock-step rounds).
// Lane l takes granules l, l + 64, ... of the row (offsets that are
// immediates off one base) and the matching x granules, read from global
// memory (the 14 KB row stays in L2) -- no staging round trip and no
// barrier precede the weight loads.  Up to DG_NG granules of each are
// requested before any is used.
constexpr int DG_NG = 14;  // granules per lane and pass: a 7168-wide row

__device__ __forceinline__ float dot_granule(const u32x4& a, const u32x4& b, float acc) {
  acc = dot2_bf16(a[0], b[0], acc);
  acc = dot2_bf16(a[1], b[1], acc);
  acc = dot2_bf16(a[2], b[2], acc);
  return dot2_bf16(a[3], b[3], acc);
}

__global__ __launch_bounds__(128) void k_dense_gemv1(const uint16_t* __restrict__ w, int N, int K,
                                                     const uint16_t* __restrict__ x, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 2 + (threadIdx.x >> 6);
  const int C8 = K / 8;
  const uint16_t* wr = w + (size_t)min(n, N - 1) * K;
  float acc = 0.0f;
  for (int c0 = lane; c0 < C8; c0 += 64 * DG_NG) {
    u32x4 q[DG_NG], xv[DG_NG];
    const u32x4 z{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < DG_NG; ++i) {
      const int c = c0 + 64 * i;
      const bool ok = c < C8;
      q[i] = ok ? ld_weight16(wr + 8 * (size_t)c) : z;
      xv[i] = ok ? ld16(x + 8 * (size_t)c) : z;
    }
#pragma unroll
    for (int i = 0; i < DG_NG; ++i)
      if (c0 + 64 * i < C8) acc = dot_granule(q[i], xv[i], acc);
  }
  acc = sum_lanes<64>(acc);
  if (lane == 0 && n < N) y[n] = f32_to_bf16(acc);
}

// Batches of 2..64 rows on the matrix cores: a workgroup takes 16 weight
// rows and every activation row at once (NCG groups of 16 columns), so each
// weight is read once per call instead of once per few rows.  One
// v_mfma_f32_16x16x32_bf16 per 32 elements and column group: lane 16 q + r
// supplies 8 elements of weight row r (A) and of activation row 16 cg + r
// (B); the four waves split K into 128-element segments (w, w + 4, ...), two
// segments of weights in flight per wave, activations read from L2; the
// partial sums meet in LDS and are rounded once to bf16.
template <int NCG>
__global__ __launch_bounds__(256) void k_dense_gemv_mf(const uint16_t* __restrict__ w, int N, int K,
                                                       const uint16_t* __restrict__ x, int B,
                                                       uint16_t* __restrict__ y) {
  __shared__ float red[4][NCG][16][16];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int S = (K + 127) / 128;
  const int P = wv < S ? (S - wv + 3) / 4 : 0;
  const uint16_t* wrow = w + (size_t)min(n0 + r, N - 1) * K;
  const uint16_t* xrow[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) xrow[cg] = x + (size_t)min(16 * cg + r, B - 1) * K;
  const u32x4 z{0u, 0u, 0u, 0u};
  f32x4 acc[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) acc[cg] = f32x4{0.f, 0.f, 0.f, 0.f};
  // XP: activation column groups fetched with the weights (the rest are read
  // in the math, from L2)
  constexpr int XP = NCG <= 2 ? NCG : 0;
  struct Buf {
    u32x4 w[4];
    u32x4 x[XP > 0 ? XP : 1][4];
  };
  Buf ba, bb;
  auto load = [&](Buf& b, int pp) {
    const int s = wv + 4 * pp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = min(s * 128 + 32 * j + 8 * q, K - 8);
      b.w[j] = ld_weight16(wrow + k0);
#pragma unroll
      for (int cg = 0; cg < XP; ++cg) b.x[cg][j] = ld16(xrow[cg] + k0);
    }
  };
  auto math = [&](const Buf& b, int pp) {
    const int s = wv + 4 * pp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = s * 128 + 32 * j + 8 * q;
      const bool ok = k0 < K;
      const bf16x8 a = __builtin_bit_cast(bf16x8, ok ? b.w[j] : z);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const u32x4 xv = ok ? (cg < XP ? b.x[cg < XP ? cg : 0][j] : ld16(xrow[cg] + k0)) : z;
        acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, xv), acc[cg], 0, 0, 0);
      }
    }
  };
  if (P > 0) load(ba, 0);
  if (P > 1) load(bb, 1);
  for (int pp = 0; pp < P; pp += 2) {
    math(ba, pp);
    if (pp + 2 < P) load(ba, pp + 2);
    if (pp + 1 < P) {
      math(bb, pp + 1);
      if (pp + 3 < P) load(bb, pp + 3);
    }
  }
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][cg][4 * q + i][r] = acc[cg][i];
  __syncthreads();
  const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float v = ((red[0][cg][row][col] + red[1][cg][row][col]) + red[2][cg][row][col]) + red[3][cg][row][col];
    const int n = n0 + row, b = 16 * cg + col;
    if (n < N && b < B) y[(size_t)b * N + n] = f32_to_bf16(v);
  }
}

hipError_t launch_dense_gemv(const uint16_t* w, int N, int K, const uint16_t* x, int B, uint16_t* y, hipStream_t s) {
  if (B == 1 && reinterpret_cast<uintptr_t>(x) % 16 == 0) {
    hipLaunchKernelGGL(k_dense_gemv1, dim3((N + 1) / 2), dim3(128), 0, s, w, N, K, x, y);
    return hipGetLastError();
  }
  if (B > 1 && reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0) {
    const dim3 grid((N + 15) / 16), block(256);
    const int ncg = (B + 15) / 16;
    if (ncg == 1) hipLaunchKernelGGL(k_dense_gemv_mf<1>, grid, block, 0, s, w, N, K, x, B, y);
    else if (ncg == 2) hipLaunchKernelGGL(k_dense_gemv_mf<2>, grid, block, 0, s, w, N, K, x, B, y);
    else if (ncg == 3) hipLaunchKernelGGL(k_dense_gemv_mf<3>, grid, block, 0, s, w, N, K, x, B, y);
    else hipLaunchKernelGGL(k_dense_gemv_mf<4>, grid, block, 0, s, w, N, K, x, B, y);
    return hipGetLastError();
  }
  size_t row_bytes = (size_t)K * 2;
  int rg = B <= 1 ? 1 : (B <= 2 ? 2 : 4);
  while (rg > 1 && rg * row_bytes > 65536) rg >>= 1;
  size_t lds = rg * row_bytes;
  dim3 grid((N + 7) / 8), block(256);
  if (rg == 1) hipLaunchKernelGGL(k_dense_gemv<1>, grid, block, lds, s, w, N, K, x, B, y);
  else if (rg == 2) hipLaunchKernelGGL(k_dense_gemv<2>, grid, block, lds, s, w, N, K, x, B, y);
  else hipLaunchKernelGGL(k_dense_gemv<4>, grid, block, lds, s, w, N, K, x, B, y);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_residual_add(float* __restrict__ h, const uint16_t* __restrict__ t, size_t n) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] += __uint_as_float((uint32_t)t[i] << 16);
}

hipError_t launch_residual_add(float* h, const uint16_t* t, int B, int H, hipStream_t s) {
  size_t n = (size_t)B * H;
  hipLaunchKernelGGL(k_residual_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h, t, n);
  return hipGetLastError();
}

// Fused residual add and RMSNorm: h[b] += float(t[b]) (fp32, written back),
// then out[b] = bf16( h[b] * rsqrt(mean(h[b]^2) + eps) ), in one pass of one
// block per row (the row stays in registers); the same sums, in the same
// order, as residual_add followed by k_rmsnorm.  Rows 16-byte aligned,
// hidden a multiple of 4 and at most 256 * 8 * 4.
__global__ __launch_bounds__(256) void k_residual_add_rmsnorm(float* __restrict__ h, const uint16_t* __restrict__ t,
                                                              int H, float eps, uint16_t* __restrict__ out) {
  constexpr int RN = 8;
  __shared__ float part[4];
  const int b = blockIdx.x;
  float* row = h + (size_t)b * H;
  const uint16_t* trow = t + (size_t)b * H;
  const int H4 = H / 4;
  f32x4 v[RN];
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < H4) {
      const f32x4 a = reinterpret_cast<const f32x4*>(row)[c];
      const u32x2 tb = reinterpret_cast<const u32x2*>(trow)[c];
      v[i] = f32x4{a.x + __uint_as_float(tb.x << 16), a.y + __uint_as_float(tb.x & 0xFFFF0000u),
                   a.z + __uint_as_float(tb.y << 16), a.w + __uint_as_float(tb.y & 0xFFFF0000u)};
      reinterpret_cast<f32x4*>(row)[c] = v[i];
    } else {
      v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = sum_lanes<64>(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* o = out + (size_t)b * H;
#pragma unroll
  for (int i = 0; i < RN; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < H4) {
      const uint32_t lo = (uint32_t)f32_to_bf16(v[i].x * r) | ((uint32_t)f32_to_bf16(v[i].y * r) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v[i].z * r) | ((uint32_t)f32_to_bf16(v[i].w * r) << 16);
      reinterpret_cast<u32x2*>(o)[c] = u32x2{lo, hi};
    }
  }
}

hipError_t launch_residual_add_rmsnorm(float* h, const uint16_t* t, int B, int H, float eps, uint16_t* out,
                                       hipStream_t s) {
  const bool fused = H % 4 == 0 && H <= 256 * 8 * 4 && reinterpret_cast<uintptr_t>(h) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(t) % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 8 == 0;
  if (!fused) {  // two passes: the add, then the norm
    hipError_t e = launch_residual_add(h, t, B, H, s);
    return e != hipSuccess ? e : launch_rmsnorm(h, B, H, eps, out, s);
  }
  hipLaunchKernelGGL(k_residual_add_rmsnorm, dim3(B), dim3(256), 0, s, h, t, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe
