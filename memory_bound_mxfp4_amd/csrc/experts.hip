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
// Work is expert-gathered: a unit is (expert, tile of output rows) and
// computes that tile for every activation row routed to the expert, so an
// expert's weights are read once per step whatever the batch.
#include "internal.h"
#include "mx_common.h"

namespace moe {

constexpr int NT1 = 16;   // routed FC1 outputs per unit (16 x 7 KB of codes at H 7168)
constexpr int NT1S = 4;   // shared FC1 outputs per unit (4 x 28 KB of bf16)
constexpr int NT2 = 64;   // routed FC2 outputs per unit (64 x 816 B at I 1536)
constexpr int NT2S = 32;  // shared FC2 outputs per unit (32 x 3 KB)
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

// bf16 weights x bf16 activations (chunk = 8 elements).
template <int RG, int LPR>
__device__ __forceinline__ void dot_bf16_bf16(const uint16_t* __restrict__ w, int C8, const uint16_t* xs, int K,
                                              int nr, int l, float (&acc)[RG]) {
  for (int c0 = l; c0 < C8; c0 += LPR * 8) {
    u32x4 q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C8) q[i] = ld_weight16(w + 8 * (size_t)c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C8) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r < nr) {
            u32x4 xv = *reinterpret_cast<const u32x4*>(xs + (size_t)r * K + 8 * c);
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

// bf16 weights x fp32 activations (chunk = 8 elements).
template <int RG, int LPR>
__device__ __forceinline__ void dot_bf16_f32(const uint16_t* __restrict__ w, int C8, const float* xs, int K, int nr,
                                             int l, float (&acc)[RG]) {
  for (int c0 = l; c0 < C8; c0 += LPR * 8) {
    u32x4 q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C8) q[i] = ld_weight16(w + 8 * (size_t)c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + LPR * i;
      if (c < C8) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r < nr) {
            const float* xp = xs + (size_t)r * K + 8 * c;
            f32x4 x0 = *reinterpret_cast<const f32x4*>(xp);
            f32x4 x1 = *reinterpret_cast<const f32x4*>(xp + 4);
            float a = acc[r];
            a = fmaf(bf16_lo(q[i][0]), x0.x, a);
            a = fmaf(bf16_hi(q[i][0]), x0.y, a);
            a = fmaf(bf16_lo(q[i][1]), x0.z, a);
            a = fmaf(bf16_hi(q[i][1]), x0.w, a);
            a = fmaf(bf16_lo(q[i][2]), x1.x, a);
            a = fmaf(bf16_hi(q[i][2]), x1.y, a);
            a = fmaf(bf16_lo(q[i][3]), x1.z, a);
            a = fmaf(bf16_hi(q[i][3]), x1.w, a);
            acc[r] = a;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Unit bookkeeping
// ---------------------------------------------------------------------------
struct ExpertParams {
  int H, I, E, k, Is, B;
  const uint16_t* x;
  const uint16_t *sg, *su, *sd;
  const uint8_t* experts;
  size_t blob_bytes;
  size_t off[6];
  Sched sched;
  float* h_shared;
  float* h_routed;
  float* o_shared;
  float* o_routed;
  const float* gate;
  float* residual;
};

// Activation-row list of a unit: for the shared expert every batch row, for
// routed expert a the slots that selected it.
struct RowList {
  const int* slots;  // NULL for the shared expert (row i is batch row i)
  int n;
};

__device__ __forceinline__ int row_batch(const RowList& rl, int i, int k) { return rl.slots ? rl.slots[i] / k : i; }
__device__ __forceinline__ int row_slot(const RowList& rl, int i) { return rl.slots ? rl.slots[i] : i; }

// Stage rows [r0, r0+nr) of the row list from src ([B or B*k][K] of T) into
// LDS dst ([RG][K]).  `by_slot` indexes src by slot (h) instead of batch row (x).
template <typename T>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, const RowList& rl, int r0, int nr, int K, int k,
                                           bool by_slot) {
  const int per_row = K * (int)sizeof(T) / 16;
  for (int i = threadIdx.x; i < nr * per_row; i += blockDim.x) {
    int r = i / per_row, c = i - r * per_row;
    int src_row = by_slot ? row_slot(rl, r0 + r) : row_batch(rl, r0 + r, k);
    reinterpret_cast<u32x4*>(dst + (size_t)r * K)[c] = reinterpret_cast<const u32x4*>(src + (size_t)src_row * K)[c];
  }
}

// ---------------------------------------------------------------------------
// FC1 + SwiGLU.  Units: [shared tiles of NT1S][routed (expert, tile of NT1)].
// A wave computes one output n at a time: lanes 0-31 the gate row, lanes
// 32-63 the up row; after the 32-lane butterflies lane 0 holds g, lane 32 u,
// and h = silu(g) * u is written (fp32).
// ---------------------------------------------------------------------------
template <int RG>
__global__ __launch_bounds__(256) void k_fc1(ExpertParams p) {
  extern __shared__ u32x4 lds_raw[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds_raw);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int U = *p.sched.n_active;
  const int n_sh = p.Is > 0 ? (p.Is + NT1S - 1) / NT1S : 0;
  const int tiles = (p.I + NT1 - 1) / NT1;
  const int total = n_sh + U * tiles;
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const bool shared = u < n_sh;
    int a = 0, t = u;
    RowList rl;
    if (shared) {
      rl.slots = nullptr;
      rl.n = p.B;
    } else {
      int v = u - n_sh;
      a = v % U;
      t = v / U;
      int r0 = p.sched.row_off[a];
      rl.slots = p.sched.rows + r0;
      rl.n = p.sched.row_off[a + 1] - r0;
    }
    const int NT = shared ? NT1S : NT1, N = shared ? p.Is : p.I;
    const int n_begin = t * NT, n_end = min(N, n_begin + NT);
    const uint8_t* blob = shared ? nullptr : p.experts + (size_t)p.sched.active[a] * p.blob_bytes;
    for (int g0 = 0; g0 < rl.n; g0 += RG) {
      const int nr = min(RG, rl.n - g0);
      __syncthreads();
      stage_rows<uint16_t>(xs, p.x, rl, g0, nr, p.H, p.k, false);
      __syncthreads();
      for (int n = n_begin + wave; n < n_end; n += 4) {
        float acc[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[r] = 0.0f;
        if (shared) {
          const uint16_t* wrow = (half ? p.su : p.sg) + (size_t)n * p.H;
          dot_bf16_bf16<RG, 32>(wrow, p.H / 8, xs, p.H, nr, l32, acc);
        } else {
          const uint8_t* codes = blob + p.off[half] + (size_t)n * (p.H / 2);
          const uint8_t* sc = blob + p.off[3 + half] + (size_t)n * (p.H / 32);
          dot_mx_bf16<RG, 32>(codes, sc, p.H / 32, xs, p.H, nr, l32, acc);
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r < nr) {
            float v = sum_lanes<32>(acc[r]);
            float upv = __shfl(v, 32, WAVE);
            if (lane == 0) {
              float h = silu_f(v) * upv;
              if (shared) p.h_shared[(size_t)(g0 + r) * p.Is + n] = h;
              else p.h_routed[(size_t)row_slot(rl, g0 + r) * p.I + n] = h;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FC2.  Units: [shared tiles of NT2S][routed (expert, tile of NT2)].  16 lanes
// per output row, 4 rows per wave at a time.
// ---------------------------------------------------------------------------
template <int RG>
__global__ __launch_bounds__(256) void k_fc2(ExpertParams p) {
  extern __shared__ u32x4 lds_raw[];
  float* hs = reinterpret_cast<float*>(lds_raw);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sub = lane >> 4, l16 = lane & 15;
  const int U = *p.sched.n_active;
  const int n_sh = p.Is > 0 ? (p.H + NT2S - 1) / NT2S : 0;
  const int tiles = (p.H + NT2 - 1) / NT2;
  const int total = n_sh + U * tiles;
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const bool shared = u < n_sh;
    int a = 0, t = u;
    RowList rl;
    if (shared) {
      rl.slots = nullptr;
      rl.n = p.B;
    } else {
      int v = u - n_sh;
      a = v % U;
      t = v / U;
      int r0 = p.sched.row_off[a];
      rl.slots = p.sched.rows + r0;
      rl.n = p.sched.row_off[a + 1] - r0;
    }
    const int NT = shared ? NT2S : NT2, K = shared ? p.Is : p.I;
    const int m_begin = t * NT, m_end = min(p.H, m_begin + NT);
    const uint8_t* blob = shared ? nullptr : p.experts + (size_t)p.sched.active[a] * p.blob_bytes;
    for (int g0 = 0; g0 < rl.n; g0 += RG) {
      const int nr = min(RG, rl.n - g0);
      __syncthreads();
      // h rows: shared h is indexed by batch row, routed h by slot
      stage_rows<float>(hs, shared ? p.h_shared : p.h_routed, rl, g0, nr, K, p.k, !shared);
      __syncthreads();
      for (int m0 = m_begin + wave * 4; m0 < m_end; m0 += 16) {
        const int m = m0 + sub;
        float acc[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[r] = 0.0f;
        if (m < m_end) {
          if (shared) {
            dot_bf16_f32<RG, 16>(p.sd + (size_t)m * K, K / 8, hs, K, nr, l16, acc);
          } else {
            const uint8_t* codes = blob + p.off[2] + (size_t)m * (K / 2);
            const uint8_t* sc = blob + p.off[5] + (size_t)m * (K / 32);
            dot_mx_f32<RG, 16>(codes, sc, K / 32, hs, K, nr, l16, acc);
          }
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (r < nr) {
            float v = sum_lanes<16>(acc[r]);
            if (l16 == 0 && m < m_end) {
              if (shared) p.o_shared[(size_t)(g0 + r) * p.H + m] = v;
              else p.o_routed[(size_t)row_slot(rl, g0 + r) * p.H + m] = v;
            }
          }
        }
      }
    }
  }
}

// residual[b][m] += o_shared[b][m] + sum_j gate[b][j] * o_routed[b*k+j][m]  (j ascending)
__global__ __launch_bounds__(256) void k_combine(ExpertParams p) {
  const int b = blockIdx.y;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= p.H) return;
  float acc = p.residual[(size_t)b * p.H + m];
  if (p.Is > 0) acc += p.o_shared[(size_t)b * p.H + m];
  for (int j = 0; j < p.k; ++j) acc = fmaf(p.gate[b * p.k + j], p.o_routed[((size_t)b * p.k + j) * p.H + m], acc);
  p.residual[(size_t)b * p.H + m] = acc;
}

int pick_rg(int B, size_t row_bytes) {
  int rg = B <= 1 ? 1 : (B <= 8 ? 2 : 4);
  while (rg > 1 && (size_t)rg * row_bytes > (size_t)LDS_BUDGET) rg >>= 1;
  return rg;
}

hipError_t launch_experts(const LayerArgs& a, hipStream_t s) {
  ExpertParams p;
  p.H = a.H;
  p.I = a.I;
  p.E = a.E;
  p.k = a.k;
  p.Is = a.Is;
  p.B = a.B;
  p.x = a.x;
  p.sg = a.sg;
  p.su = a.su;
  p.sd = a.sd;
  p.experts = a.experts;
  p.blob_bytes = a.blob.bytes;
  for (int i = 0; i < 6; ++i) p.off[i] = a.blob.off[i];
  p.sched = a.ws.sched;
  p.h_shared = a.ws.h_shared;
  p.h_routed = a.ws.h_routed;
  p.o_shared = a.ws.o_shared;
  p.o_routed = a.ws.o_routed;
  p.gate = a.gate;
  p.residual = a.residual;
  const int grid = num_cus() * 4;
  // FC1: x rows are bf16 [H]
  {
    int rg = pick_rg(a.B, (size_t)a.H * 2);
    size_t lds = (size_t)rg * a.H * 2;
    if (rg == 1) hipLaunchKernelGGL(k_fc1<1>, dim3(grid), dim3(256), lds, s, p);
    else if (rg == 2) hipLaunchKernelGGL(k_fc1<2>, dim3(grid), dim3(256), lds, s, p);
    else hipLaunchKernelGGL(k_fc1<4>, dim3(grid), dim3(256), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // FC2: h rows are fp32 [I] (routed) or [Is] (shared)
  {
    int K = a.I > a.Is ? a.I : a.Is;
    int rg = pick_rg(a.B, (size_t)K * 4);
    size_t lds = (size_t)rg * K * 4;
    if (rg == 1) hipLaunchKernelGGL(k_fc2<1>, dim3(grid), dim3(256), lds, s, p);
    else if (rg == 2) hipLaunchKernelGGL(k_fc2<2>, dim3(grid), dim3(256), lds, s, p);
    else hipLaunchKernelGGL(k_fc2<4>, dim3(grid), dim3(256), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_combine, dim3((a.H + 255) / 256, a.B), dim3(256), 0, s, p);
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
