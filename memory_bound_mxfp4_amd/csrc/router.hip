// router.hip -- router GEMV with exact fp64 accumulation, wave-level top-k
// with renormalised gates, and the device-side expert-gathered schedule.
//
// The router, top-16 selection and shared/routed experts are the per-layer
// work of "Kimi K3 on GB300: 13 kernels a layer" (section "What one decode
// step of Kimi K3 does"); the same page's section "Why batch 1 on a rack is
// not only a bandwidth problem" names router scores and top-16 selection as
// short, dependent, bandwidth-idle work -- so these kernels aim at latency:
// every expert row is streamed once by one wave, and selection is a handful
// of wave-wide butterfly reductions with no host round trip.
#include "internal.h"
#include "mx_common.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits.  One wave per expert row, all batch rows per wave; x rows
// are staged in LDS (RB rows at a time).  bf16 x bf16 products are exact in
// fp32; they are summed in fp64 (exact for this data up to 2^-52 relative),
// the bias is added in fp64 and the result is rounded to fp32 once.
// grid: ceil(E/4) blocks of 256 threads; LDS: RB * H * 2 bytes.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x, int B, int H,
                                                       const uint16_t* __restrict__ wr, const float* __restrict__ bias,
                                                       int E, float* __restrict__ logits) {
  extern __shared__ u32x4 xs_raw[];
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(xs_raw);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  const int C = H / 8;  // 16-byte chunks per row
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + (size_t)(e < E ? e : 0) * H);
  for (int b0 = 0; b0 < B; b0 += RB) {
    const int nb = min(RB, B - b0);
    __syncthreads();
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)b0 * H);
    for (int i = threadIdx.x; i < nb * C; i += 256) xs_raw[i] = src[i];
    __syncthreads();
    if (e >= E) continue;
    double acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.0;
    for (int c = lane; c < C; c += 64) {
      u32x4 w = ld_weight16(wrow + c);
      float wf[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        wf[2 * d] = bf16_lo(w[d]);
        wf[2 * d + 1] = bf16_hi(w[d]);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < nb) {
          u32x4 xv = reinterpret_cast<const u32x4*>(xs + (size_t)r * H)[c];
          double a = acc[r];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            a += (double)(wf[2 * d] * bf16_lo(xv[d]));
            a += (double)(wf[2 * d + 1] * bf16_hi(xv[d]));
          }
          acc[r] = a;
        }
      }
    }
    const double bb = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < nb) {
        double t = sum_lanes_f64<64>(acc[r]);
        if (lane == 0) logits[(size_t)(b0 + r) * E + e] = (float)(t + bb);
      }
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, int B, int H, const uint16_t* wr, const float* bias, int E,
                                float* logits, hipStream_t s) {
  const int RB = 4;
  size_t lds = (size_t)RB * H * 2;
  dim3 grid((E + 3) / 4);
  hipLaunchKernelGGL(k_router_logits<RB>, grid, dim3(256), lds, s, x, B, H, wr, bias, E, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k + gates.  One wave per row.  Each logit becomes a 64-bit key whose
// high word orders fp32 values (with -0 folded onto +0) and whose low word is
// ~e, so the largest key is the largest logit with the lowest index.  k rounds
// of (lane-local max, 6-step butterfly max, winner clears its key) select the
// experts in order; lane j then holds slot j.
// gate_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the softmax renormalised
// over the selected experts.
// grid: B blocks of 64 threads.  KPL = keys per lane (E <= 64 * KPL).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t logit_key(float l, int e) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

template <int KPL>
__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ logits, int E, int k, int32_t* __restrict__ idx,
                                             float* __restrict__ gate) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* l = logits + (size_t)b * E;
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    int e = lane + 64 * i;
    key[i] = (e < E) ? logit_key(l[e], e) : 0ull;
  }
  int my_e = 0;
  uint64_t top0 = 0, mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) m = key[i] > m ? key[i] : m;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      uint64_t o = shfl_xor_u64(m, s);
      m = o > m ? o : m;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (key[i] == m) key[i] = 0ull;
    if (j == 0) top0 = m;
    if (lane == j) {
      mine = m;
      my_e = (int)(~(uint32_t)m);
    }
  }
  // recover the logit values from the keys (exact inverse of logit_key)
  auto key_val = [](uint64_t kk) {
    uint32_t ord = (uint32_t)(kk >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
  };
  const float l0 = key_val(top0);
  float num = (lane < k) ? expf(key_val(mine) - l0) : 0.0f;
  float den = sum_lanes<64>(num);
  if (lane < k) {
    idx[(size_t)b * k + lane] = my_e;
    gate[(size_t)b * k + lane] = num / den;
  }
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

// ---------------------------------------------------------------------------
// Expert-gathered schedule: invert [B][k] routing into the distinct experts
// (ascending) and, for each, the list of slots s = b*k + j that use it.  One
// block of 1024 threads; per-expert counts live in LDS.  The order of slots
// within one expert's list is irrelevant to every result (each slot's output
// is computed independently).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_schedule(const int32_t* __restrict__ idx, int nslots, int E, int* n_active,
                                                   int* active, int* row_off, int* rows) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int start[MOE_MAX_EXPERTS];
  __shared__ int wave_tot[16];
  __shared__ int wave_act[16];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int s = t; s < nslots; s += 1024) atomicAdd(&cnt[idx[s]], 1);
  __syncthreads();
  // exclusive scans of cnt[] and of (cnt[] > 0) over E entries: each thread
  // owns a contiguous run of ceil(E/1024) entries.
  const int per = (E + 1023) / 1024;
  const int e0 = t * per;
  int run_rows = 0, run_act = 0;
  for (int i = 0; i < per; ++i) {
    int e = e0 + i;
    if (e < E) {
      run_rows += cnt[e];
      run_act += cnt[e] > 0;
    }
  }
  // inclusive wave scan
  const int lane = t & 63, w = t >> 6;
  int ir = run_rows, ia = run_act;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int vr = __shfl_up(ir, d, 64), va = __shfl_up(ia, d, 64);
    if (lane >= d) {
      ir += vr;
      ia += va;
    }
  }
  if (lane == 63) {
    wave_tot[w] = ir;
    wave_act[w] = ia;
  }
  __syncthreads();
  int base_r = 0, base_a = 0;
  for (int i = 0; i < w; ++i) {
    base_r += wave_tot[i];
    base_a += wave_act[i];
  }
  int pr = base_r + ir - run_rows, pa = base_a + ia - run_act;  // exclusive prefix at e0
  for (int i = 0; i < per; ++i) {
    int e = e0 + i;
    if (e < E) {
      start[e] = pr;
      if (cnt[e] > 0) {
        active[pa] = e;
        row_off[pa] = pr;
        ++pa;
      }
      pr += cnt[e];
    }
  }
  if (t == 1023) {
    *n_active = base_a + ia;
    row_off[base_a + ia] = base_r + ir;
  }
  __syncthreads();
  for (int s = t; s < nslots; s += 1024) {
    int e = idx[s];
    int pos = atomicAdd(&start[e], 1);
    rows[pos] = s;
  }
}

hipError_t launch_schedule(const int32_t* idx, int B, int k, int E, Sched sc, hipStream_t s) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), 0, s, idx, B * k, E, sc.n_active, sc.active, sc.row_off,
                     sc.rows);
  return hipGetLastError();
}

}  // namespace moe
