// moe_device.h -- device building blocks of the decode layer: DPP wave
// reductions, the wave top-k with renormalised gates, the fp64-exact router
// dot product, and software-pipelined weight streams for the expert GEMVs.
// Internal to libmoe_mxfp4.so.
#pragma once

#include "mx_common.h"

namespace moe {

// ---------------------------------------------------------------------------
// DPP reductions over a 64-lane wave (gfx9 DPP: quad_perm, row mirrors, row
// broadcasts).  After the four in-row steps every lane of a 16-lane row holds
// the row's result; row_bcast:15 / row_bcast:31 fold rows into lane 63.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));        // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));        // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));       // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));       // row_mirror
  v = max(v, dpp_u32<0x142, 0xA>(v));  // row_bcast:15 into rows 1, 3
  v = max(v, dpp_u32<0x143, 0xC>(v));  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  v = min(v, dpp_u32<0x142, 0xA>(v));
  v = min(v, dpp_u32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---------------------------------------------------------------------------
// Top-k of one row of E fp32 logits by one wave, then renormalised gates.
// Order key: fp32 bits mapped to an unsigned order (-0 folded onto +0), 0 is
// the "taken" sentinel (no finite value maps to 0).  Each of the k rounds
// takes the wave max of the order keys, then the lowest expert index holding
// it, and clears that one entry; lane j keeps the j-th winner.
// gate_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float l) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int KPL>
__device__ __forceinline__ void topk_row(const float* __restrict__ l, int E, int k, int32_t* __restrict__ idx_out,
                                         float* __restrict__ gate_out) {
  const int lane = threadIdx.x & 63;
  // all KPL coherent loads are issued before any is used (one round trip)
  float lv[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) lv[i] = ld_coh(l + min(lane + 64 * i, E - 1));
  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) key[i] = (lane + 64 * i < E) ? order_key(lv[i]) : 0u;
  uint32_t my_ord = 0, top = 0;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) m = max(m, key[i]);
    const uint32_t M = wave_max_u32(m);
    uint32_t cand = 0xFFFFFFFFu;
#pragma unroll
    for (int i = KPL - 1; i >= 0; --i)
      if (key[i] == M && lane + 64 * i < E) cand = (uint32_t)(lane + 64 * i);
    const uint32_t emin = wave_min_u32(cand);
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if ((uint32_t)(lane + 64 * i) == emin) key[i] = 0u;
    if (j == 0) top = M;
    if (lane == j) {
      my_ord = M;
      my_e = (int)emin;
    }
  }
  const float l0 = order_value(top);
  const float num = (lane < k) ? expf(order_value(my_ord) - l0) : 0.0f;
  const float den = sum_lanes<64>(num);
  if (lane < k) {
    st_coh(idx_out + lane, (int32_t)my_e);
    st_coh(gate_out + lane, num / den);
  }
}

// ---------------------------------------------------------------------------
// Workgroup top-k of one row (4 waves), for the fused layer kernel.
//   phase 1: wave w takes the order keys of experts [w*Q, (w+1)*Q), Q =
//            ceil(E/4), at most TPL per lane; every lane sorts its keys by
//            (key desc, index asc); k rounds pick the wave's best remaining
//            head (DPP max of the heads; ties -- rare -- broken by a DPP min
//            of the tied heads' indices) and pop it -> 4 lists of <= k
//            candidates in LDS;
//   phase 2: wave 0 repeats the same rounds over the <= 4k candidates.
// The k experts found are exactly those of (logit desc, index asc) order
// over all E (the global top-k is contained in the union of the four
// per-quarter top-k lists).  Requires E <= 256*TPL and k <= 64.
// cand: LDS, 640 words.  Writes idx/gate (coherent) from wave 0, and returns
// slot j's expert index to lane j of wave 0.
// ---------------------------------------------------------------------------
template <int TPL>
__device__ __forceinline__ void wave_select_sorted(uint32_t (&key)[TPL], uint32_t (&ix)[TPL], int k,
                                                   uint32_t* out_key, uint32_t* out_ix) {
  const int lane = threadIdx.x & 63;
  // sort this lane's TPL entries by (key desc, index asc): insertion network
#pragma unroll
  for (int i = 1; i < TPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1] || (key[j] == key[j - 1] && ix[j] < ix[j - 1]);
      const uint32_t k0 = key[j - 1], k1 = key[j], i0 = ix[j - 1], i1 = ix[j];
      key[j - 1] = sw ? k1 : k0;
      key[j] = sw ? k0 : k1;
      ix[j - 1] = sw ? i1 : i0;
      ix[j] = sw ? i0 : i1;
    }
  for (int j = 0; j < k; ++j) {
    const uint32_t M = wave_max_u32(key[0]);
    const uint64_t tied = __ballot(key[0] == M);
    int win;
    if (__popcll(tied) == 1) {
      win = __ffsll((long long)tied) - 1;
    } else {
      const uint32_t emin = wave_min_u32(key[0] == M ? ix[0] : 0xFFFFFFFFu);
      win = __ffsll((long long)__ballot(key[0] == M && ix[0] == emin)) - 1;
    }
    const uint32_t wix = (uint32_t)__builtin_amdgcn_readlane((int)ix[0], win);
    if (lane == 0) {
      out_key[j] = M;
      out_ix[j] = wix;
    }
    if (lane == win) {  // pop the winner's head
#pragma unroll
      for (int i = 0; i + 1 < TPL; ++i) {
        key[i] = key[i + 1];
        ix[i] = ix[i + 1];
      }
      key[TPL - 1] = 0u;
      ix[TPL - 1] = 0xFFFFFFFFu;
    }
  }
}

template <int TPL>
__device__ __forceinline__ int topk_row_wg(const float* __restrict__ l, int E, int k, uint32_t* cand,
                                           int32_t* __restrict__ idx_out, float* __restrict__ gate_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Q = (E + 3) / 4, e0 = w * Q, e1 = min(E, e0 + Q);
  const int kw = min(k, max(e1 - e0, 0));
  uint32_t* ck = cand + w * 64;        // wave w's candidate keys  [64]
  uint32_t* cx = cand + 256 + w * 64;  // and expert indices       [64]
  {
    uint32_t key[TPL], ix[TPL];
    float lv[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) lv[i] = ld_coh(l + min(e0 + lane + 64 * i, E - 1));
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int e = e0 + lane + 64 * i;
      key[i] = e < e1 ? order_key(lv[i]) : 0u;
      ix[i] = e < e1 ? (uint32_t)e : 0xFFFFFFFFu;
    }
    if (kw > 0) wave_select_sorted<TPL>(key, ix, kw, ck, cx);
    for (int j = kw + lane; j < 64; j += 64) {  // unused candidate slots
      ck[j] = 0u;
      cx[j] = 0xFFFFFFFFu;
    }
  }
  __syncthreads();
  if (w == 0) {
    uint32_t key[4], ix[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      key[i] = cand[i * 64 + lane];
      ix[i] = cand[256 + i * 64 + lane];
    }
    uint32_t* fk = cand + 512;  // final keys [64]
    uint32_t* fx = cand + 576;  // final indices [64]
    wave_select_sorted<4>(key, ix, k, fk, fx);
    // lane j < k holds slot j (LDS written by lane 0 of this same wave)
    const uint32_t myk = lane < k ? fk[lane] : 0u, myx = lane < k ? fx[lane] : 0u;
    const float l0 = order_value(fk[0]);
    const float num = (lane < k) ? expf(order_value(myk) - l0) : 0.0f;
    const float den = sum_lanes<64>(num);
    if (lane < k) {
      st_coh(idx_out + lane, (int32_t)myx);
      st_coh(gate_out + lane, num / den);
    }
    return (int)myx;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// LDS activation rows are stored in 16-byte granules with granule g of a row
// at position swz(g) = g ^ ((g >> 3) & 7).  Every reader pattern in the layer
// -- consecutive granules across lanes (router, bf16 weights), granules 4c+d
// with c consecutive across lanes (MXFP4 x bf16 activations), 8c+e and 2c+e
// (fp32 activations) -- then touches 8 distinct 16-byte bank groups per 8
// lanes, i.e. no bank conflicts.  Row strides are padded to 8 granules.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int g) { return g ^ ((g >> 3) & 7); }

// ---------------------------------------------------------------------------
// Partial router dot products over granules [g_begin, g_end) of one expert
// row (8 bf16 per granule) with nr (<= RB) activation rows in LDS (swizzled,
// row stride `xstride` granules).  bf16 x bf16 products are exact in fp32 and
// are summed in fp64.  All of a lane's loads (up to 8) are issued before any
// is used; granules past g_end are multiplied by zeroed weights.  Returns the
// wave's fp64 partial sums in every lane.
template <int RB>
__device__ __forceinline__ void router_dot(const uint16_t* __restrict__ wrow, int g_begin, int g_end,
                                           const u32x4* xs, int xstride, int nr, double (&acc)[RB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.0;
  for (int c0 = g_begin + lane; c0 < g_end; c0 += 64 * 8) {
    u32x4 q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = ld_weight16(wrow + 8 * (size_t)min(c0 + 64 * i, g_end - 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = min(c0 + 64 * i, g_end - 1);
      const uint32_t msk = (c0 + 64 * i < g_end) ? 0xFFFFFFFFu : 0u;
      float wf[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        wf[2 * d] = bf16_lo(q[i][d] & msk);
        wf[2 * d + 1] = bf16_hi(q[i][d] & msk);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (RB == 1 || r < nr) {
          const u32x4 xv = xs[r * xstride + swz(c)];
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
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
    if (RB == 1 || r < nr) acc[r] = sum_lanes_f64<64>(acc[r]);
}

// ---------------------------------------------------------------------------
// Software-pipelined weight streams.  A wave walks a list of weight rows; LPR
// lanes share a row (lane l takes 16-byte chunks l, l+LPR, ...), and a row is
// cut into segments of CPL chunks per lane.  One "pass" = one segment of the
// wave's current rows.  The loads of the next two passes are in flight while
// a pass's math runs, so every wave keeps CPL to 2 x CPL 16-byte loads in
// flight per lane.  The Traits type supplies load() and math() (math of a
// row's last segment also reduces and stores that row's outputs).
// ---------------------------------------------------------------------------
template <int CPL>
struct MxBuf {  // MXFP4: 32 codes per chunk plus its E8M0 scale byte
  u32x4 q[CPL];
  uint32_t s[CPL];  // per-chunk scale bytes (general shapes)
  uint32_t sa, sb;  // two dwords of the row's scale bytes (full segments; bytes found by lane shuffles)
};

template <int CPL>
struct BfBuf {  // bf16: 8 weights per chunk
  u32x4 q[CPL];
};

// Drives P passes of a wave; Traits::load(buf, p) / Traits::math(buf, p).
// prime_passes issues the loads of the first two passes; drive_passes then
// alternates math of one pass with the loads of the pass after next, so two
// passes are in flight.  A unit may do other work (wait, stage activations)
// between the two while its first weights arrive.
template <class Buf, class Traits>
__device__ __forceinline__ void prime_passes(Traits& t, int P, Buf& a, Buf& b) {
  if (P > 0) t.load(a, 0);
  if (P > 1) t.load(b, 1);
}

template <class Buf, class Traits>
__device__ __forceinline__ void drive_passes(Traits& t, int P, Buf& a, Buf& b) {
  for (int p = 0; p < P; p += 2) {
    t.math(a, p);
    if (p + 2 < P) t.load(a, p + 2);
    if (p + 1 < P) {
      t.math(b, p + 1);
      if (p + 3 < P) t.load(b, p + 3);
    }
  }
}

template <class Buf, class Traits>
__device__ __forceinline__ void run_passes(Traits& t, int P) {
  Buf a, b;
  prime_passes(t, P, a, b);
  drive_passes(t, P, a, b);
}

}  // namespace moe
