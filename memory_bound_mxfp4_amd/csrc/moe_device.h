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

// Tagged 8-byte pairs (32-bit value | 32-bit tag << 32): data handed between
// workgroups of one launch, polled by the consumer until its tag matches.
__device__ __forceinline__ uint64_t make_pair(uint32_t v, uint32_t tag) { return ((uint64_t)tag << 32) | v; }
__device__ __forceinline__ bool pair_has(uint64_t v, uint32_t tag) { return (uint32_t)(v >> 32) == tag; }
__device__ __forceinline__ float pair_f32(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ uint64_t ld_pair(const uint64_t* p) { return ld_coh(p); }
__device__ __forceinline__ void st_pair_f32(uint64_t* p, float v, uint32_t tag) {
  st_coh(p, make_pair(__float_as_uint(v), tag));
}

// Polls until all `n` (<= N) pairs at p[idx(i)] carry `tag`.  Bounded: gives
// up (returns false) after `limit` tries, or early once the sticky error word
// *err is set (another wait of the launch already gave up).  Per-thread: no
// barrier.
template <int N, class Idx>
__device__ __forceinline__ bool poll_pairs(const uint64_t* p, int n, Idx idx, uint32_t tag, uint64_t (&v)[N],
                                           unsigned limit, const unsigned* err) {
  for (unsigned it = 0;; ++it) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ld_pair(p + idx(min(i, n - 1)));
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok &= (i >= n) || pair_has(v[i], tag);
    if (ok) return true;
    if (it >= limit || ((it & 255) == 255 && ld_coh(err) != 0u)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// poll_pairs for pairs that many workgroups read: one cached read first
// (workgroup-scope atomic loads, which may hit in this XCD's L2), and the
// coherent poll only if a pair does not carry `tag` yet.  A cached copy of a
// pair that carries this call's tag was fetched after the pair was written
// (value and tag are one 8-byte word, written by one store), so its value is
// this call's; a stale copy fails the tag test and the pair is read at the
// device coherence point instead.  A row of h that every FC2 unit of an
// expert reads is then fetched from memory about once per XCD, not once per
// unit.
template <int N, class Idx>
__device__ __forceinline__ bool poll_pairs_cached(const uint64_t* p, int n, Idx idx, uint32_t tag, uint64_t (&v)[N],
                                                  unsigned limit, const unsigned* err) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = __hip_atomic_load(const_cast<uint64_t*>(p + idx(min(i, n - 1))), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
  bool ok = true;
#pragma unroll
  for (int i = 0; i < N; ++i) ok &= (i >= n) || pair_has(v[i], tag);
  return ok || poll_pairs<N>(p, n, idx, tag, v, limit, err);
}

// ---------------------------------------------------------------------------
// Workgroup top-k of one row (4 waves), for the fused layer kernel.  Order:
// (key desc, index asc) on order-preserving integer keys, so ties go to the
// lower expert index; an entry is packed as key << 32 | ~index, so that order
// is plain 64-bit unsigned order (0 = no entry).  Every step is a short run
// of independent operations -- no serial rounds over the experts:
//   1. wave w holds experts [w Q, (w+1) Q), Q = ceil(E/4), <= TPL per lane;
//      each lane takes the best of its own entries;
//   2. the lanes are cut into G = (k rounded up to a power of two) groups of
//      64/G consecutive lanes, each group spanning all four waves; its best
//      entry comes from a few DPP steps per wave and a max over the waves.
//      T = the worst of the G group bests: the G groups are disjoint, so at
//      least G >= k entries are at least as good as T, i.e. T is no better
//      than the row's k-th best, and keeping the entries at least as good as
//      T loses none of the top k (about 50 survive at E 896, k 16);
//   3. survivors are compacted into LDS (ballot + prefix count + one LDS
//      atomic per wave);
//   4. every survivor is ranked against all survivors, the comparisons split
//      over 1, 2 or 4 adjacent lanes whose counts are added by DPP; rank
//      j < k is slot j.
// LDS `cand`: topk_lds_words(TPL) 32-bit words, 16-byte aligned.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool beats(uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__host__ __device__ constexpr int topk_lds_words(int tpl) { return 4 * 64 * 2 + 4 * 64 * tpl * 2 + 4 + 2 * 64; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Max (MAX) or min over each block of `bs` consecutive lanes (bs a power of
// two, wave-uniform); every lane of a block ends with its block's result.
template <bool MAX>
__device__ __forceinline__ uint64_t block_reduce_u64(uint64_t v, int bs) {
  auto op = [](uint64_t a, uint64_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  if (bs >= 2) v = op(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  if (bs >= 4) v = op(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  if (bs >= 8) v = op(v, dpp_u64<0x141>(v));  // row_half_mirror
  if (bs >= 16) v = op(v, dpp_u64<0x140>(v)); // row_mirror
  if (bs >= 32) v = op(v, shfl_xor_u64(v, 16));
  if (bs >= 64) v = op(v, shfl_xor_u64(v, 32));
  return v;
}

// dry: one pass over whatever the logits hold, no outputs -- run while the
// router is still working, it brings this code into the instruction cache so
// the real pass does not wait on instruction fetches.
template <int TPL>
__device__ __forceinline__ bool topk_row_wg(const uint64_t* __restrict__ l, int E, int k, uint32_t tag,
                                            unsigned limit, const unsigned* err, uint32_t* cand,
                                            int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
                                            uint64_t* idx_p, uint64_t* gate_p, bool dry) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Q = (E + 3) / 4, e0 = w * Q, e1 = min(E, e0 + Q);
  int G = 1;
  while (G < k) G <<= 1;
  const int bs = 64 / G;
  uint64_t* gbest = reinterpret_cast<uint64_t*>(cand);  // [4 waves][64] group bests
  uint32_t* surv = cand + 4 * 64 * 2;                    // [4 * 64 TPL] (key, index) pairs
  uint32_t* nsurv = surv + 4 * 64 * TPL * 2;             // survivor count
  uint32_t* out = nsurv + 4;                             // [64] (key, index) of slots 0..63
  if (threadIdx.x == 0) *nsurv = 0u;
  bool ok;
  uint32_t key[TPL], ix[TPL];
  uint64_t pk[TPL];
  {
    uint64_t lv[TPL];
    const int mine = max(0, min(TPL, (e1 - e0 - lane + 63) / 64));
    ok = poll_pairs<TPL>(l, max(mine, 1), [&](int i) { return min(e0 + lane + 64 * i, E - 1); }, tag, lv,
                         dry ? 0u : limit, err) || dry;
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int e = e0 + lane + 64 * i;
      key[i] = e < e1 ? order_key(pair_f32(lv[i])) : 0u;
      ix[i] = (uint32_t)e;
      pk[i] = key[i] != 0u ? ((uint64_t)key[i] << 32) | (0xFFFFFFFFu - ix[i]) : 0ull;
      best = pk[i] > best ? pk[i] : best;
    }
    best = block_reduce_u64<true>(best, bs);
    if ((lane & (bs - 1)) == 0) gbest[w * 64 + lane / bs] = best;
  }
  __syncthreads();
  uint64_t T;
  {
    uint64_t g = ~0ull;  // neutral for the min
    if (lane < G) {
      const uint64_t a = max(gbest[lane], gbest[64 + lane]), b = max(gbest[128 + lane], gbest[192 + lane]);
      g = max(a, b);
    }
    g = block_reduce_u64<false>(g, G);
    T = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(g >> 32), 0) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)g, 0);
  }
  {
    bool keep[TPL];
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      keep[i] = pk[i] != 0ull && pk[i] >= T;
      n += (uint32_t)__popcll(__ballot(keep[i]));
    }
    uint32_t base = 0;
    if (lane == 0 && n > 0) base = atomicAdd(nsurv, n);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint64_t m = __ballot(keep[i]);
      const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (keep[i]) {
        surv[2 * pos] = key[i];
        surv[2 * pos + 1] = ix[i];
      }
      base += (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  // rank every survivor against all survivors; survivor s is compared by the
  // `parts` adjacent threads s * parts + (0 .. parts-1), each taking an even
  // stretch of the list (two entries per 16-byte LDS read)
  const uint32_t n = *nsurv;
  const int lp = n <= 64u ? 2 : (n <= 128u ? 1 : 0);  // log2(parts)
  const uint32_t span = (((n + (1u << lp) - 1) >> lp) + 1u) & ~1u;
  for (uint32_t base = 0; base < (n << lp); base += 256) {
    const uint32_t t = base + threadIdx.x, sidx = t >> lp, part = t & ((1u << lp) - 1u);
    const bool live = sidx < n;
    uint32_t mk = 0, mi = 0;
    int r = 0;
    if (live) {
      mk = surv[2 * sidx];
      mi = surv[2 * sidx + 1];
      const uint32_t j0 = min(n, part * span), j1 = min(n, j0 + span);
      uint32_t j = j0;
      for (; j + 4 <= j1; j += 4) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(surv + 2 * j);
        const u32x4 b = *reinterpret_cast<const u32x4*>(surv + 2 * j + 4);
        r += (beats(a[0], a[1], mk, mi) ? 1 : 0) + (beats(a[2], a[3], mk, mi) ? 1 : 0) +
             (beats(b[0], b[1], mk, mi) ? 1 : 0) + (beats(b[2], b[3], mk, mi) ? 1 : 0);
      }
      for (; j < j1; ++j) r += beats(surv[2 * j], surv[2 * j + 1], mk, mi) ? 1 : 0;
    }
    if (lp >= 1) r += (int)dpp_u32<0xB1>((uint32_t)r);  // quad_perm [1,0,3,2]: the partner lane's count
    if (lp >= 2) r += (int)dpp_u32<0x4E>((uint32_t)r);  // quad_perm [2,3,0,1]
    if (live && part == 0u && r < k) {
      out[2 * r] = mk;
      out[2 * r + 1] = mi;
    }
  }
  __syncthreads();
  if (w == 0) {
    const uint32_t myk = lane < k ? out[2 * lane] : 0u, myx = lane < k ? out[2 * lane + 1] : 0u;
    const float l0 = order_value(out[0]);
    const float num = (lane < k) ? expf(order_value(myk) - l0) : 0.0f;
    const float den = sum_lanes<64>(num);
    if (lane < k && !dry) {
      const float g = num / den;
      idx_out[lane] = (int32_t)myx;
      gate_out[lane] = g;
      st_coh(idx_p + lane, make_pair(myx, tag));
      st_pair_f32(gate_p + lane, g, tag);
    }
  }
  return ok;
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
