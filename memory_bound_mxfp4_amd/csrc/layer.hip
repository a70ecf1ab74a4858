// layer.hip -- the whole MoE decode layer as ONE persistent kernel.
//
// The pages this follows ("Kimi K3 on GB300: 13 kernels a layer", sections
// "Why batch 1 on a rack is not only a bandwidth problem" and "What the fused
// path changes") find that at batch 1 most of a decode step is spent between
// kernels -- launch ramps, drains, serial router/top-k work -- and answer with
// a fused MoE front, one persistent kernel for the routed experts' FC1+FC2,
// and a tail that folds the down-projection reduction into what follows.
// On one MI355X the same goal is met with a single launch:
//
//   * workgroups pop "units" from an in-order device queue (one atomic);
//   * unit kinds, in queue order:
//       router GEMV (4 experts x a block of rows)      -> logits
//       routing (top-k + gates of one row; the last one builds the
//                expert-gathered schedule)             -> idx, gate, schedule
//       shared-expert FC1+SwiGLU (tile of Is rows)     -> h_shared
//       routed FC1+SwiGLU (expert, tile of I rows)     -> h_routed
//       shared-expert FC2 (64 rows of H)               -> o_shared
//       routed FC2 (expert, tile of 256 rows of H)     -> o_routed, and the
//                last contribution to a 256-row tile folds residual +=
//                o_shared + sum_j gate_j o_j for that tile (fixed j order);
//   * a unit waits only on units earlier in the queue (on a counter their
//     completions bump), so the smallest unfinished unit can always run: no
//     residency assumption, no deadlock; every wait is bounded and sets a
//     sticky error word instead of hanging;
//   * data handed between workgroups moves with coherent (sc1) loads and
//     stores, so no L2 write-back or invalidate is ever issued -- on MI355X
//     those serialise device-wide at a few per microsecond; coherent loads
//     travel to the device coherence point, so they are always issued in
//     batches (one round trip per batch);
//   * the router and the shared expert need no routing, so they stream while
//     top-k runs, hiding its latency; routed FC2 of one expert overlaps FC1 of
//     the next; the combine happens in the FC2 tail.
//
// Weight streams are branch-free: every lane issues all of a pass's 16-byte
// loads (clamped to the row), and chunks past the row end are masked to zero
// in the math, so the compiler keeps a whole pass (and the next pass) in
// flight instead of waiting load by load.
//
// The control block at the start of the workspace is zeroed once by
// moe_workspace_init and left zeroed by every call (the last workgroup to
// exit clears it), so a call needs no separate clearing launch.
#include "internal.h"
#include "moe_device.h"

#include <algorithm>

namespace moe {

constexpr int NT1 = 16;   // routed FC1 rows (of I) per unit: 16 x 2 x 3.8 KB at H 7168
constexpr int NTS1 = 4;   // shared FC1 rows (of Is) per unit: 4 x 2 x 14 KB of bf16
constexpr int NT2 = 256;  // FC2 tile (rows of H): the combine's granularity
constexpr int NTS2 = 32;  // shared FC2 rows per unit
constexpr int NTR2 = 128; // routed FC2 rows per unit
constexpr int SUB2 = NT2 / NTS2;  // shared FC2 units per tile
constexpr int SUBR = NT2 / NTR2;  // routed FC2 units per tile and expert
constexpr int CPL1 = 7;   // FC1: 16-byte chunks per lane per pass (half-wave rows)
constexpr int CPL2 = 6;   // FC2: 16-byte chunks per lane per pass (8 lanes per row)
constexpr int MAX_ROWS = MOE_MAX_BATCH;    // activation rows one expert can have
constexpr unsigned SPIN_LIMIT = 1u << 20;  // ~1 s of polls (at ~1 us each) before a wait gives up

struct LayerParams {
  int H, I, E, k, Is, B;
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  const uint16_t *sg, *su, *sd;
  const uint8_t* experts;
  size_t blob_bytes;
  size_t off[6];
  float* residual;
  int32_t* idx;
  float* gate;
  float* logits;
  int* active;
  int* row_off;
  int* rows;
  float* h_shared;
  float* h_routed;
  float* o_shared;
  float* o_routed;
  unsigned* ctrl;
  int umax;
  int n_rt_e;  // router expert pairs (2 experts per unit, 2 waves per expert)
  int n_rt;    // router units = n_rt_e * row blocks
  int n_rb;    // router row blocks
  int n_static;  // units 0 .. n_static-1 go to workgroups 0 .. n_static-1
  int n_s1;    // shared FC1 units
  int T1;      // routed FC1 tiles per expert
  int T2;      // FC2 tiles over H (the combine's granularity)
  int n_s2;    // shared FC2 units (SUB2 per tile)
  int ctrl_words;
  int xstride;        // LDS x row stride, 16-byte granules (multiple of 8)
  int hstride;        // LDS h row stride, 16-byte granules (multiple of 8)
  int lds_h_off;      // byte offset of the h staging region in dynamic LDS
  int lds_sched_off;  // byte offset of the schedule copy in dynamic LDS
};

// ---- synchronisation helpers (the whole workgroup calls them) ---------------
//
// Producers write shared data with coherent stores (st_coh), wait until all
// of their memory operations have completed (s_waitcnt 0), meet at a barrier,
// and one thread bumps a counter with an agent-scope atomic.  Consumers poll
// the counter (agent-scope atomic loads), meet at a barrier, and read the data
// with coherent loads (ld_coh).  Compiler signal fences keep the accesses on
// their side of the handshake.  There is no L2 write-back or invalidate.

__device__ __forceinline__ unsigned ld_ctrl(const unsigned* a) {
  return __hip_atomic_load(const_cast<unsigned*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *a >= target.  Polls back off exponentially (to ~1 us between
// polls) so that hundreds of waiting workgroups do not flood the coherence
// point that every coherent access goes through.  Gives up after about a
// second and sets the sticky error word (the unit then computes on whatever
// it finds).
__device__ __forceinline__ void wg_wait_geq(const LayerParams& p, const unsigned* a, unsigned target) {
  if (threadIdx.x == 0) {
    unsigned it = 0, nap = 1;
    while (ld_ctrl(a) < target) {
      if (nap <= 1) __builtin_amdgcn_s_sleep(1);
      else if (nap <= 2) __builtin_amdgcn_s_sleep(2);
      else if (nap <= 4) __builtin_amdgcn_s_sleep(4);
      else if (nap <= 8) __builtin_amdgcn_s_sleep(8);
      else if (nap <= 16) __builtin_amdgcn_s_sleep(16);
      else __builtin_amdgcn_s_sleep(32);
      nap = nap < 32 ? 2 * nap : 32;
      if (++it >= SPIN_LIMIT) {
        __hip_atomic_fetch_or((p.ctrl + ctrl_word(CTRL_ERR)), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// All of this workgroup's coherent stores complete, then *a += 1.
// Returns the old value to thread 0 (others get 0).
__device__ __forceinline__ unsigned wg_signal_add(unsigned* a) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old;
}

__device__ __forceinline__ uint64_t ld_coh64(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ---- per-workgroup state ------------------------------------------------------

struct Lds {  // static LDS of the kernel
  int next;        // next unit index
  int flag;        // "this workgroup is the last arriver"
  int wtot[8];     // scan scratch
  int nrows;       // rows of the current unit
  int expert;      // expert of the current routed unit (batch 1)
  double part[4][4];  // router: partial sums of the second half-row waves [wave][row]
  int slot[MAX_ROWS];  // slot ids (routed) or batch rows (shared) of the current unit
};

struct WgState {
  bool x_cached;    // batch 1: x row 0 already in LDS
  bool route_seen;  // this workgroup has seen the routing published
  int U;
  const int* s_active;   // LDS copy of the schedule (valid once route_seen)
  const int* s_row_off;
  const int* s_rows;
};

// Copy the published schedule into this workgroup's LDS (one batch of
// coherent loads), so routed units read it without a round trip.
__device__ __forceinline__ void cache_schedule(const LayerParams& p, WgState& st, int* sc) {
  const int U = st.U, nslots = p.B * p.k;
  int* a = sc;
  int* ro = sc + p.umax;
  int* rw = ro + p.umax + 1;
  const int total = U + (U + 1) + nslots;
  for (int base = threadIdx.x; base < total; base += 256 * 8) {
    int v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = min(base + 256 * t, total - 1);
      v[t] = i < U ? ld_coh(p.active + i) : (i < 2 * U + 1 ? ld_coh(p.row_off + (i - U)) : ld_coh(p.rows + (i - 2 * U - 1)));
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = base + 256 * t;
      if (i < total) {
        if (i < U) a[i] = v[t];
        else if (i < 2 * U + 1) ro[i - U] = v[t];
        else rw[i - 2 * U - 1] = v[t];
      }
    }
  }
  __syncthreads();
  st.s_active = a;
  st.s_row_off = ro;
  st.s_rows = rw;
}

// Row list of the current unit: batch rows 0..B-1 for the shared expert,
// slots s = b*k + j of routed expert a (from the LDS schedule copy).
__device__ __forceinline__ void load_rows(const LayerParams& p, const WgState& st, Lds& L, int a) {
  __syncthreads();
  if (a < 0) {
    if (threadIdx.x < p.B) L.slot[threadIdx.x] = threadIdx.x;
    if (threadIdx.x == 0) L.nrows = p.B;
  } else {
    const int r0 = st.s_row_off[a], n = min(st.s_row_off[a + 1] - r0, MAX_ROWS);
    if (threadIdx.x < n) L.slot[threadIdx.x] = st.s_rows[r0 + threadIdx.x];
    if (threadIdx.x == 0) L.nrows = n;
  }
  __syncthreads();
}

// x rows (bf16 input of the launch) of the current unit's rows [g0, g0+nr)
// into LDS (swizzled granules, row stride p.xstride granules).
__device__ __forceinline__ void stage_x(const LayerParams& p, WgState& st, const Lds& L, u32x4* xs, bool routed,
                                        int g0, int nr) {
  if (p.B == 1 && st.x_cached) return;
  __syncthreads();
  const int per_row = p.H / 8;
  for (int i = threadIdx.x; i < nr * per_row; i += 256) {
    const int r = i / per_row, c = i - r * per_row;
    const int b = routed ? L.slot[g0 + r] / p.k : L.slot[g0 + r];
    xs[r * p.xstride + swz(c)] = reinterpret_cast<const u32x4*>(p.x + (size_t)b * p.H)[c];
  }
  __syncthreads();
  st.x_cached = (p.B == 1);
}

// h rows (fp32 intermediate written earlier in this launch) of rows [g0,
// g0+nr), row r taken from src[slot(r)]; coherent 8-byte loads, 8 per thread
// per batch, into LDS (swizzled 16-byte granules, row stride p.hstride).
__device__ __forceinline__ void stage_h(const LayerParams& p, u32x4* hs, const float* src, const Lds& L, int g0,
                                        int nr, int K) {
  __syncthreads();
  const int per_row = K / 2, total = nr * per_row;
  uint64_t* h64 = reinterpret_cast<uint64_t*>(hs);
  for (int base = threadIdx.x; base < total; base += 256 * 8) {
    uint64_t v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = min(base + 256 * t, total - 1);
      const int r = i / per_row, c = i - r * per_row;
      v[t] = ld_coh64(src + (size_t)L.slot[g0 + r] * K + 2 * c);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = base + 256 * t;
      if (i < total) {
        const int r = i / per_row, c = i - r * per_row;  // u64 c = granule c/2, half c%2
        h64[2 * (r * p.hstride + swz(c >> 1)) + (c & 1)] = v[t];
      }
    }
  }
  __syncthreads();
}

// ---- weight streams (see run_passes) ------------------------------------------
//
// FC1: half a wave per weight row -- lanes 0-31 the gate row, lanes 32-63 the
// up row of the same output n -- rows n = n0, n0+4, ... of the unit's tile.
// FC2: 8 lanes per weight row, 8 rows per wave pass, 32 rows per block pass.

// FULL: every segment of every row is complete and every row of the tile
// exists, so chunk offsets are compile-time immediates and nothing is clamped
// or masked (the case at the K3 shapes); otherwise loads are clamped and the
// overhang masked.
template <int RG, bool FULL>
struct Fc1Mx {
  const uint8_t *codes, *scales;  // this lane's matrix (gate or up), row 0
  int H, C, nseg, n0;
  const u32x4* xs;  // LDS x rows (swizzled)
  int xstride;
  int nr;
  float acc[RG];
  float* out;  // h rows, indexed by slot
  int out_ld;
  const int* slot;
  __device__ void load(MxBuf<CPL1>& b, int p) {
    const int i = p / nseg, s = p - i * nseg, n = n0 + 4 * i;
    const int l = threadIdx.x & 31;
    const int c0 = s * 32 * CPL1 + l;
    const uint8_t* cr = codes + (size_t)n * (H / 2) + 16 * c0;
    const uint8_t* sr = scales + (size_t)n * (H / 32) + c0;
#pragma unroll
    for (int ci = 0; ci < CPL1; ++ci) {
      const int dc = FULL ? 32 * ci : min(c0 + 32 * ci, C - 1) - c0;
      b.q[ci] = ld_weight16(cr + 16 * dc);
      if (!FULL) b.s[ci] = sr[dc];
    }
    if (FULL) {  // this half-wave's 224 scale bytes of the segment: two dwords per lane
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(scales + (size_t)n * (H / 32) + s * 32 * CPL1);
      b.sa = __builtin_nontemporal_load(s32 + l);
      b.sb = __builtin_nontemporal_load(s32 + 32 + min(l, 8 * CPL1 - 33));
    }
  }
  __device__ void math(const MxBuf<CPL1>& b, int p) {
    const int i = p / nseg, s = p - i * nseg;
    const int lane = threadIdx.x & 63, l = lane & 31;
#pragma unroll
    for (int ci = 0; ci < CPL1; ++ci) {
      const int craw = s * 32 * CPL1 + l + 32 * ci;
      const int c = FULL ? craw : min(craw, C - 1);
      const uint32_t msk = (FULL || craw < C) ? 0xFFFFFFFFu : 0u;
      uint32_t sbyte;
      if (FULL) {  // byte l + 32 ci of the segment = dword l/4 + 8 ci, held by lane (l/4 + 8 ci) mod 32
        const int q = (l >> 2) + 8 * ci;
        const uint32_t wv = __shfl(ci < 4 ? b.sa : b.sb, (lane & 32) | (q & 31), WAVE);
        sbyte = (wv >> (8 * (l & 3))) & 0xFFu;
      } else {
        sbyte = b.s[ci];
      }
      const float sc = e8m0_scale(sbyte);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        bf16x2 w[4];
        dq4_bf16(FULL ? b.q[ci][d] : (b.q[ci][d] & msk), sc, w);
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (RG == 1 || r < nr) {
            const u32x4 xv = xs[r * xstride + swz(4 * c + d)];
            float a = acc[r];
            a = dot2_bf16(w[0], xv[0], a);
            a = dot2_bf16(w[1], xv[1], a);
            a = dot2_bf16(w[2], xv[2], a);
            a = dot2_bf16(w[3], xv[3], a);
            acc[r] = a;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each chunk's LDS reads and dequant local
    }
    if (s == nseg - 1) {
      const int n = n0 + 4 * i;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const float g = sum_lanes<32>(acc[r]);
          const float u = __shfl(g, 32, WAVE);
          if (lane == 0) st_coh(out + (size_t)slot[r] * out_ld + n, silu_f(g) * u);
        }
        acc[r] = 0.0f;
      }
    }
  }
};

template <int RG, bool FULL>
struct Fc1Bf {
  const uint16_t* w;  // this lane's matrix (gate or up), row 0
  int H, C8, nseg, n0;
  const u32x4* xs;  // LDS x rows (swizzled)
  int xstride;
  int nr;
  float acc[RG];
  float* out;  // h_shared rows, indexed by batch row
  int out_ld;
  const int* row;
  __device__ void load(BfBuf<CPL1>& b, int p) {
    const int i = p / nseg, s = p - i * nseg, n = n0 + 4 * i;
    const int l = threadIdx.x & 31;
    const int c0 = s * 32 * CPL1 + l;
    const uint16_t* wrow = w + (size_t)n * H + 8 * c0;
#pragma unroll
    for (int ci = 0; ci < CPL1; ++ci) {
      const int dc = FULL ? 32 * ci : min(c0 + 32 * ci, C8 - 1) - c0;
      b.q[ci] = ld_weight16(wrow + 8 * dc);
    }
  }
  __device__ void math(const BfBuf<CPL1>& b, int p) {
    const int i = p / nseg, s = p - i * nseg;
    const int l = threadIdx.x & 31;
#pragma unroll
    for (int ci = 0; ci < CPL1; ++ci) {
      const int craw = s * 32 * CPL1 + l + 32 * ci;
      const int c = FULL ? craw : min(craw, C8 - 1);
      const uint32_t msk = (FULL || craw < C8) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const u32x4 xv = xs[r * xstride + swz(c)];
          float a = acc[r];
          a = dot2_bf16(b.q[ci][0] & msk, xv[0], a);
          a = dot2_bf16(b.q[ci][1] & msk, xv[1], a);
          a = dot2_bf16(b.q[ci][2] & msk, xv[2], a);
          a = dot2_bf16(b.q[ci][3] & msk, xv[3], a);
          acc[r] = a;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s == nseg - 1) {
      const int n = n0 + 4 * i;
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const float g = sum_lanes<32>(acc[r]);
          const float u = __shfl(g, 32, WAVE);
          if (lane == 0) st_coh(out + (size_t)row[r] * out_ld + n, silu_f(g) * u);
        }
        acc[r] = 0.0f;
      }
    }
  }
};

template <int RG, bool FULL>
struct Fc2Mx {
  const uint8_t *codes, *scales;  // down matrix row 0
  int K, C, nseg, m_begin, m_end;
  const u32x4* hs;  // LDS h rows (swizzled)
  int hstride;
  int nr;
  float acc[RG];
  float* out;  // o_routed rows, indexed by slot
  int out_ld;
  const int* slot;
  __device__ int row_of(int grp) const {
    return m_begin + ((threadIdx.x >> 6) + 4 * grp) * 8 + ((threadIdx.x & 63) >> 3);
  }
  __device__ void load(MxBuf<CPL2>& b, int p) {
    const int grp = p / nseg, s = p - grp * nseg;
    const int m = FULL ? row_of(grp) : min(row_of(grp), m_end - 1);
    const int l = threadIdx.x & 7;
    const int c0 = s * 8 * CPL2 + l;
    const uint8_t* cr = codes + (size_t)m * (K / 2) + 16 * c0;
    const uint8_t* sr = scales + (size_t)m * (K / 32) + c0;
#pragma unroll
    for (int ci = 0; ci < CPL2; ++ci) {
      const int dc = FULL ? 8 * ci : min(c0 + 8 * ci, C - 1) - c0;
      b.q[ci] = ld_weight16(cr + 16 * dc);
      if (!FULL) b.s[ci] = sr[dc];
    }
    if (FULL) {  // this 8-lane group's 48 scale bytes of the segment: two dwords per lane
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(scales + (size_t)m * (K / 32) + s * 8 * CPL2);
      b.sa = __builtin_nontemporal_load(s32 + l);
      b.sb = __builtin_nontemporal_load(s32 + 8 + min(l, 2 * CPL2 - 9));
    }
  }
  __device__ void math(const MxBuf<CPL2>& b, int p) {
    const int grp = p / nseg, s = p - grp * nseg, m = row_of(grp);
    const int lane = threadIdx.x & 63, l = lane & 7;
#pragma unroll
    for (int ci = 0; ci < CPL2; ++ci) {
      const int craw = s * 8 * CPL2 + l + 8 * ci;
      const int c = FULL ? craw : min(craw, C - 1);
      const uint32_t msk = (FULL || craw < C) ? 0xFFFFFFFFu : 0u;
      uint32_t sbyte;
      if (FULL) {  // byte l + 8 ci = dword l/4 + 2 ci, held by group lane (l/4 + 2 ci) mod 8
        const int q = (l >> 2) + 2 * ci;
        const uint32_t wv = __shfl(ci < 4 ? b.sa : b.sb, (lane & ~7) | (q & 7), WAVE);
        sbyte = (wv >> (8 * (l & 3))) & 0xFFu;
      } else {
        sbyte = b.s[ci];
      }
      const float sc = e8m0_scale(sbyte);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f32x2 w[4];
        dq4_f32(FULL ? b.q[ci][d] : (b.q[ci][d] & msk), sc, w);
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          if (RG == 1 || r < nr) {
            const f32x4 x0 = __builtin_bit_cast(f32x4, hs[r * hstride + swz(8 * c + 2 * d)]);
            const f32x4 x1 = __builtin_bit_cast(f32x4, hs[r * hstride + swz(8 * c + 2 * d + 1)]);
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
        __builtin_amdgcn_sched_barrier(0);  // one dword of codes at a time
      }
    }
    if (s == nseg - 1) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const float v = sum_lanes<8>(acc[r]);
          if (l == 0 && (FULL || m < m_end)) st_coh(out + (size_t)slot[r] * out_ld + m, v);
        }
        acc[r] = 0.0f;
      }
    }
  }
};

template <int RG, bool FULL>
struct Fc2Bf {
  const uint16_t* w;  // shared down [H][Is]
  int K, C8, nseg, m_begin, m_end;
  const u32x4* hs;  // LDS h rows (swizzled)
  int hstride;
  int nr;
  float acc[RG];
  float* out;  // o_shared rows, indexed by batch row
  int out_ld;
  const int* row;
  __device__ int row_of(int grp) const {
    return m_begin + ((threadIdx.x >> 6) + 4 * grp) * 8 + ((threadIdx.x & 63) >> 3);
  }
  __device__ void load(BfBuf<CPL2>& b, int p) {
    const int grp = p / nseg, s = p - grp * nseg;
    const int m = FULL ? row_of(grp) : min(row_of(grp), m_end - 1);
    const int l = threadIdx.x & 7;
    const int c0 = s * 8 * CPL2 + l;
    const uint16_t* wrow = w + (size_t)m * K + 8 * c0;
#pragma unroll
    for (int ci = 0; ci < CPL2; ++ci) {
      const int dc = FULL ? 8 * ci : min(c0 + 8 * ci, C8 - 1) - c0;
      b.q[ci] = ld_weight16(wrow + 8 * dc);
    }
  }
  __device__ void math(const BfBuf<CPL2>& b, int p) {
    const int grp = p / nseg, s = p - grp * nseg, m = row_of(grp);
    const int l = threadIdx.x & 7;
#pragma unroll
    for (int ci = 0; ci < CPL2; ++ci) {
      const int craw = s * 8 * CPL2 + l + 8 * ci;
      const int c = FULL ? craw : min(craw, C8 - 1);
      const uint32_t msk = (FULL || craw < C8) ? 0xFFFFFFFFu : 0u;
      const uint32_t q0 = b.q[ci][0] & msk, q1 = b.q[ci][1] & msk, q2 = b.q[ci][2] & msk, q3 = b.q[ci][3] & msk;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const f32x4 x0 = __builtin_bit_cast(f32x4, hs[r * hstride + swz(2 * c)]);
          const f32x4 x1 = __builtin_bit_cast(f32x4, hs[r * hstride + swz(2 * c + 1)]);
          float a = acc[r];
          a = fmaf(bf16_lo(q0), x0.x, a);
          a = fmaf(bf16_hi(q0), x0.y, a);
          a = fmaf(bf16_lo(q1), x0.z, a);
          a = fmaf(bf16_hi(q1), x0.w, a);
          a = fmaf(bf16_lo(q2), x1.x, a);
          a = fmaf(bf16_hi(q2), x1.y, a);
          a = fmaf(bf16_lo(q3), x1.z, a);
          a = fmaf(bf16_hi(q3), x1.w, a);
          acc[r] = a;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s == nseg - 1) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (RG == 1 || r < nr) {
          const float v = sum_lanes<8>(acc[r]);
          if (l == 0 && (FULL || m < m_end)) st_coh(out + (size_t)row[r] * out_ld + m, v);
        }
        acc[r] = 0.0f;
      }
    }
  }
};

// ---- units --------------------------------------------------------------------

__device__ __forceinline__ unsigned* ctrl_at(const LayerParams& p, int line) { return p.ctrl + ctrl_word(line); }
__device__ __forceinline__ int line_fc1(int a) { return CTRL_FC1 + a; }
__device__ __forceinline__ int line_tile(const LayerParams& p, int t) { return CTRL_FC1 + p.umax + t; }
__device__ __forceinline__ int line_rb(const LayerParams& p, int rb) { return CTRL_FC1 + p.umax + p.T2 + rb; }
__device__ __forceinline__ int line_pub(const LayerParams& p, int j) {
  return CTRL_FC1 + p.umax + p.T2 + MOE_MAX_BATCH + j;
}

// Expert-gathered schedule from idx[B][k] (LDS counting; 256 threads).
// LDS: cnt[E], start[E], ids[B*k].
__device__ void build_schedule(const LayerParams& p, int* cnt, int* wtot /* LDS [8] */) {
  int* start = cnt + p.E;
  int* ids = start + p.E;
  const int t = threadIdx.x, nslots = p.B * p.k;
  // every slot's expert id, coherent loads in batches of 4 per thread
  for (int base = t; base < nslots; base += 256 * 4) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_coh(p.idx + min(base + 256 * i, nslots - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + 256 * i < nslots) ids[base + 256 * i] = v[i];
  }
  for (int e = t; e < p.E; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int s = t; s < nslots; s += 256) atomicAdd(&cnt[ids[s]], 1);
  __syncthreads();
  const int per = (p.E + 255) / 256, e0 = t * per;
  int run_rows = 0, run_act = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < p.E) {
      run_rows += cnt[e];
      run_act += cnt[e] > 0;
    }
  }
  const int lane = t & 63, w = t >> 6;
  int ir = run_rows, ia = run_act;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int vr = __shfl_up(ir, d, 64), va = __shfl_up(ia, d, 64);
    if (lane >= d) {
      ir += vr;
      ia += va;
    }
  }
  if (lane == 63) {
    wtot[w] = ir;
    wtot[4 + w] = ia;
  }
  __syncthreads();
  int base_r = 0, base_a = 0;
  for (int i = 0; i < w; ++i) {
    base_r += wtot[i];
    base_a += wtot[4 + i];
  }
  int pr = base_r + ir - run_rows, pa = base_a + ia - run_act;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < p.E) {
      start[e] = pr;
      if (cnt[e] > 0) {
        st_coh(p.active + pa, e);
        st_coh(p.row_off + pa, pr);
        ++pa;
      }
      pr += cnt[e];
    }
  }
  if (t == 255) {
    st_coh(p.row_off + base_a + ia, base_r + ir);
    st_coh(ctrl_at(p, CTRL_U), (unsigned)(base_a + ia));
  }
  __syncthreads();
  for (int s = t; s < nslots; s += 256) {
    const int pos = atomicAdd(&start[ids[s]], 1);
    st_coh(p.rows + pos, s);
  }
}

// Routing of rows [b0, b0+nr), run by the workgroup that completed their
// logits.  Top-k keys and candidates live in LDS (the x region): routing runs
// a handful of times per call, and holding its state in registers would set
// the register budget -- and so the occupancy -- of the whole kernel.
//   batch 1: each selected expert is published at once in its slot's counter
//            line (expert + 1), which is all a routed unit needs;
//   batch > 1: the workgroup that routes the last rows inverts the routing
//            into the expert-gathered schedule and publishes READY.
template <int TPL>
__device__ void route_rows(const LayerParams& p, WgState& st, Lds& L, int* lds_ints, int b0, int nr) {
  __builtin_amdgcn_s_setprio(3);  // on the critical path: issue ahead of streaming waves
  for (int r = 0; r < nr; ++r) {
    __syncthreads();  // the LDS region is reused
    const int b = b0 + r;
    const int myx = topk_row_wg<TPL>(p.logits + (size_t)b * p.E, p.E, p.k, reinterpret_cast<uint32_t*>(lds_ints),
                                     p.idx + (size_t)b * p.k, p.gate + (size_t)b * p.k);
    if (p.B == 1 && threadIdx.x < p.k) {
      __builtin_amdgcn_s_waitcnt(0);  // this lane's idx and gate stores are complete
      st_coh(ctrl_at(p, line_pub(p, threadIdx.x)), (unsigned)myx + 1u);
    }
  }
  st.x_cached = false;
  if (p.B > 1) {
    const unsigned old = wg_signal_add(ctrl_at(p, CTRL_ROUTING));
    if (threadIdx.x == 0) L.flag = (old == (unsigned)p.n_rb - 1);
    __syncthreads();
    if (L.flag) {
      build_schedule(p, lds_ints, L.wtot);
      wg_signal_add(ctrl_at(p, CTRL_READY));
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Router unit: experts 2u and 2u+1 for a block of rows.  Waves 0-1 take the
// two halves of expert 2u's row, waves 2-3 those of expert 2u+1, so every wave
// streams 7 KB at H 7168 in one pass of loads; the halves meet in LDS.  The
// last unit of a row block to finish routes its rows.
template <int RG, int TPL>
__device__ void router_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int u) {
  const int pe = u % p.n_rt_e, rb = u / p.n_rt_e;
  const int b0 = rb * RG, nr = min(RG, p.B - b0);
  load_rows(p, st, L, -1);
  stage_x(p, st, L, xs, false, b0, nr);
  const int w = threadIdx.x >> 6, half = w & 1;
  const int e = 2 * pe + (w >> 1);
  const int C = p.H / 8, gh = (C + 1) / 2;
  double acc[RG];
  router_dot<RG>(p.wr + (size_t)min(e, p.E - 1) * p.H, half * gh, half ? C : gh, xs, p.xstride, nr, acc);
  if (half && (threadIdx.x & 63) == 0) {
#pragma unroll
    for (int r = 0; r < RG; ++r) L.part[w][r] = acc[r];
  }
  __syncthreads();
  if (!half && e < p.E && (threadIdx.x & 63) == 0) {
    const double bb = p.bias ? (double)p.bias[e] : 0.0;
#pragma unroll
    for (int r = 0; r < RG; ++r)
      if (r < nr) st_coh(p.logits + (size_t)(b0 + r) * p.E + e, (float)(acc[r] + L.part[w + 1][r] + bb));
  }
  const unsigned old = wg_signal_add(ctrl_at(p, line_rb(p, rb)));
  if (threadIdx.x == 0) L.flag = (old == (unsigned)p.n_rt_e - 1);
  __syncthreads();
  if (L.flag) route_rows<TPL>(p, st, L, reinterpret_cast<int*>(xs), b0, nr);
}

// Batch 1: wait until slot a's expert is published (and, if fc1_target > 0,
// until that many FC1 units of the slot are done); both counters are read in
// one round trip per poll.  Sets the unit's row list to the slot itself.
__device__ __forceinline__ int wait_slot(const LayerParams& p, Lds& L, int a, unsigned fc1_target) {
  if (threadIdx.x == 0) {
    const unsigned* pub = ctrl_at(p, line_pub(p, a));
    const unsigned* done = ctrl_at(p, line_fc1(a));
    unsigned it = 0, nap = 1, v;
    for (;;) {
      v = ld_ctrl(pub);
      const unsigned c = fc1_target ? ld_ctrl(done) : 0u;
      if (v != 0u && c >= fc1_target) break;
      if (nap <= 1) __builtin_amdgcn_s_sleep(1);
      else if (nap <= 4) __builtin_amdgcn_s_sleep(4);
      else __builtin_amdgcn_s_sleep(16);
      nap = nap < 32 ? 2 * nap : 32;
      if (++it >= SPIN_LIMIT) {
        __hip_atomic_fetch_or(ctrl_at(p, CTRL_ERR), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = 1u;
        break;
      }
    }
    L.expert = (int)min(v - 1u, (unsigned)p.E - 1u);
    L.slot[0] = a;
    L.nrows = 1;
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return L.expert;
}

template <int RG, bool FULL>
__device__ void shared_fc1_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int t) {
  const int n_begin = t * NTS1, n_end = min(p.Is, n_begin + NTS1);
  const int half = (threadIdx.x & 63) >> 5;
  load_rows(p, st, L, -1);
  for (int g0 = 0; g0 < p.B; g0 += RG) {
    const int nr = min(RG, p.B - g0);
    Fc1Bf<RG, FULL> f;
    f.w = half ? p.su : p.sg;
    f.H = p.H;
    f.C8 = p.H / 8;
    f.nseg = (f.C8 + 32 * CPL1 - 1) / (32 * CPL1);
    f.n0 = n_begin + (threadIdx.x >> 6);
    f.xs = xs;
    f.xstride = p.xstride;
    f.nr = nr;
    for (int r = 0; r < RG; ++r) f.acc[r] = 0.0f;
    f.out = p.h_shared;
    f.out_ld = p.Is;
    f.row = L.slot + g0;
    const int nrows = f.n0 < n_end ? (n_end - f.n0 + 3) / 4 : 0;
    const int P = nrows * f.nseg;
    BfBuf<CPL1> ba, bb;
    prime_passes(f, P, ba, bb);
    stage_x(p, st, L, xs, false, g0, nr);
    drive_passes(f, P, ba, bb);
  }
  wg_signal_add(ctrl_at(p, CTRL_SH1));
}

template <int RG, bool FULL>
__device__ void routed_fc1_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int a, int t) {
  int expert;
  if (p.B == 1) {
    expert = wait_slot(p, L, a, 0u);
  } else {
    load_rows(p, st, L, a);
    expert = st.s_active[a];
  }
  const int nrows_unit = L.nrows;
  const uint8_t* blob = p.experts + (size_t)expert * p.blob_bytes;
  const int half = (threadIdx.x & 63) >> 5;
  const int n_begin = t * NT1, n_end = min(p.I, n_begin + NT1);
  for (int g0 = 0; g0 < nrows_unit; g0 += RG) {
    const int nr = min(RG, nrows_unit - g0);
    Fc1Mx<RG, FULL> f;
    f.codes = blob + p.off[half];
    f.scales = blob + p.off[3 + half];
    f.H = p.H;
    f.C = p.H / 32;
    f.nseg = (f.C + 32 * CPL1 - 1) / (32 * CPL1);
    f.n0 = n_begin + (threadIdx.x >> 6);
    f.xs = xs;
    f.xstride = p.xstride;
    f.nr = nr;
    for (int r = 0; r < RG; ++r) f.acc[r] = 0.0f;
    f.out = p.h_routed;
    f.out_ld = p.I;
    f.slot = L.slot + g0;
    const int nrows = f.n0 < n_end ? (n_end - f.n0 + 3) / 4 : 0;
    const int P = nrows * f.nseg;
    MxBuf<CPL1> ba, bb;
    prime_passes(f, P, ba, bb);
    stage_x(p, st, L, xs, true, g0, nr);
    drive_passes(f, P, ba, bb);
  }
  wg_signal_add(ctrl_at(p, line_fc1(a)));
}

// After a FC2 unit of tile t: count it; the last contribution folds the tile
// into the residual (fixed order: shared, then j = 0..k-1).
__device__ void fc2_ticket(const LayerParams& p, int U, Lds& L, int t) {
  const unsigned expected = (unsigned)((p.Is > 0 ? SUB2 : 0) + SUBR * U);
  const unsigned old = wg_signal_add(ctrl_at(p, line_tile(p, t)));
  if (threadIdx.x == 0) L.flag = (old == expected - 1);
  __syncthreads();
  if (!L.flag) return;
  const int m_begin = t * NT2, m_end = min(p.H, m_begin + NT2), w = m_end - m_begin;
  for (int i = threadIdx.x; i < p.B * w; i += 256) {
    const int b = i / w, m = m_begin + (i - b * w);
    float acc = p.residual[(size_t)b * p.H + m];
    if (p.Is > 0) acc += ld_coh(p.o_shared + (size_t)b * p.H + m);
    for (int j0 = 0; j0 < p.k; j0 += 8) {  // 16 coherent loads per batch
      float gv[8], ov[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = min(j0 + q, p.k - 1);
        gv[q] = ld_coh(p.gate + b * p.k + j);
        ov[q] = ld_coh(p.o_routed + ((size_t)b * p.k + j) * p.H + m);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q < p.k) acc = fmaf(gv[q], ov[q], acc);
    }
    p.residual[(size_t)b * p.H + m] = acc;
  }
}

template <int RG, bool FULL>
__device__ void shared_fc2_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* hs, int v) {
  const int t = v / SUB2, sub = v - t * SUB2;
  const int m_begin = t * NT2 + sub * NTS2, m_end = min(p.H, m_begin + NTS2);
  load_rows(p, st, L, -1);
  for (int g0 = 0; g0 < p.B; g0 += RG) {
    const int nr = min(RG, p.B - g0);
    Fc2Bf<RG, FULL> f;
    f.w = p.sd;
    f.K = p.Is;
    f.C8 = p.Is / 8;
    f.nseg = (f.C8 + 8 * CPL2 - 1) / (8 * CPL2);
    f.m_begin = m_begin;
    f.m_end = m_end;
    f.hs = hs;
    f.hstride = p.hstride;
    f.nr = nr;
    for (int r = 0; r < RG; ++r) f.acc[r] = 0.0f;
    f.out = p.o_shared;
    f.out_ld = p.H;
    f.row = L.slot + g0;
    const int groups = (m_end - m_begin + 31) / 32;  // 32 rows per block pass (4 waves x 8)
    const int P = m_begin < m_end ? groups * f.nseg : 0;
    BfBuf<CPL2> ba, bb;
    prime_passes(f, P, ba, bb);  // the weights do not depend on FC1
    if (g0 == 0) wg_wait_geq(p, ctrl_at(p, CTRL_SH1), (unsigned)p.n_s1);
    stage_h(p, hs, p.h_shared, L, g0, nr, p.Is);
    drive_passes(f, P, ba, bb);
  }
  fc2_ticket(p, st.U, L, t);
}

template <int RG, bool FULL>
__device__ void routed_fc2_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* hs, int a, int v) {
  const int t = v / SUBR, sub = v - t * SUBR;
  const int m_begin = t * NT2 + sub * NTR2, m_end = min(p.H, m_begin + NTR2);
  int expert;
  if (p.B == 1) {
    expert = wait_slot(p, L, a, (unsigned)p.T1);
  } else {
    load_rows(p, st, L, a);
    expert = st.s_active[a];
  }
  const int nrows_unit = L.nrows;
  const uint8_t* blob = p.experts + (size_t)expert * p.blob_bytes;
  for (int g0 = 0; g0 < nrows_unit; g0 += RG) {
    const int nr = min(RG, nrows_unit - g0);
    Fc2Mx<RG, FULL> f;
    f.codes = blob + p.off[2];
    f.scales = blob + p.off[5];
    f.K = p.I;
    f.C = p.I / 32;
    f.nseg = (f.C + 8 * CPL2 - 1) / (8 * CPL2);
    f.m_begin = m_begin;
    f.m_end = m_end;
    f.hs = hs;
    f.hstride = p.hstride;
    f.nr = nr;
    for (int r = 0; r < RG; ++r) f.acc[r] = 0.0f;
    f.out = p.o_routed;
    f.out_ld = p.H;
    f.slot = L.slot + g0;
    const int groups = (m_end - m_begin + 31) / 32;
    const int P = m_begin < m_end ? groups * f.nseg : 0;
    MxBuf<CPL2> ba, bb;
    prime_passes(f, P, ba, bb);  // the weights do not depend on FC1
    if (g0 == 0 && p.B > 1) wg_wait_geq(p, ctrl_at(p, line_fc1(a)), (unsigned)p.T1);
    stage_h(p, hs, p.h_routed, L, g0, nr, p.I);
    drive_passes(f, P, ba, bb);
  }
  fc2_ticket(p, st.U, L, t);
}

// Next unit of the in-order queue (the first p.n_static units are handed out
// by workgroup index; they never wait).
__device__ __forceinline__ int pop_unit(const LayerParams& p, Lds& L) {
  __syncthreads();
  if (threadIdx.x == 0)
    L.next = p.n_static +
             (int)__hip_atomic_fetch_add(ctrl_at(p, CTRL_HEAD), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return L.next;
}

// ---- the kernel ------------------------------------------------------------------

// FULL: the layer's shape makes every weight-stream segment and FC2 row group
// complete (H % 7168 == 0, I % 1536 == 0, Is % 384 == 0), so the streams need
// no clamping or masking.
template <int RG, bool FULL, int TPL>
__global__ __launch_bounds__(256, RG == 1 ? 3 : 2) void k_moe_layer(LayerParams p) {
  extern __shared__ u32x4 lds_raw[];
  u32x4* xs = lds_raw;
  u32x4* hs = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(lds_raw) + p.lds_h_off);
  __shared__ Lds L;
  WgState st{false, false, 0, nullptr, nullptr, nullptr};
  // First units (router and shared FC1 -- they wait on nothing) by workgroup
  // index, so the launch ramp does not queue on the head counter.
  int u = (int)blockIdx.x < p.n_static ? (int)blockIdx.x : pop_unit(p, L);
  for (;;) {
    int rel = u;
    if (rel < p.n_rt) {
      router_unit<RG, TPL>(p, st, L, xs, rel);
    } else if ((rel -= p.n_rt) < p.n_s1) {
      shared_fc1_unit<RG, FULL>(p, st, L, xs, rel);
    } else {
      rel -= p.n_s1;
      if (!st.route_seen) {
        if (p.B == 1) {
          st.U = p.k;  // one row: k distinct experts, one per slot
        } else {
          wg_wait_geq(p, ctrl_at(p, CTRL_READY), 1u);
          st.U = (int)ld_ctrl(ctrl_at(p, CTRL_U));
          cache_schedule(p, st, reinterpret_cast<int*>(reinterpret_cast<char*>(lds_raw) + p.lds_sched_off));
        }
        st.route_seen = true;
      }
      const int U = st.U;
      if (rel < U * p.T1) {
        routed_fc1_unit<RG, FULL>(p, st, L, xs, rel / p.T1, rel % p.T1);
      } else if ((rel -= U * p.T1) < p.n_s2) {
        shared_fc2_unit<RG, FULL>(p, st, L, hs, rel);
      } else if ((rel -= p.n_s2) < U * p.T2 * SUBR) {
        routed_fc2_unit<RG, FULL>(p, st, L, hs, rel / (p.T2 * SUBR), rel % (p.T2 * SUBR));
      } else {
        break;
      }
    }
    u = pop_unit(p, L);
  }
  // Exit: the last workgroup out clears the control block for the next call
  // (all other workgroups have made their final control-block access).
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctrl_at(p, CTRL_EXIT), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L.flag = (old == gridDim.x - 1);
  }
  __syncthreads();
  if (L.flag) {
    for (int i = threadIdx.x; i < p.ctrl_words / CTRL_STRIDE; i += 256)
      if (i != CTRL_ERR) st_coh(ctrl_at(p, i), 0u);
  }
}

// ---- host side -------------------------------------------------------------------

struct LaunchShape {
  int rg;
  bool full;
  int xstride, hstride;
  size_t lds;
  int lds_h_off, lds_sched_off;
};

static LaunchShape launch_shape(int H, int I, int E, int k, int Is, int B) {
  LaunchShape s;
  s.rg = (B == 1) ? 1 : 4;
  s.full = (H % (32 * 32 * CPL1) == 0) && (H % (8 * 32 * CPL1) == 0) && (I % (32 * 8 * CPL2) == 0) &&
           (Is % (8 * 8 * CPL2) == 0) && (H % NT2 == 0);
  s.xstride = ((H / 8 + 7) / 8) * 8;
  int K2 = I > Is ? I : Is;
  s.hstride = ((K2 / 4 + 7) / 8) * 8;
  size_t x_bytes = (size_t)s.rg * s.xstride * 16;
  // routing reuses this region: top-k candidates (640 words), then the
  // schedule's counts (2E) and slot ids (B*k)
  size_t keys_bytes = 640 * 4, cnt_bytes = (size_t)(2 * E + B * k) * 4;
  size_t sched_bytes = keys_bytes > cnt_bytes ? keys_bytes : cnt_bytes;
  size_t xr = align256(x_bytes > sched_bytes ? x_bytes : sched_bytes);
  s.lds_h_off = (int)xr;
  size_t hr = align256((size_t)s.rg * s.hstride * 16);
  s.lds_sched_off = (int)(xr + hr);
  const size_t slots = (size_t)B * k, umax = slots < (size_t)E ? slots : (size_t)E;
  s.lds = xr + hr + align256(4 * (2 * umax + 1 + slots));
  return s;
}

template <int RG, bool FULL, int TPL>
static hipError_t launch_t(LayerParams p, size_t lds, hipStream_t s) {
  auto kern = k_moe_layer<RG, FULL, TPL>;
  static thread_local int cached[2] = {-1, -1};  // (lds bytes, blocks per CU)
  int per_cu = 0;
  if (cached[0] == (int)lds) {
    per_cu = cached[1];
  } else {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) per_cu = 1;
    cached[0] = (int)lds;
    cached[1] = per_cu;
  }
  const int grid = num_cus() * per_cu;
  p.n_static = std::min(grid, p.n_rt + p.n_s1);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_layer(const LayerArgs& a, const float* bias, const uint16_t* wr, int32_t* idx, hipStream_t s) {
  LayerParams p;
  p.H = a.H;
  p.I = a.I;
  p.E = a.E;
  p.k = a.k;
  p.Is = a.Is;
  p.B = a.B;
  p.x = a.x;
  p.wr = wr;
  p.bias = bias;
  p.sg = a.sg;
  p.su = a.su;
  p.sd = a.sd;
  p.experts = a.experts;
  p.blob_bytes = a.blob.bytes;
  for (int i = 0; i < 6; ++i) p.off[i] = a.blob.off[i];
  p.residual = a.residual;
  p.idx = idx;
  p.gate = const_cast<float*>(a.gate);
  p.logits = a.ws.logits;
  p.active = a.ws.sched.active;
  p.row_off = a.ws.sched.row_off;
  p.rows = a.ws.sched.rows;
  p.h_shared = a.ws.h_shared;
  p.h_routed = a.ws.h_routed;
  p.o_shared = a.ws.o_shared;
  p.o_routed = a.ws.o_routed;
  p.ctrl = a.ws.ctrl;
  p.umax = a.ws.umax;
  p.ctrl_words = a.ws.ctrl_words;
  const LaunchShape sh = launch_shape(a.H, a.I, a.E, a.k, a.Is, a.B);
  p.n_rt_e = (a.E + 1) / 2;
  p.xstride = sh.xstride;
  p.hstride = sh.hstride;
  p.n_rt = p.n_rt_e * ((a.B + sh.rg - 1) / sh.rg);
  p.n_rb = (a.B + sh.rg - 1) / sh.rg;
  p.n_s1 = a.Is > 0 ? (a.Is + NTS1 - 1) / NTS1 : 0;
  p.T1 = (a.I + NT1 - 1) / NT1;
  p.T2 = (a.H + NT2 - 1) / NT2;
  p.n_s2 = a.Is > 0 ? p.T2 * SUB2 : 0;
  p.lds_h_off = sh.lds_h_off;
  p.lds_sched_off = sh.lds_sched_off;
// top-k keys per lane in the first selection phase: E <= 1024 -> 4, else 16
  if (a.E <= 1024) {
    if (sh.rg == 1) return sh.full ? launch_t<1, true, 4>(p, sh.lds, s) : launch_t<1, false, 4>(p, sh.lds, s);
    return sh.full ? launch_t<4, true, 4>(p, sh.lds, s) : launch_t<4, false, 4>(p, sh.lds, s);
  }
  if (sh.rg == 1) return sh.full ? launch_t<1, true, 16>(p, sh.lds, s) : launch_t<1, false, 16>(p, sh.lds, s);
  return sh.full ? launch_t<4, true, 16>(p, sh.lds, s) : launch_t<4, false, 16>(p, sh.lds, s);
}

int layer_tiles_fc2(int H) { return (H + NT2 - 1) / NT2; }

}  // namespace moe
