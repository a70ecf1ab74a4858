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
//   * workgroups take "units" from an in-order device queue (one atomic,
//     issued one unit ahead so its latency hides behind the current unit);
//   * unit kinds, in queue order:
//       router GEMV (2 experts x a block of rows)          -> logits
//       routing (top-k + gates of one row)                 -> idx, gate
//       schedule (batch > 1: expert-gathered row lists)    -> schedule
//       shared-expert FC1+SwiGLU (tile of Is rows)         -> shared h
//       routed FC1+SwiGLU (expert, 16 rows of I)           -> routed h
//       shared-expert FC2 (tile of H rows)                 -> shared output
//       routed FC2 (expert, 128 rows of H)                 -> routed outputs
//       combine (row, 256 rows of H): residual += shared + sum_j gate_j o_j
//                (fixed j order, so the result is deterministic);
//   * a unit only ever waits on data written by units earlier in the queue,
//     so the smallest unfinished unit can always run: no residency
//     assumption, no deadlock; every wait is bounded and sets a sticky error
//     word instead of hanging;
//   * data handed between workgroups travels as 8-byte (value, tag) pairs
//     written and read with single coherent accesses (the tag identifies the
//     call), and the consumer polls the data itself.  A producer therefore
//     never drains its stores or bumps a completion counter: under a
//     saturated HBM each such handshake is a multi-microsecond round trip,
//     and there would be several per unit.  Coherent accesses are performed
//     at the device coherence point, so no L2 write-back or invalidate (which
//     serialise device-wide) is ever issued;
//   * the router and the shared expert need no routing, so they stream while
//     top-k runs, hiding its latency; routed FC2 of one expert overlaps FC1
//     of the next.
//
// Weight streams are branch-free: every lane issues all of a pass's 16-byte
// loads (clamped to the row), and chunks past the row end are masked to zero
// in the math, so the compiler keeps a whole pass (and the next pass) in
// flight instead of waiting load by load.
//
// The control block at the start of the workspace is zeroed once by
// moe_workspace_init; the last workgroup of every call resets the queue and
// advances the call epoch (whose value + 1 is the next call's tag).
#include <atomic>
#include "internal.h"
#include "moe_device.h"

#include <algorithm>
#include <type_traits>

namespace moe {

// The thread index through an empty asm, for the batch > 1 code: values
// derived from it cannot be hoisted out of the unit loop, where they would
// hold registers across every other unit (the batch > 1 kernel is register
// bound); each unit recomputes them.
__device__ __forceinline__ int tidx() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}


constexpr int NT1 = 16;   // routed FC1 rows (of I) per unit: one packed row group, 16 x 2 x 3.8 KB at H 7168
constexpr int NTS1 = 4;   // shared FC1 rows (of Is) per unit: 4 x 2 x 14 KB of bf16
constexpr int NT2 = 256;  // combine tile (rows of H)
constexpr int NTS2 = 32;  // shared FC2 rows per unit
constexpr int NTR2 = 128; // routed FC2 rows per unit: 8 packed row groups
constexpr int CPL1 = 7;   // FC1: 16-byte chunks per lane per pass (half-wave rows)
constexpr int CPL2 = 6;   // FC2: 16-byte chunks per lane per pass (8 lanes per row)
constexpr int MAX_ROWS = MOE_MAX_BATCH;    // activation rows one expert can have
constexpr unsigned SPIN_LIMIT = 1u << 20;  // ~1 s of polls (at ~1 us each) before a wait gives up
constexpr int RT_F64_MIN_BATCH = 16;       // batches above this run the router on the fp64 matrix cores

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
  uint64_t* logits_p;
  uint64_t* idx_p;
  uint64_t* gate_p;
  int* active;
  int* row_off;
  int* rows;
  int* cg_off;
  uint64_t* hflag;
  int hflag_tiles;
  uint64_t* hs_p;
  uint64_t* hr_p;
  uint64_t* os_p;
  uint64_t* or_p;
  unsigned* ctrl;
  int umax;
  int rt_f64;    // batch > 16: router units on the matrix cores (16 experts x 16 rows)
  int n_rt_e;    // router units per row block (4 experts a unit; 16 on the matrix cores)
  int n_rb;      // router row blocks
  int n_rt;      // router units = n_rt_e * n_rb
  int n_ro;      // routing units (one per row)
  int n_sch;     // schedule units (batch > 1: 1)
  int n_s1;      // shared FC1 units
  int T1;        // routed FC1 tiles per expert
  int n_s2;      // shared FC2 units
  int n_r2;      // routed FC2 units per expert
  int n_tile;    // combine tiles over H
  int mf_t1;     // batch > 1: routed FC1 units per column group (64 rows of I each)
  int mf_t1s;    // batch > 1: shared FC1 units per column group (16 rows of Is each)
  int mf_t2;     // batch > 1: routed FC2 units per column group (MF_NT2 rows of H each)
  int mf_t2s;    // batch > 1: shared FC2 units per column group (128 rows of H each)
  int mf_cgs;    // batch > 1: shared-expert column groups (16 batch rows each)
  int n_front;   // units before the routed ones (router .. shared FC1)
  int n_static;  // units 0 .. n_static-1 go to workgroups 0 .. n_static-1
  int n_total;   // batch 1: units in the queue (k experts); 0 for the matrix-core kernel
  int nq;        // work queues after them: 2 (1 for grids under 16 workgroups)
  int xstride;        // LDS x row stride, 16-byte granules (multiple of 8)
  int hstride;        // LDS h row stride, 16-byte granules (multiple of 8)
  int lds_h_off;      // byte offset of the h staging region in dynamic LDS
  int lds_sched_off;  // byte offset of the schedule copy in dynamic LDS
};

__device__ __forceinline__ void set_error(const LayerParams& p) {
  __hip_atomic_fetch_or(p.ctrl + CTRL_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- per-workgroup state ------------------------------------------------------

struct Lds {  // static LDS of the kernel
  int next;        // next unit index (first claim)
  int nxt[2];      // next unit index, alternating between iterations of the unit loop
  int U;           // distinct experts (once known)
  int sched_ok;    // batch > 1: the schedule's ready word arrived
  uint64_t pre;    // batch 1: (unit-loop iteration + 1, next unit) posted mid-unit by thread 0
  int wtot[12];    // scan scratch
  int nrows;       // rows of the current unit
  float gates[MOE_MAX_TOPK];  // combine: gates of the current row
  alignas(16) float red[4][4][16][2];  // routed FC1: per-wave partial sums [wave][row][tile row][gate/up]; batch > 1 router: [4][32] doubles
  int slot[MAX_ROWS];  // slot ids (routed) or batch rows (shared) of the current unit
};

struct WgState {
  bool x_cached;    // batch 1: x row 0 already in LDS
  bool route_seen;  // this workgroup holds the schedule in LDS
  int U;
  uint32_t tag;
  const int* s_active;   // LDS copy of the schedule (valid once route_seen)
  const int* s_row_off;
  const int* s_rows;
  const int* s_cg_off;
  bool exited = false;     // batch 1, thread 0: this workgroup has counted itself out early
  unsigned exit_old = 0u;  // ... and the exit count it saw
};

// Bounded poll of one control word until it has `tag` in its high half
// (thread 0 only).  Returns the low half, or -1 if the wait gave up (the
// sticky error word is then set).
__device__ __forceinline__ int poll_ready(const LayerParams& p, uint32_t tag) {
  const uint64_t* a = reinterpret_cast<const uint64_t*>(p.ctrl + CTRL_READY);
  for (unsigned it = 0;; ++it) {
    const uint64_t v = ld_pair(a);
    if (pair_has(v, tag)) return (int)min((uint32_t)v, 0x7FFFFFFFu);
    if (it >= SPIN_LIMIT || ((it & 255) == 255 && ld_coh(p.ctrl + CTRL_ERR) != 0u)) {
      set_error(p);
      return -1;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The schedule into this workgroup's LDS.  Batch 1: one row, so slot j is
// "active expert" j with row list {j}; its expert comes from the routing
// pairs.  Batch > 1: wait for the schedule unit's ready word, then copy the
// published schedule (one batch of coherent loads).
template <bool OPQ>
__device__ __forceinline__ void cache_schedule(const LayerParams& p, WgState& st, Lds& L, int* sc) {
  const int TID_ = OPQ ? tidx() : (int)threadIdx.x;
  int* a = sc;
  int* ro = sc + p.umax;
  int* rw = ro + p.umax + 1;
  int* cgo = rw + p.B * p.k;
  if (!OPQ) {  // the batch-1 kernel (the matrix-core kernel builds a schedule at every batch)
    if (TID_ < p.k) {
      uint64_t v[1];
      const int j = TID_;
      if (!poll_pairs<1>(p.idx_p, 1, [&](int) { return j; }, st.tag, v, SPIN_LIMIT, p.ctrl + CTRL_ERR)) set_error(p);
      a[j] = (int)min((uint32_t)v[0], (uint32_t)p.E - 1u);
      ro[j] = j;
      rw[j] = j;
    }
    if (TID_ == 0) {
      ro[p.k] = p.k;
      L.U = p.k;
    }
  } else {
    if (TID_ == 0) {
      const int u = poll_ready(p, st.tag);
      L.sched_ok = u >= 0;
      L.U = u < 0 ? 0 : min(u, p.umax);
    }
    __syncthreads();
    const int U = L.U, nslots = p.B * p.k;
    if (!L.sched_ok) {
      // The schedule never arrived (the call's outputs are invalid and the
      // status word says so): no active experts, so no routed unit reads an
      // expert, a row list or a flag that this call did not write.
      if (TID_ == 0) {
        ro[0] = 0;
        cgo[0] = 0;
      }
    } else {
      // Published before the ready word, so consistent; the clamps only keep
      // every later index inside its buffer whatever the memory holds.
      const int total = U + (U + 1) + nslots + (U + 1);
      for (int base = TID_; base < total; base += 256 * 8) {
        int v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int i = min(base + 256 * t, total - 1);
          v[t] = i < U ? ld_coh(p.active + i)
                       : (i < 2 * U + 1 ? ld_coh(p.row_off + (i - U))
                                        : (i < 2 * U + 1 + nslots ? ld_coh(p.rows + (i - 2 * U - 1))
                                                                  : ld_coh(p.cg_off + (i - 2 * U - 1 - nslots))));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int i = base + 256 * t;
          if (i < total) {
            if (i < U) a[i] = min(max(v[t], 0), p.E - 1);
            else if (i < 2 * U + 1) ro[i - U] = min(max(v[t], 0), nslots);
            else if (i < 2 * U + 1 + nslots) rw[i - 2 * U - 1] = min(max(v[t], 0), nslots - 1);
            else cgo[i - 2 * U - 1 - nslots] = min(max(v[t], 0), 4 * U);
          }
        }
      }
    }
  }
  __syncthreads();
  st.U = L.U;
  st.s_active = a;
  st.s_row_off = ro;
  st.s_rows = rw;
  st.s_cg_off = cgo;
  st.route_seen = true;
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
    const int b = p.B == 1 ? 0 : (routed ? L.slot[g0 + r] / p.k : L.slot[g0 + r]);
    xs[r * p.xstride + swz(c)] = reinterpret_cast<const u32x4*>(p.x + (size_t)b * p.H)[c];
  }
  __syncthreads();
  st.x_cached = (p.B == 1);
}

// h rows (tagged pairs written earlier in this launch) of rows [g0, g0+nr),
// row r taken from src[slot(r)], polled until every pair carries this call's
// tag, into LDS as fp32 (swizzled 16-byte granules, row stride p.hstride).
// 8 pairs per thread per batch.
__device__ __forceinline__ void stage_h(const LayerParams& p, const WgState& st, u32x4* hs, const uint64_t* src,
                                        const Lds& L, int g0, int nr, int K) {
  __syncthreads();
  const int total = nr * K;
  float* hf = reinterpret_cast<float*>(hs);
  bool ok = true;
  for (int base = threadIdx.x; base < total; base += 256 * 8) {
    uint64_t v[8];
    const int n = min(8, (total - base + 255) / 256);
    ok &= poll_pairs_cached<8>(src, n, [&](int t) {
      const int i = base + 256 * t;
      const int r = i / K, e = i - r * K;
      return (size_t)L.slot[g0 + r] * K + e;
    }, st.tag, v, SPIN_LIMIT, p.ctrl + CTRL_ERR);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = base + 256 * t;
      if (i < total) {
        const int r = i / K, e = i - r * K;
        hf[(r * p.hstride + swz(e >> 2)) * 4 + (e & 3)] = pair_f32(v[t]);
      }
    }
  }
  if (!ok) set_error(p);
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
struct Fc1Bf {
  const uint16_t* w;  // this lane's matrix (gate or up), row 0
  int H, C8, nseg, n0;
  const u32x4* xs;  // LDS x rows (swizzled)
  int xstride;
  int nr;
  float acc[RG];
  uint64_t* out;  // shared h pairs, indexed by batch row
  uint32_t tag;
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
          if (lane == 0) st_pair_f32(out + (size_t)row[r] * out_ld + n, silu_f(g) * u, tag);
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
  uint64_t* out;  // shared output pairs, indexed by batch row
  uint32_t tag;
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
          if (l == 0 && (FULL || m < m_end)) st_pair_f32(out + (size_t)row[r] * out_ld + m, v, tag);
        }
        acc[r] = 0.0f;
      }
    }
  }
};

// ---- packed-tile streams of the routed experts ---------------------------------
//
// An expert's MXFP4 matrices are packed (moe_pack_experts) into tiles of 16
// rows x 16 blocks of 32 elements: codes [SC][16 rows] x 16 B, then scales
// [16 rows][SC] B.  Lane l = 16 q + r of a wave reads, from 1 KB slab kb of a
// tile, block 4 kb + q of row r: each load instruction is one contiguous KB.
// A lane therefore accumulates row r over blocks q, q+4, q+8, ...; the four
// lanes r, r+16, r+32, r+48 are summed at the end of the row.

__host__ __device__ inline size_t tile_off(int g, int s, int C) {
  return (size_t)g * 16 * C * 17 + (size_t)s * 16 * 272;
}

// 8 FP4 elements (one dword) -> 8 bf16, exact (E2M1 x 2^k fits bf16), in
// element order: the A or B operand of one 16x16x32 bf16 MFMA lane.
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w, float s) {
  bf16x2 t[4];
  dq4_bf16(w, s, t);
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, t[0]), __builtin_bit_cast(uint32_t, t[1]),
                                          __builtin_bit_cast(uint32_t, t[2]), __builtin_bit_cast(uint32_t, t[3])});
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct TileBuf1 {  // one FC1 segment: gate and up codes (4 slabs each) and scale vectors
  u32x4 gq[4], uq[4];
  u32x4 gs, us;
};

struct TileBuf2 {  // one FC2 segment of two row groups
  u32x4 q[2][4];
  u32x4 s[2];
};

// A lane (16 q + r) decodes blocks 4 kb + q (kb = 0..3) of row r of a tile,
// and holds their four scale bytes as one dword, byte kb.  A full tile
// stores each row's scales so that this dword is one aligned load (block
// 4 kb + q at byte 4 q + kb of the row); a partial tile's are gathered.
__device__ __forceinline__ uint32_t tile_scale(uint32_t v, int kb) { return (v >> (8 * kb)) & 0xFFu; }

// Byte offset, in a tile's scale area, of block c of row r (SC blocks).
__device__ __forceinline__ int scale_pos(int SC, int r, int c) {
  return SC == 16 ? r * 16 + (c & 3) * 4 + (c >> 2) : r * SC + c;
}

__device__ __forceinline__ uint32_t ld_weight4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// OPQ: take the thread index through tidx() (the batch > 1 units).
template <bool FULL, bool OPQ = false>
__device__ __forceinline__ void load_tile(const uint8_t* t, int SC, u32x4 (&cq)[4], uint32_t& sv) {
  const int l = (OPQ ? tidx() : (int)threadIdx.x) & 63, r = l & 15, q = l >> 4;
  if (FULL) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cq[kb] = ld_weight16(t + kb * 1024 + l * 16);
    sv = ld_weight4(t + 4096 + r * 16 + q * 4);
  } else {
    uint32_t b = 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int c = min(4 * kb + q, SC - 1);
      cq[kb] = ld_weight16(t + c * 256 + r * 16);
      b |= (uint32_t)t[SC * 256 + scale_pos(SC, r, c)] << (8 * kb);
    }
    sv = b;
  }
}

// One 1 KB slab kb of a tile's codes (lane 16 q + r: block 4 kb + q of row
// r), and the tile's scale dword, as load_tile reads them.
template <bool FULL>
__device__ __forceinline__ u32x4 load_slab(const uint8_t* t, int SC, int kb) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  if (FULL) return ld_weight16(t + kb * 1024 + l * 16);
  return ld_weight16(t + min(4 * kb + q, SC - 1) * 256 + r * 16);
}

// The batch-1 streams hold a row's 16 scale bytes as one vector (FULL: as
// stored; partial: the lane's 4 gathered bytes in the first dword) and take
// the lane's dword out of it when a pass's math starts, where the data is
// needed anyway.
template <bool FULL>
__device__ __forceinline__ uint32_t scale_dword16(const u32x4& v, int q) {
  if (!FULL) return v[0];
  return q < 2 ? (q == 0 ? v[0] : v[1]) : (q == 2 ? v[2] : v[3]);
}

template <bool FULL>
__device__ __forceinline__ void load_tile16(const uint8_t* t, int SC, u32x4 (&cq)[4], u32x4& sv) {
  const int l = threadIdx.x & 63, r = l & 15;
  if (FULL) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cq[kb] = ld_weight16(t + kb * 1024 + l * 16);
    sv = ld_weight16(t + 4096 + r * 16);
  } else {
    uint32_t b;
    load_tile<false>(t, SC, cq, b);
    sv = u32x4{b, 0u, 0u, 0u};
  }
}

template <bool FULL>
__device__ __forceinline__ u32x4 load_scales16(const uint8_t* t, int SC);

template <bool FULL>
__device__ __forceinline__ uint32_t load_scales(const uint8_t* t, int SC) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  if (FULL) return ld_weight4(t + 4096 + r * 16 + q * 4);
  uint32_t b = 0;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) b |= (uint32_t)t[SC * 256 + scale_pos(SC, r, min(4 * kb + q, SC - 1))] << (8 * kb);
  return b;
}

template <bool FULL>
__device__ __forceinline__ u32x4 load_scales16(const uint8_t* t, int SC) {
  const int r = threadIdx.x & 15;
  if (FULL) return ld_weight16(t + 4096 + r * 16);
  return u32x4{load_scales<false>(t, SC), 0u, 0u, 0u};
}

// An address offset (always 0) that the compiler must compute after `dep`:
// it ties a refill load to the last use of the registers it overwrites, so the
// load is neither hoisted into fresh registers nor delayed.
__device__ __forceinline__ int after_u(int idx, uint32_t dep) {
  asm volatile("" : "+v"(idx) : "v"(dep));
  return idx;
}

// Output rows of a matrix-core product, regrouped for wide stores.  After a
// 16x16 MFMA, lane 16 q + r holds rows 4 q .. 4 q + 3 of column r (v[0..3]).
// regroup_rows gives lane 16 q + r rows 8 h + 2 q and 8 h + 2 q + 1 of column
// r (h = 0, 1: two calls), so that one 16-byte store per lane writes rows
// 8 h .. 8 h + 7 of a column as 64 contiguous bytes across lanes r, 16 + r,
// 32 + r, 48 + r (4 x 8-byte stores at a 32-byte stride wrote every line of
// the outputs four times over).  Every lane of the wave must take part.
__device__ __forceinline__ void regroup_rows(const f32x4& v, int h, float& a, float& b) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  const int src = 16 * (2 * h + (q >> 1)) + (lane & 15);
  const float x0 = __shfl(v[0], src), x1 = __shfl(v[1], src), x2 = __shfl(v[2], src), x3 = __shfl(v[3], src);
  a = (q & 1) ? x2 : x0;
  b = (q & 1) ? x3 : x1;
}

// 16-byte stores with the coherence of st_coh's 8-byte atomic stores
// (written through to the device-coherent level), as buffer stores: `base`
// is wave-uniform (a workspace region), `off` the lane's byte offset in it
// (16-byte aligned, below 2 GiB).  A buffer store lets the compiler see the
// store (and keep its registers until the hardware has read them), which a
// store written in inline asm would not.
__device__ __forceinline__ void st16_coh(const void* base, uint32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0x10);  // 0x10: sc1
}

// Two consecutive tagged pairs, pairs idx and idx + 1 (idx even) of `base`, in
// one 16-byte store.  A reader polls each 8-byte pair on its own, so it needs
// no more than each aligned 8-byte half to be written whole.
__device__ __forceinline__ void st_pair2_f32(const uint64_t* base, size_t idx, float a, float b, uint32_t tag) {
  st16_coh(base, (uint32_t)(idx * 8), u32x4{__float_as_uint(a), tag, __float_as_uint(b), tag});
}

// Four fp32 values, elements idx .. idx + 3 (idx a multiple of 4) of `base`, in
// one 16-byte store; readers take them only after a flag that the writer sets
// once all its stores have completed.
__device__ __forceinline__ void st_f32x4_coh(const float* base, size_t idx, const float (&v)[4]) {
  st16_coh(base, (uint32_t)(idx * 4),
           u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
}

// The LDS reads of a pass's activations are software-pipelined one step
// ahead of the math, and each read's address is tied (through an empty asm)
// to the accumulator of the step before, so the compiler cannot hoist every
// read of the pass to its top: that would hold 16-32 granules (64-128
// VGPRs) live and push the kernel into spilling.
__device__ __forceinline__ int after(int idx, float dep) {
  asm volatile("" : "+v"(idx) : "v"(dep));
  return idx;
}

// FC1 + SwiGLU of one 16-row group g of an expert against the x row (LDS),
// on the matrix cores.  Wave w takes segments w, w+4, ...; partial sums meet
// in LDS afterwards.  Step i = 4 kb + d of a segment is one 16x16x32 MFMA per
// tile: lane l = 16 q + r supplies row r's elements 8 d .. 8 d + 7 of block
// 4 kb + q (dword d of its slab kb, decoded to bf16) as the A operand and the
// matching 8 x values as the B operand, so all 16 columns of the product are
// the same dot products and lane l ends with rows 4 (l / 16) .. + 3.  This
// takes the dot products off the vector ALU, which otherwise bounds the
// stream (the FP4 decode stays there: 4 conversions per dword).
template <int RG, bool FULL>
struct Fc1Tile {
  static_assert(RG == 1, "the batch-1 streams take one row");
  const uint8_t* blob;
  int C1, g, w;
  const u32x4* xs;
  int xstride;
  f32x4 ag, au;
  __device__ int seg(int p) const { return w + 4 * p; }
  __device__ void load(TileBuf1& b, int p) {
    const int s = seg(p);
    const int SC = FULL ? 16 : min(16, C1 - 16 * s);
    // issued only after the math of the pass before (its accumulator), so the
    // compiler cannot start this pass's loads early and hold a third buffer
    const uint8_t* gt = blob + 2 * tile_off(g, s, C1) + after(after(0, ag[0]), au[0]);
    load_tile16<FULL>(gt, SC, b.gq, b.gs);
    load_tile16<FULL>(gt + SC * 272, SC, b.uq, b.us);
  }
  // x granule of step i = 4 kb + d (block 4 kb + q of the segment)
  __device__ int xg(int s, int SC, int i) const {
    const int q = (threadIdx.x & 63) >> 4, c = 4 * (i >> 2) + q;
    return swz((16 * s + (FULL ? c : min(c, SC - 1))) * 4 + (i & 3));
  }
  // The x granules are read one slab ahead; with `refill`, slab kb of both
  // tiles is refilled from the gate/up tile pair at gt2 (SC2 blocks: a pass
  // two ahead, of this unit or of the next) as soon as its last dword is
  // decoded, the scale vectors after the last slab.
  __device__ void math(TileBuf1& b, int p, bool refill, const uint8_t* gt2, int SC2) {
    const int s = seg(p);
    const int q = (threadIdx.x & 63) >> 4;
    const int SC = FULL ? 16 : min(16, C1 - 16 * s);
    u32x4 xv[4], xn[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) xv[d] = xs[xg(s, SC, d)];
    const uint32_t gsd = scale_dword16<FULL>(b.gs, q), usd = scale_dword16<FULL>(b.us, q);
    int o = 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb < 3) {
#pragma unroll
        for (int d = 0; d < 4; ++d) xn[d] = xs[after(xg(s, SC, 4 * kb + 4 + d), ag[0])];
      }
      const int c = 4 * kb + q;
      const uint32_t msk = (FULL || c < SC) ? 0xFFFFFFFFu : 0u;
      const float sg = e8m0_scale(tile_scale(gsd, kb));
      const float su = e8m0_scale(tile_scale(usd, kb));
      bf16x8 wg, wu;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        wg = fp4x8_bf16(b.gq[kb][d] & msk, sg);
        wu = fp4x8_bf16(b.uq[kb][d] & msk, su);
        const bf16x8 x8 = __builtin_bit_cast(bf16x8, xv[d]);
        ag = mfma_bf16(wg, x8, ag);
        au = mfma_bf16(wu, x8, au);
      }
      if (refill) {
        o = after_u(after_u(o, __builtin_bit_cast(u32x4, wg)[3]), __builtin_bit_cast(u32x4, wu)[3]);
        b.gq[kb] = load_slab<FULL>(gt2 + o, SC2, kb);
        b.uq[kb] = load_slab<FULL>(gt2 + SC2 * 272 + o, SC2, kb);
      }
      if (kb < 3) {
#pragma unroll
        for (int d = 0; d < 4; ++d) xv[d] = xn[d];
      }
    }
    if (refill) {
      b.gs = load_scales16<FULL>(gt2 + o, SC2);
      b.us = load_scales16<FULL>(gt2 + SC2 * 272 + o, SC2);
    }
  }
};

// FC2 of two 16-row groups g0, g0 + 4 (rows of H) of an expert against the h
// row staged in LDS as bf16 hi and lo parts (h = hi + lo to about 2^-17), on
// the matrix cores: one 16x16x32 MFMA per tile and step, whose B operand
// takes hi in the even columns and lo in the odd ones, so that column 0 plus
// column 1 of the product is the FC2 row against h.  Lane l ends with rows
// 4 (l / 16) .. + 3 of column l % 16.
template <int RG, bool FULL>
struct Fc2Tile {
  static_assert(RG == 1, "the batch-1 streams take one row");
  const uint8_t* down;  // packed down region of the blob
  int C2, g0, ng;
  const u32x4* hs;      // hi granules at 0, lo granules at hlo (8 bf16 each, swizzled)
  int hlo;
  f32x4 acc[2];
  __device__ void load(TileBuf2& b, int s) {
    const int SC = FULL ? 16 : min(16, C2 - 16 * s);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      load_tile16<FULL>(down + tile_off(g0 + 4 * (t < ng ? t : 0), s, C2) + after(after(0, acc[0][0]), acc[1][0]), SC, b.q[t], b.s[t]);
  }
  // h granule of step i = 4 kb + d (block 4 kb + q of the segment); odd
  // columns read the lo part
  __device__ int hg(int s, int SC, int i) const {
    const int l = threadIdx.x & 63, q = l >> 4, c = 4 * (i >> 2) + q;
    return (l & 1) * hlo + swz((16 * s + (FULL ? c : min(c, SC - 1))) * 4 + (i & 3));
  }
  // With `refill`, slab kb of both tiles is refilled as soon as its last
  // dword is decoded from the tile pair rt0, rt1 (SC2 blocks: a pass two
  // ahead, of this unit or of the next), the scale vectors after the last slab.
  __device__ void math(TileBuf2& b, int s, bool refill, const uint8_t* rt0, const uint8_t* rt1, int SC2) {
    const int q = (threadIdx.x & 63) >> 4;
    const int SC = FULL ? 16 : min(16, C2 - 16 * s);
    u32x4 hv[4], hn[4];  // h granules of this slab and of the next (read one slab ahead)
#pragma unroll
    for (int d = 0; d < 4; ++d) hv[d] = hs[hg(s, SC, d)];
    const uint32_t sd[2] = {scale_dword16<FULL>(b.s[0], q), scale_dword16<FULL>(b.s[1], q)};
    int o = 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb < 3) {
#pragma unroll
        for (int d = 0; d < 4; ++d) hn[d] = hs[after(hg(s, SC, 4 * kb + 4 + d), acc[0][0])];
      }
      const int c = 4 * kb + q;
      const uint32_t msk = (FULL || c < SC) ? 0xFFFFFFFFu : 0u;
      bf16x8 wv[2];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 h8 = __builtin_bit_cast(bf16x8, hv[d]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          wv[t] = fp4x8_bf16(b.q[t][kb][d] & msk, e8m0_scale(tile_scale(sd[t], kb)));
          acc[t] = mfma_bf16(wv[t], h8, acc[t]);
        }
      }
      if (refill) {
        o = after_u(after_u(o, __builtin_bit_cast(u32x4, wv[0])[3]), __builtin_bit_cast(u32x4, wv[1])[3]);
#pragma unroll
        for (int t = 0; t < 2; ++t) b.q[t][kb] = load_slab<FULL>((t == 0 ? rt0 : rt1) + o, SC2, kb);
      }
      if (kb < 3) {
#pragma unroll
        for (int d = 0; d < 4; ++d) hv[d] = hn[d];
      }
    }
    if (refill) {
#pragma unroll
      for (int t = 0; t < 2; ++t) b.s[t] = load_scales16<FULL>((t == 0 ? rt0 : rt1) + o, SC2);
    }
  }
};

// Granule offset of the lo part of an h row staged by stage_h_split: the hi
// part takes granules [0, K/8) (rounded up to 8), the lo part follows.
__host__ __device__ inline int h_lo_offset(int K) { return ((K / 8 + 7) / 8) * 8; }

// bf16 round-to-nearest-even of an fp32 value (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The h row of `slot` (tagged pairs written earlier in this launch),
// polled until every pair carries this call's tag, into LDS as two bf16
// rows: hi = bf16(h) and lo = bf16(h - hi), so that hi + lo is h to within
// about 2^-17 relative.  Element e sits at bf16 (swz(e / 8), e % 8) of each
// row (8-element granules, the layout of the x row), lo at granule offset hlo.
// The caller's unit starts right after the unit loop's barrier, so no wave
// still reads the previous unit's LDS h.
__device__ __forceinline__ void stage_h_split(const LayerParams& p, const WgState& st, u32x4* hs, const uint64_t* src,
                                              int slot, int K, int hlo) {
  uint16_t* h16 = reinterpret_cast<uint16_t*>(hs);
  const size_t row = (size_t)slot * K;
  bool ok = true;
  for (int base = threadIdx.x; base < K; base += 256 * 8) {
    uint64_t v[8];
    const int n = min(8, (K - base + 255) / 256);
    ok &= poll_pairs_cached<8>(src, n, [&](int t) { return row + base + 256 * t; }, st.tag, v, SPIN_LIMIT,
                               p.ctrl + CTRL_ERR);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = base + 256 * t;
      if (e < K) {
        const float h = pair_f32(v[t]);
        const uint32_t hi = bf16_rne(h);
        const uint32_t lo = bf16_rne(h - __uint_as_float(hi << 16));
        h16[swz(e >> 3) * 8 + (e & 7)] = (uint16_t)hi;
        h16[(hlo + swz(e >> 3)) * 8 + (e & 7)] = (uint16_t)lo;
      }
    }
  }
  if (!ok) set_error(p);
  __syncthreads();
}

// ---- units --------------------------------------------------------------------

// Expert-gathered schedule from the routing pairs of all B*k slots (LDS
// counting; 256 threads).  LDS: cnt[E], start[E], ids[B*k].
template <bool OPQ>
__device__ __forceinline__ void build_schedule(const LayerParams& p, const WgState& st, int* cnt, int* wtot /* LDS [12] */) {
  const int TID_ = OPQ ? tidx() : (int)threadIdx.x;
  // Per expert, the set of batch rows that picked it (bit r: row r; a row
  // picks an expert at most once): its size is the expert's row count, and a
  // slot's place in the expert's row list is the number of lower rows in the
  // set, so every call lists an expert's rows in row order whatever order the
  // threads run in.  Which rows share a column group is then the same on
  // every call, and so are the results (the narrow and wide FC2 paths sum in
  // different orders).
  uint64_t* rowset = reinterpret_cast<uint64_t*>(cnt);  // [E], 8-byte aligned (the LDS region's start)
  int* start = cnt + 2 * p.E;
  int* ids = start + p.E;
  const int t = TID_, nslots = p.B * p.k;
  bool ok = true;
  for (int base = t; base < nslots; base += 256 * 8) {
    uint64_t v[8];
    const int n = min(8, (nslots - base + 255) / 256);
    ok &= poll_pairs<8>(p.idx_p, n, [&](int i) { return base + 256 * i; }, st.tag, v, SPIN_LIMIT, p.ctrl + CTRL_ERR);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (base + 256 * i < nslots) ids[base + 256 * i] = (int)min((uint32_t)v[i], (uint32_t)p.E - 1u);
  }
  if (!ok) set_error(p);
  for (int e = t; e < p.E; e += 256) rowset[e] = 0ull;
  __syncthreads();
  for (int s = t; s < nslots; s += 256) atomicOr(reinterpret_cast<unsigned long long*>(&rowset[ids[s]]), 1ull << (s / p.k));
  __syncthreads();
  const int per = (p.E + 255) / 256, e0 = t * per;
  int run_rows = 0, run_act = 0, run_cg = 0;  // rows, active experts, column groups
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < p.E) {
      const int ce = __popcll(rowset[e]);
      run_rows += ce;
      run_act += ce > 0;
      run_cg += (ce + 15) >> 4;
    }
  }
  const int lane = t & 63, w = t >> 6;
  int ir = run_rows, ia = run_act, ic = run_cg;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int vr = __shfl_up(ir, d, 64), va = __shfl_up(ia, d, 64), vc = __shfl_up(ic, d, 64);
    if (lane >= d) {
      ir += vr;
      ia += va;
      ic += vc;
    }
  }
  if (lane == 63) {
    wtot[w] = ir;
    wtot[4 + w] = ia;
    wtot[8 + w] = ic;
  }
  __syncthreads();
  int base_r = 0, base_a = 0, base_c = 0;
  for (int i = 0; i < w; ++i) {
    base_r += wtot[i];
    base_a += wtot[4 + i];
    base_c += wtot[8 + i];
  }
  int pr = base_r + ir - run_rows, pa = base_a + ia - run_act, pc = base_c + ic - run_cg;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < p.E) {
      const int ce = __popcll(rowset[e]);
      start[e] = pr;
      if (ce > 0) {
        st_coh(p.active + pa, e);
        st_coh(p.row_off + pa, pr);
        st_coh(p.cg_off + pa, pc);
        ++pa;
      }
      pr += ce;
      pc += (ce + 15) >> 4;
    }
  }
  if (t == 255) {
    st_coh(p.row_off + base_a + ia, base_r + ir);
    st_coh(p.cg_off + base_a + ia, base_c + ic);
  }
  __syncthreads();
  for (int s = t; s < nslots; s += 256) {
    const int e = ids[s], r = s / p.k;
    st_coh(p.rows + start[e] + __popcll(rowset[e] & ((1ull << r) - 1ull)), s);
  }
  // publish: every thread's schedule stores complete, then the ready word
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0)
    st_coh(reinterpret_cast<uint64_t*>(p.ctrl + CTRL_READY), make_pair((uint32_t)(wtot[4] + wtot[5] + wtot[6] + wtot[7]), st.tag));
}

// Router unit (batch 1): experts 4u .. 4u+3, one per wave; lane l takes
// 8-element granules l, l + 64, ... of the wave's expert row.  The weight
// granules and the matching activation granules (read from global memory: the
// one 14 KB row stays in L2 for every unit) are all requested before any is
// used, so a unit costs a single memory round trip, and no wave waits for
// another.  With four experts a unit, the router takes the first quarter of
// the launch's workgroups -- the first workgroup of each CU, which starts
// streaming before the CU's second one.  bf16 x bf16 products are exact in
// fp32 and are summed in fp64.
__device__ __forceinline__ void router_unit(const LayerParams& p, WgState& st, int u) {
  constexpr int NG = 14;  // granules in flight per lane: a whole row at H 7168
  const int lane = threadIdx.x & 63;
  const int e = 4 * u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = p.H / 8;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(p.wr + (size_t)min(e, p.E - 1) * p.H);
  const u32x4* xr = reinterpret_cast<const u32x4*>(p.x);
  double acc = 0.0;
  for (int c0 = lane; c0 < C; c0 += 64 * NG) {
    u32x4 q[NG], xv[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int c = min(c0 + 64 * i, C - 1);
      q[i] = ld_weight16(wrow + c);
      xv[i] = ld16(xr + c);
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const uint32_t msk = (c0 + 64 * i < C) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wq = q[i][d] & msk;
        acc += (double)(bf16_lo(wq) * bf16_lo(xv[i][d]));
        acc += (double)(bf16_hi(wq) * bf16_hi(xv[i][d]));
      }
    }
  }
  acc = sum_lanes_f64<64>(acc);
  if (e < p.E && lane == 0) {
    const double bb = p.bias ? (double)p.bias[e] : 0.0;
    st_pair_f32(p.logits_p + e, (float)(acc + bb), st.tag);
  }
}

// Sum over the 64 lanes of each of N (a power of two <= 32) per-lane values,
// reduce-scatter style: at each step a lane keeps half of its values and adds
// its partner's copy of that half, so N - 1 shuffles (plus 6 - log2 N for the
// last value) replace 6 per value.  Lane l ends with the total of value
// (l >> (6 - log2 N)) ... for N 32: value (l >> 1) & 31, held by lanes 2 m and
// 2 m + 1.

template <int CNT, int M, int N>
__device__ __forceinline__ void reduce_scatter_step(double (&v)[N], int lane) {
  if constexpr (CNT > 1) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < CNT / 2; ++i) {
      const double recv = __shfl_xor(up ? v[i] : v[i + CNT / 2], M, WAVE);
      v[i] = (up ? v[i + CNT / 2] : v[i]) + recv;
    }
    reduce_scatter_step<CNT / 2, M / 2>(v, lane);
  }
}

template <int N>
__device__ __forceinline__ double reduce_scatter_f64(double (&v)[N]) {
  static_assert(N >= 1 && N <= 32 && (N & (N - 1)) == 0, "N: a power of two up to 32");
  const int lane = threadIdx.x & 63;
  reduce_scatter_step<N, 32>(v, lane);
  double t = v[0];
#pragma unroll
  for (int m = 64 / (2 * N); m >= 1; m >>= 1) t += __shfl_xor(t, m, WAVE);
  return t;
}

// Router unit at batch > 1: experts 4 eg .. 4 eg + 3 against rows 8 rb ..
// 8 rb + 7 (u = rb * groups + eg).  The four waves split K into quarters;
// lane l takes 8-element chunks l, l + 64, ... of its wave's quarter for all
// 4 experts and 8 rows, so every activation chunk read from global memory
// (the few hundred KB of x stay in L2) serves 4 experts (the unit is bound by
// its fp64 arithmetic, not by these loads).  bf16 values and their
// products are exact in fp64 and are summed by fp64 FMA (the exact sums the
// batch-1 router computes); the quarters meet in LDS.
__device__ __forceinline__ void router_mf_unit(const LayerParams& p, WgState& st, Lds& L, int u) {
  constexpr int RB = 8, EW = 4;  // rows and experts per unit
  const int eg = u % p.n_rt_e, rb = u / p.n_rt_e;
  const int w = tidx() >> 6, lane = tidx() & 63;
  const int e0 = EW * eg, b0 = RB * rb, nr = min(RB, p.B - b0);
  const int C = p.H / 8, Q = (C + 3) / 4, c_lo = w * Q, c_hi = min(C, c_lo + Q);
  const int J = (Q + 63) / 64;
  const u32x4* wr[EW];
#pragma unroll
  for (int e = 0; e < EW; ++e) wr[e] = reinterpret_cast<const u32x4*>(p.wr + (size_t)min(e0 + e, p.E - 1) * p.H);
  const u32x4* xr[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) xr[r] = reinterpret_cast<const u32x4*>(p.x + (size_t)(b0 + min(r, nr - 1)) * p.H);
  double acc[EW * RB];
#pragma unroll
  for (int i = 0; i < EW * RB; ++i) acc[i] = 0.0;
  for (int j = 0; j < J; ++j) {
    u32x4 wv[EW], xv[RB];
    {
      const int c = min(c_lo + lane + 64 * j, C - 1);
#pragma unroll
      for (int e = 0; e < EW; ++e) wv[e] = ld_weight16(wr[e] + c);
#pragma unroll
      for (int r = 0; r < RB; ++r) xv[r] = xr[r][c];
    }
    const uint32_t msk = (c_lo + lane + 64 * j < c_hi) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      double xd[RB], wd[EW];
#pragma unroll
      for (int r = 0; r < RB; ++r) xd[r] = (double)((d & 1) ? bf16_hi(xv[r][d >> 1]) : bf16_lo(xv[r][d >> 1]));
#pragma unroll
      for (int e = 0; e < EW; ++e)
        wd[e] = (double)((d & 1) ? bf16_hi(wv[e][d >> 1] & msk) : bf16_lo(wv[e][d >> 1] & msk));
#pragma unroll
      for (int e = 0; e < EW; ++e)
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[e * RB + r] = fma(wd[e], xd[r], acc[e * RB + r]);
    }
  }
  const double v = reduce_scatter_f64<EW * RB>(acc);  // lanes 2 m, 2 m + 1: value m = (e, r)
  double* part = reinterpret_cast<double*>(L.red);   // [4 waves][32]
  __syncthreads();  // L.red is free (the previous unit is done with it)
  if ((lane & 1) == 0) part[w * 32 + (lane >> 1)] = v;
  __syncthreads();
  if (tidx() < EW * RB) {
    const int i = tidx(), e = e0 + i / RB, r = i % RB;
    if (e < p.E && r < nr) {
      const double bb = p.bias ? (double)p.bias[e] : 0.0;
      const double t = ((part[i] + part[32 + i]) + part[64 + i]) + part[96 + i];
      st_pair_f32(p.logits_p + (size_t)(b0 + r) * p.E + e, (float)(t + bb), st.tag);
    }
  }
}

// Router unit on the matrix cores (batch > 16): experts 16 et .. 16 et + 15
// against activation rows 16 rt .. 16 rt + 15, one v_mfma_f64_16x16x4_f64 per
// 4 elements of K, the four waves splitting K.  Per step lane 16 q + r holds
// the 8-element granule 4 j + q of expert row r (A) and of activation row r
// (B), and 8 MFMAs take element i of it as k-slot q.  bf16 values and their
// products are exact in fp64 and every partial sum is exact, so the logits
// are the same exact sums, rounded once, as the other router units'; one
// conversion per operand element instead of one per product, and the sums
// run on the matrix pipe.  Eight 4-granule chunks per wave stay in flight;
// the waves' partial tiles meet in LDS.  The result tile: element i of lane
// 16 q + r is expert row 4 i + q, activation column r.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void router_f64_unit(const LayerParams& p, WgState& st, char* mfb, int u) {
  constexpr int D = 16;  // chunks in flight per wave
  const int et = u % p.n_rt_e, rt = u / p.n_rt_e;
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int e0 = 16 * et, b0 = 16 * rt;
  const int C = p.H / 8, NCH = (C + 3) / 4, per = (NCH + 3) / 4;
  const int ch0 = w * per, ch1 = min(NCH, ch0 + per);
  const u32x4* wrow = reinterpret_cast<const u32x4*>(p.wr + (size_t)min(e0 + r, p.E - 1) * p.H);
  const u32x4* xrow = reinterpret_cast<const u32x4*>(p.x + (size_t)min(b0 + r, p.B - 1) * p.H);
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  u32x4 wb[D], xb[D];
  auto gran = [&](int ch) { return min(4 * min(ch, NCH - 1) + q, C - 1); };
#pragma unroll
  for (int i = 0; i < D; ++i) {
    wb[i] = ld_weight16(wrow + gran(ch0 + i));
    xb[i] = xrow[gran(ch0 + i)];
  }
  for (int j0 = ch0; j0 < ch1; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int ch = j0 + i;
      const bool live = ch < ch1 && 4 * ch + q < C;
      const uint32_t msk = live ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wv = wb[i][d] & msk, xv = xb[i][d];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(wv), (double)bf16_lo(xv), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(wv), (double)bf16_hi(xv), acc, 0, 0, 0);
      }
      if (j0 + D + i < ch1) {  // refill this slot with the chunk D ahead
        const int g = gran(j0 + D + i) + after(0, (float)acc[0]);
        wb[i] = ld_weight16(wrow + g);
        xb[i] = xrow[g];
      }
    }
  }
  double* part = reinterpret_cast<double*>(mfb);  // [4 waves][16 expert rows][16 columns]
#pragma unroll
  for (int i = 0; i < 4; ++i) part[(w * 16 + 4 * i + q) * 16 + r] = acc[i];
  __syncthreads();
  const int t = tidx(), row = t >> 4, col = t & 15, e = e0 + row, b = b0 + col;
  if (e < p.E && b < p.B) {
    const double sum = ((part[t] + part[256 + t]) + part[512 + t]) + part[768 + t];
    const double bb = p.bias ? (double)p.bias[e] : 0.0;
    st_pair_f32(p.logits_p + (size_t)b * p.E + e, (float)(sum + bb), st.tag);
  }
}

// Routing unit of row b: top-k over the row's logits (polled until the router
// has written them all) and the gates.  Top-k state lives in LDS (the x
// region): holding it in registers would set the register budget -- and so
// the occupancy -- of the whole kernel.
template <int TPL>
__device__ __forceinline__ void routing_unit(const LayerParams& p, WgState& st, Lds& L, int* lds_ints, int b) {
  __builtin_amdgcn_s_setprio(3);  // on the critical path: issue ahead of streaming waves
  const size_t s0 = (size_t)b * p.k;
  uint32_t* cand = reinterpret_cast<uint32_t*>(lds_ints);
  // Pass 0 is the dry run, pass 1 the real one.  Both run the SAME instructions
  // (one copy of the code: the loop is not unrolled and the pass number is
  // opaque to the compiler), so the dry run leaves exactly the code of the real
  // pass in the instruction cache.
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
    int dry = pass == 0;
    asm volatile("" : "+v"(dry));
    dry = __builtin_amdgcn_readfirstlane(dry);
    __syncthreads();  // the LDS region is reused
    if (!topk_row_wg<TPL>(p.logits_p + (size_t)b * p.E, p.E, p.k, st.tag, SPIN_LIMIT, p.ctrl + CTRL_ERR, cand,
                          p.idx + s0, p.gate + s0, p.idx_p + s0, p.gate_p + s0, dry != 0))
      set_error(p);
  }
  st.x_cached = false;
  __builtin_amdgcn_s_setprio(0);
}

template <int RG, bool FULL>
__device__ __forceinline__ void shared_fc1_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int t) {
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
    f.out = p.hs_p;
    f.out_ld = p.Is;
    f.row = L.slot + g0;
    const int nrows = f.n0 < n_end ? (n_end - f.n0 + 3) / 4 : 0;
    const int P = nrows * f.nseg;
    BfBuf<CPL1> ba, bb;
    prime_passes(f, P, ba, bb);
    f.tag = st.tag;
    stage_x(p, st, L, xs, false, g0, nr);
    drive_passes(f, P, ba, bb);
  }
}

// The units after the static ones form two interleaved work queues with a
// counter each: workgroup w takes units n_static + q + 2 c (q = bit 3 of w,
// c = 0, 1, ... from counter q).  One counter for all workgroups serialised
// the claims of the batch-1 layer (about 3,300 in ~70 us) enough to cost it
// ~4-5 us.  Workgroups are dealt to the 8 XCDs in turn, so bit 3 puts half of
// every XCD's workgroups in each queue, and both queues get the same mix of
// workgroups (first units, XCDs, counter latency) and advance together; a
// split by workgroup parity (queue = XCD parity) measured ~1 us slower, a
// split by the workgroup's slot on its CU drifted apart and gained nothing,
// and four or eight queues gained less.  A unit waits only on units of lower
// index, so the lowest unfinished unit is either claimed (its inputs are
// done, it completes) or unclaimed with every claimed unit of its queue below
// it and finished, and then that queue's workgroups are free to take it: no
// deadlock while each queue has a workgroup (grids under 16 workgroups run
// one queue).
__device__ __forceinline__ int queue_id(const LayerParams& p) { return p.nq > 1 ? (int)((blockIdx.x >> 3) & 1u) : 0; }

__device__ __forceinline__ unsigned claim_next(const LayerParams& p) {
  return __hip_atomic_fetch_add(p.ctrl + (queue_id(p) ? CTRL_HEAD1 : CTRL_HEAD), 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

// Unit index of this workgroup's claim number c (claim_next's result).
__device__ __forceinline__ int queue_unit(const LayerParams& p, unsigned c) {
  return p.n_static + queue_id(p) + p.nq * (int)c;
}

// The next unit of the queue, which thread 0 claimed at the top of the
// current one, posted for the waves to read in the middle of the unit
// (unext: thread 0's claim number, as claimed): the
// word carries the unit-loop iteration it belongs to, and a wave polls LDS
// until it shows the current one.  One word serves every iteration: all of
// iteration i's reads come before the barrier that ends i, and iteration
// i + 1's write after it.
__device__ __forceinline__ void post_next(const LayerParams& p, Lds& L, int it, unsigned unext) {
  if (threadIdx.x == 0)
    __hip_atomic_store(&L.pre, ((uint64_t)(uint32_t)(it + 1) << 32) | (uint32_t)queue_unit(p, unext),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Batch 1 (thread 0): once the claimed next unit is past the end of the
// queue, this workgroup will claim nothing more, so it counts itself out on
// the exit counter now, during its last unit, instead of after it: the last
// count -- and the queue reset it triggers -- then leaves the layer's end
// one memory round trip earlier.  (The unit loop stops before claiming once
// its index is past the end, so no claim follows a count.)
__device__ __forceinline__ void count_out_early(const LayerParams& p, WgState& st, unsigned unext) {
  if (p.n_total > 0 && !st.exited && queue_unit(p, unext) >= p.n_total) {
    st.exit_old = __hip_atomic_fetch_add(p.ctrl + CTRL_EXIT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st.exited = true;
  }
}

__device__ __forceinline__ int read_next(Lds& L, int it) {
  uint64_t v;
  while (((v = __hip_atomic_load(&L.pre, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >> 32) !=
         (uint64_t)(uint32_t)(it + 1))
    __builtin_amdgcn_s_sleep(1);
  return __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}

// Passes of wave w in a batch-1 routed FC1 unit: wave w takes segments w,
// w + 4, w + 8, ... (Fc1Tile::seg); at H 7168 (14 segments) 4, 4, 3 and 3.
__device__ __forceinline__ int fc1_passes(int S1, int w) { return w < S1 ? (S1 - w + 3) / 4 : 0; }

// One routed FC1 + SwiGLU unit at batch 1 (row group g of active expert a).
// `held`: the unit before already issued this unit's first two passes into
// the tile buffers.  The wave's refills run two passes ahead; when its pass
// count P is even (>= 2) the last two refills of the unit take the first two
// passes of the next unit of the queue instead, if that is a routed FC1 unit
// too (`nfc1`, resolved from the posted next index just before the first of
// them; pass 0 then lands in buffer a, pass 1 in b).  So the stream of the
// waves that set the unit's length (4 passes at H 7168) goes on across the
// unit boundary instead of draining, and the next unit starts with their
// data already in flight.  Waves with an odd count (3 passes, one pass of
// slack) load their first passes at the unit's start: handing those on too,
// or re-dealing the segments 4, 4, 4, 2 so that every wave hands on, measured
// no better, as did claiming the queue in pairs.
//
// Thread 0 posts the next unit index (`unext`, claimed at the top of the
// unit) for the other waves at wave 0's pass 1 (pass 0 if P < 3): reading
// the claim's result waits for every load issued before it, and by then the
// wave needs the first two passes' data anyway.  Wave 0 always has a pass,
// posts before it resolves, and waits for no other wave between the unit's
// start and the post, so every wave's poll ends.
template <bool FULL>
__device__ __forceinline__ void fc1_unit_b1(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int a, int g, int it,
                                            unsigned unext, bool held, TileBuf1& ba, TileBuf1& bb, bool& nfc1,
                                            unsigned& unext2) {
  const int slot = __builtin_amdgcn_readfirstlane(st.s_rows[st.s_row_off[a]]);  // batch 1: one row per expert
  const uint8_t* blob = p.experts + (size_t)__builtin_amdgcn_readfirstlane(st.s_active[a]) * p.blob_bytes;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // w: wave-uniform (scalar)
  const int C1 = p.H / 32, S1 = (C1 + 15) / 16;
  const int P = fc1_passes(S1, w);
  const int base = p.n_rt + p.n_ro + p.n_sch + p.n_s1, n1 = st.U * p.T1;
  Fc1Tile<1, FULL> f;
  f.blob = blob;
  f.C1 = C1;
  f.g = g;
  f.w = w;
  f.xs = xs;
  f.xstride = p.xstride;
  f.ag = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f.au = f.ag;
  if (!held) prime_passes(f, P, ba, bb);
  stage_x(p, st, L, xs, true, 0, 1);
  const bool hand_on = P >= 2 && (P & 1) == 0;
  bool resolved = false;
  const uint8_t* nblob = blob;
  int ng = 0;
  nfc1 = false;
  const int post_pp = P >= 3 ? 1 : 0;
  // pass pp's refill: this unit's pass pp + 2, or pass pp + 2 - P (0 or 1) of the next
  auto step = [&](TileBuf1& b, int pp) {
    const int q = pp + 2;
    if (pp == post_pp) post_next(p, L, it, unext);
    if (q >= P && !resolved && hand_on) {
      resolved = true;
      const int rn = read_next(L, it) - base;
      if ((unsigned)rn < (unsigned)n1) {
        const int an = rn / p.T1;
        ng = rn - an * p.T1;
        nblob = p.experts + (size_t)__builtin_amdgcn_readfirstlane(st.s_active[an]) * p.blob_bytes;
        nfc1 = true;
      }
    }
    const bool own = q < P;
    const int s2 = f.seg(own ? q : q - P);
    const int SC2 = FULL ? 16 : min(16, C1 - 16 * s2);
    f.math(b, pp, own || nfc1, (own ? blob : nblob) + 2 * tile_off(own ? g : ng, s2, C1), SC2);
  };
  for (int pp = 0; pp < P; pp += 2) {
    step(ba, pp);
    if (pp + 1 < P) step(bb, pp + 1);
  }
  // when the next unit is a routed FC1 unit too (the run goes on), the claim
  // of the one after it goes out now, so its result is in when the next unit
  // posts it
  if (threadIdx.x == 0 && (unsigned)(queue_unit(p, unext) - base) < (unsigned)n1) unext2 = claim_next(p);
  if ((lane & 15) == 0) {  // column 0: lane 16 q holds rows 4 q .. 4 q + 3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      L.red[w][0][4 * (lane >> 4) + i][0] = f.ag[i];
      L.red[w][0][4 * (lane >> 4) + i][1] = f.au[i];
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < 16) {
    const int row = threadIdx.x;
    float vg = 0.0f, vu = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      vg += L.red[ww][0][row][0];
      vu += L.red[ww][0][row][1];
    }
    st_pair_f32(p.hr_p + (size_t)slot * p.I + 16 * g + row, silu_f(vg) * vu, st.tag);
  }
  // L.red is next written by a later unit, after the unit loop's barrier
}

// Routed FC1 + SwiGLU at batch 1 over a run of consecutive units of the
// queue that are all routed FC1 units, unit u first (its successor already
// claimed into thread 0's `nxt`).  Each unit hands its two tile buffers on to
// the next (fc1_unit_b1), so they stay live only inside this loop.  The
// unit-loop protocol is kept unit by unit: at the end publish the claimed
// next index, take the barrier, advance `it`.  The claim of the one after is
// issued by the unit before, after its last pass and only when the run goes
// on: a claim is a memory round trip (~3-5 us under full streaming), and
// claimed at the next unit's start its result held every wave at the hand-on
// (~1.5 us a layer).  Returns the first unit index that is not a routed FC1
// unit, claimed but not started (its successor not yet claimed).
template <bool FULL>
__device__ __forceinline__ int routed_fc1_run(const LayerParams& p, WgState& st, Lds& L, u32x4* xs, int u, int& it,
                                              unsigned& nxt) {
  const int base = p.n_rt + p.n_ro + p.n_sch + p.n_s1, n1 = st.U * p.T1;
  TileBuf1 b0, b1;
  bool held = false;
  unsigned nxt2 = 0;
  for (;;) {
    const int rel = u - base, a = rel / p.T1, g = rel - a * p.T1;
    bool next_held;
    fc1_unit_b1<FULL>(p, st, L, xs, a, g, it, nxt, held, b0, b1, next_held, nxt2);
    held = next_held;
    if (threadIdx.x == 0) L.nxt[it & 1] = queue_unit(p, nxt);
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(L.nxt[it & 1]);
    ++it;
    if ((unsigned)(u - base) >= (unsigned)n1) return u;
    if (threadIdx.x == 0) nxt = nxt2;  // claimed by the unit before (the run goes on)
  }
}

template <int RG, bool FULL>
__device__ __forceinline__ void shared_fc2_unit(const LayerParams& p, WgState& st, Lds& L, u32x4* hs, int v) {
  const int m_begin = v * NTS2, m_end = min(p.H, m_begin + NTS2);
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
    f.out = p.os_p;
    f.out_ld = p.H;
    f.row = L.slot + g0;
    const int groups = (m_end - m_begin + 31) / 32;  // 32 rows per block pass (4 waves x 8)
    const int P = m_begin < m_end ? groups * f.nseg : 0;
    BfBuf<CPL2> ba, bb;
    prime_passes(f, P, ba, bb);  // the weights do not depend on FC1
    f.tag = st.tag;
    stage_h(p, st, hs, p.hs_p, L, g0, nr, p.Is);
    drive_passes(f, P, ba, bb);
  }
}

// Routed FC2 at batch 1, unit v of active expert a: 8 row groups (128 rows
// of H); wave w takes groups 8v + w and 8v + w + 4 and runs one pass per
// 16-block segment along I (P = 3 at I 1536), two passes in flight.  The h
// rows alternate between two LDS buffers by unit-loop iteration.
// `held`: the unit before already issued this unit's passes 0 and 1 (per
// wave), and `hheld`, staged its h row (all waves).  Handing on: the refills
// that would run past the unit's last pass take the next queue unit's first
// two passes instead when that is a routed FC2 unit too -- pass 1 first
// (into buffer b) when P is odd, so that pass 0 still lands in buffer a --
// and once the unit's outputs are stored the next unit's h row is staged in
// the other buffer; so the stream goes on across the unit boundary instead
// of draining to one pass in flight for the unit's last round trip and then
// to none while the next unit's h row is read.  The next index comes from
// thread 0's claim at the top of the unit, posted in LDS at wave 0's pass 1
// (pass 0 if P < 3), as for FC1.
template <bool FULL>
__device__ __forceinline__ void fc2_unit_b1(const LayerParams& p, WgState& st, Lds& L, u32x4* hs, int a, int v, int it,
                                            unsigned unext, bool& held, bool& hheld, TileBuf2& ba, TileBuf2& bb,
                                            unsigned& unext2) {
  const int slot = __builtin_amdgcn_readfirstlane(st.s_rows[st.s_row_off[a]]);  // batch 1: the active expert's one row
  const int C1 = p.H / 32, C2 = p.I / 32, S2 = (C2 + 15) / 16;
  const size_t down_off = (size_t)2 * p.I * C1 * 17;
  const uint8_t* down = p.experts + (size_t)__builtin_amdgcn_readfirstlane(st.s_active[a]) * p.blob_bytes + down_off;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // w: wave-uniform (scalar)
  const int G = p.H / 16, g0 = 8 * v + w;
  const int ng = g0 < G ? (g0 + 4 < G ? 2 : 1) : 0;
  const int P = ng > 0 ? S2 : 0;
  const int hlo = h_lo_offset(p.I);
  const int base2 = p.n_rt + p.n_ro + p.n_sch + p.n_s1 + st.U * p.T1 + p.n_s2, n2 = st.U * p.n_r2;
  u32x4* hcur = hs + (it & 1) * p.hstride;
  Fc2Tile<1, FULL> f;
  f.down = down;
  f.C2 = C2;
  f.g0 = min(g0, G - 1);
  f.ng = ng;
  f.hs = hcur;
  f.hlo = hlo;
  f.acc[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f.acc[1] = f.acc[0];
  if (!held) prime_passes(f, P, ba, bb);  // the weights do not depend on FC1
  if (!hheld) stage_h_split(p, st, hcur, p.hr_p, slot, p.I, hlo);
  bool resolved = false, nfc2 = false, nnext = false;
  const uint8_t* ndown = down;
  int ng0 = f.g0, nng = ng, nslot = slot;
  const int post_pp = P >= 3 ? 1 : 0;
  // the next unit, from the posted index: is it a routed FC2 unit, and does
  // this wave have rows in it
  auto resolve = [&]() {
    resolved = true;
    const int rn = read_next(L, it) - base2;
    if ((unsigned)rn < (unsigned)n2) {
      const int an = rn / p.n_r2, gn = 8 * (rn - an * p.n_r2) + w;
      nnext = true;
      nslot = __builtin_amdgcn_readfirstlane(st.s_rows[st.s_row_off[an]]);
      if (gn < G && P >= 2) {
        ng0 = gn;
        nng = gn + 4 < G ? 2 : 1;
        ndown = p.experts + (size_t)__builtin_amdgcn_readfirstlane(st.s_active[an]) * p.blob_bytes + down_off;
        nfc2 = true;
      }
    }
  };
  auto step = [&](TileBuf2& b, int pp) {
    const int q = pp + 2;
    if (pp == post_pp) {
      post_next(p, L, it, unext);
      if (threadIdx.x == 0) count_out_early(p, st, unext);
    }
    if (q >= P && !resolved) resolve();
    const bool own = q < P;
    const int s2 = own ? q : ((q - P) ^ (P & 1));
    const uint8_t* d = own ? down : ndown;
    const int gg = own ? f.g0 : ng0, gk = own ? ng : nng;
    f.math(b, pp, own || nfc2, d + tile_off(gg, s2, C2), d + tile_off(gg + (gk > 1 ? 4 : 0), s2, C2),
           FULL ? 16 : min(16, C2 - 16 * s2));
  };
  for (int pp = 0; pp < P; pp += 2) {
    step(ba, pp);
    if (pp + 1 < P) step(bb, pp + 1);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 val;  // column 0 (hi part) plus column 1 (lo part): lanes 16 q and 16 q + 1
#pragma unroll
    for (int i = 0; i < 4; ++i) val[i] = f.acc[t][i] + __uint_as_float(dpp_u32<0xB1>(__float_as_uint(f.acc[t][i])));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float a, b;
      regroup_rows(val, h, a, b);
      if ((lane & 15) == 0 && t < ng)
        st_pair2_f32(p.or_p, (size_t)slot * p.H + 16 * (g0 + 4 * t) + 8 * h + 2 * (lane >> 4), a, b, st.tag);
    }
  }
  if (!resolved) resolve();  // a wave with no pass (partial last unit) learns the next unit here
  // every wave read the same index, so all of them stage or none does (the
  // staging ends with a barrier)
  if (nnext) {
    // the claim of the unit after next goes out now, beside the next h row's
    // reads, so its result is in when the next unit posts it (claimed at the
    // next unit's start it held every wave ~one memory round trip at pass 1)
    if (threadIdx.x == 0) unext2 = claim_next(p);
    stage_h_split(p, st, hs + ((it + 1) & 1) * p.hstride, p.hr_p, nslot, p.I, hlo);
  }
  held = nfc2;
  hheld = nnext;
}

// Routed FC2 at batch 1 over a run of consecutive units of the queue that
// are all routed FC2 units, unit u first (its successor already claimed into
// thread 0's `nxt`); the tile buffers are handed from unit to unit
// (fc2_unit_b1) and stay live only inside this loop.  The unit-loop protocol
// is kept unit by unit, and the unit before claims the one after next, as in
// routed_fc1_run.  Returns the first unit index that is not a routed FC2
// unit, claimed but not started.
template <bool FULL>
__device__ __forceinline__ int routed_fc2_run(const LayerParams& p, WgState& st, Lds& L, u32x4* hs, int u, int& it,
                                              unsigned& nxt) {
  const int base2 = p.n_rt + p.n_ro + p.n_sch + p.n_s1 + st.U * p.T1 + p.n_s2, n2 = st.U * p.n_r2;
  TileBuf2 b0, b1;
  bool held = false, hheld = false;
  unsigned nxt2 = 0;
  for (;;) {
    const int rel = u - base2, a = rel / p.n_r2, v = rel - a * p.n_r2;
    fc2_unit_b1<FULL>(p, st, L, hs, a, v, it, nxt, held, hheld, b0, b1, nxt2);
    if (threadIdx.x == 0) L.nxt[it & 1] = queue_unit(p, nxt);
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(L.nxt[it & 1]);
    ++it;
    if ((unsigned)(u - base2) >= (unsigned)n2) return u;
    if (threadIdx.x == 0) nxt = nxt2;  // claimed by the unit before (it hands on only to a routed FC2 unit)
  }
}

// Combine unit (row b, tile t of NT2 rows of H): residual += shared output +
// sum_j gate_j * o_j in fixed j order, polling the outputs until they are
// this call's.  Thread i owns row m = t*NT2 + i.
template <bool OPQ>
__device__ __forceinline__ void combine_unit(const LayerParams& p, WgState& st, Lds& L, int b, int t, unsigned unext) {
  const int TID_ = OPQ ? tidx() : (int)threadIdx.x;
  __syncthreads();
  const size_t s0 = (size_t)b * p.k;
  if (TID_ < p.k) {
    uint64_t g[1];
    if (!poll_pairs<1>(p.gate_p + s0, 1, [&](int) { return TID_; }, st.tag, g, SPIN_LIMIT, p.ctrl + CTRL_ERR))
      set_error(p);
    L.gates[TID_] = pair_f32(g[0]);
  }
  __syncthreads();
  const int m = t * NT2 + TID_;
  if (m >= p.H) return;
  float acc = p.residual[(size_t)b * p.H + m];
  bool ok = true;
  if (p.Is > 0) {
    uint64_t v[1];
    ok &= poll_pairs<1>(p.os_p + (size_t)b * p.H + m, 1, [](int) { return 0; }, st.tag, v, SPIN_LIMIT, p.ctrl + CTRL_ERR);
    acc += pair_f32(v[0]);
  }
  for (int j0 = 0; j0 < p.k; j0 += 8) {
    uint64_t v[8];
    const int n = min(8, p.k - j0);
    ok &= poll_pairs<8>(p.or_p + (s0 + j0) * p.H + m, n, [&](int q) { return (size_t)q * p.H; }, st.tag, v,
                        SPIN_LIMIT, p.ctrl + CTRL_ERR);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < n) acc = fmaf(L.gates[j0 + q], pair_f32(v[q]), acc);
  }
  if (!ok) set_error(p);
  if (!OPQ && threadIdx.x == 0) count_out_early(p, st, unext);  // the claim returned before the polls did
  p.residual[(size_t)b * p.H + m] = acc;
}

// ---- MFMA path (batch > 1) ----------------------------------------------------
//
// With more than one activation row per expert the contraction is dense
// enough for the matrix cores: an expert's rows are taken 16 at a time (a
// "column group"), and every 16x16x32 bf16 MFMA multiplies 16 weight rows x
// 32 elements (A) by 32 elements x 16 activation rows (B) into fp32.
//   * A: the packed MXFP4 tiles already hold what a lane needs -- lane
//     l = 16 q + r has, in slab kb, block 4 kb + q of row r (32 elements);
//     dword d of it is exactly the 8 elements of its k-slot for MFMA (kb, d),
//     decoded to bf16 exactly by the scaled conversion.  The bf16 shared
//     expert is read in place (lane l: 8 elements of row r at 32 j + 8 q).
//   * B: activations for a K segment are staged in LDS as [16 columns][KS]
//     bf16 (row stride KS*2 + 16 bytes, so the 16 lanes of a k-slot hit
//     distinct banks); lane l reads column r, the 8 elements of its k-slot.
//     FC2's fp32 h is split into bf16 hi + lo (two MFMAs), which keeps the
//     product within ~2^-17 of the fp32 one.
//   * D: lane l holds rows 4 q .. 4 q + 3 of the tile for column r.
// FC1 stages x segments double-buffered (one barrier per segment); FC2
// stages h per segment after a barrier.  An FC1 unit publishes "tile done"
// (a tagged flag, after its h stores have completed); FC2 units of that
// column group wait for all of its FC1 tiles, then read plain fp32 h.
constexpr int MF_COLS = 16;   // activation rows per column group
constexpr int MF_NT1 = 64;    // FC1 rows per unit: one 16-row group per wave
constexpr int MF_MT2 = 4;     // FC2 unit: four 128-row tiles (two 16-row groups per wave each)
constexpr int MF_NT2 = 128 * MF_MT2;  // FC2 rows of H per unit
constexpr int MF_XS_FP4 = 512 * 2 + 16;  // LDS column stride (bytes) of a 512-element segment
constexpr int MF_XS_BF = 128 * 2 + 16;   // ... of a 128-element segment (bf16 weights)
constexpr int MF_STAGE_BYTES = 2 * MF_COLS * MF_XS_FP4;  // LDS staging region of the MFMA units
constexpr int MF_LA = 2;  // MFMA steps between an LDS read of a B fragment and its use

// Number of columns of a unit's column group, from this workgroup's copy of
// the schedule (no barrier): what load_cols publishes as L.nrows.
__device__ __forceinline__ int unit_ncols(const LayerParams& p, const WgState& st, int a, int cg) {
  if (a < 0) return min(MF_COLS, p.B - MF_COLS * cg);
  return min(MF_COLS, st.s_row_off[a + 1] - (st.s_row_off[a] + MF_COLS * cg));
}

// Column list of a unit: batch rows 16 cg .. of the shared expert (a < 0),
// or rows 16 cg .. of active expert a's row list (slot ids).
__device__ __forceinline__ void load_cols(const LayerParams& p, const WgState& st, Lds& L, int a, int cg) {
  __syncthreads();
  const int n = unit_ncols(p, st, a, cg);
  if ((int)threadIdx.x < n) L.slot[threadIdx.x] = a < 0 ? MF_COLS * cg + threadIdx.x
                                                         : st.s_rows[st.s_row_off[a] + MF_COLS * cg + threadIdx.x];
  if (threadIdx.x == 0) L.nrows = n;
  __syncthreads();
}

// (active expert, column group) of global column group gc (binary search of
// the LDS copy of cg_off).
__device__ __forceinline__ int find_expert(const WgState& st, int gc) {
  int lo = 0, hi = st.U - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.s_cg_off[mid] <= gc) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint64_t* hflag_at(const LayerParams& p, int ex /* umax = shared */, int cg, int t) {
  return p.hflag + ((size_t)ex * 4 + cg) * p.hflag_tiles + t;
}

// x segment [s*KS, s*KS + KS) of the unit's columns into registers (16 B per
// chunk; NCH chunks per thread), zero for absent columns and beyond H.
template <int KS>
struct XSeg {
  static constexpr int NCH = MF_COLS * KS * 2 / 16 / 256;  // 16-byte chunks per thread
  u32x4 v[NCH];
  __device__ void load(const LayerParams& p, const Lds& L, bool routed, int s, int nc) {
    constexpr int CPC = KS * 2 / 16;  // chunks per column
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = threadIdx.x + 256 * i, c = ch / CPC, j = ch - c * CPC;
      const int k0 = s * KS + 8 * j;
      const bool ok = c < nc && k0 < p.H;
      const int b = ok ? (routed ? L.slot[c] / p.k : L.slot[c]) : 0;
      v[i] = ok ? *reinterpret_cast<const u32x4*>(p.x + (size_t)b * p.H + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* buf) const {
    constexpr int CPC = KS * 2 / 16, XS = KS * 2 + 16;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = threadIdx.x + 256 * i, c = ch / CPC, j = ch - c * CPC;
      *reinterpret_cast<u32x4*>(buf + c * XS + 16 * j) = v[i];
    }
  }
};

// One FC1 segment of a wave: gate and up A-operand data.
//   FP4:  q[m][kb] = packed slab kb of the gate (m 0) / up (m 1) tile; s[m] its scales
//   bf16: q[m][j]  = 8 elements of row r at s*128 + 32 j + 8 q
struct MfBuf {
  u32x4 q[2][4];
  uint32_t s[2];
};

template <bool FP4, bool FULL>
__device__ __forceinline__ void mf1_load(const LayerParams& p, const uint8_t* blob, int g, int s, MfBuf& b, float dep) {
  const int lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  if (FP4) {
    const int C1 = p.H / 32;
    const int SC = FULL ? 16 : min(16, C1 - 16 * s);
    const uint8_t* gt = blob + 2 * tile_off(g, s, C1) + after(0, dep);
    load_tile<FULL, true>(gt, SC, b.q[0], b.s[0]);
    load_tile<FULL, true>(gt + SC * 272, SC, b.q[1], b.s[1]);
  } else {
    const int n = min(16 * g + r, p.Is - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = min(s * 128 + 32 * j + 8 * q, p.H - 8) + after(0, dep);
      b.q[0][j] = ld_weight16(p.sg + (size_t)n * p.H + k0);
      b.q[1][j] = ld_weight16(p.su + (size_t)n * p.H + k0);
    }
  }
}

// xb: the segment's activations for this lane's column (column stride
// already applied); xoff: byte offset of the segment inside that column;
// live: this lane's column exists (else its B fragment is zero).
template <bool FP4, bool FULL>
__device__ __forceinline__ void mf1_math(const LayerParams& p, int s, const MfBuf& b, const char* xb, int xoff,
                                         bool live, f32x4& ag, f32x4& au) {
  const int lane = tidx() & 63, q = lane >> 4;
  const u32x4 z{0u, 0u, 0u, 0u};
  if (FP4) {
    const int C1 = p.H / 32;
    const int SC = FULL ? 16 : min(16, C1 - 16 * s);
    // B fragments are read from LDS MF_LA steps ahead; each read is tied to
    // the accumulator of the step before, so the compiler cannot hoist all
    // sixteen (and spill) but the read latency overlaps MF_LA steps of MFMAs.
    auto rd = [&](int i) {
      const int kb = i >> 2, d = i & 3, c = 4 * kb + q;
      return *reinterpret_cast<const u32x4*>(xb + after(xoff + (128 * kb + 32 * q + 8 * (FULL || c < SC ? d : 0)) * 2, ag[0]));
    };
    u32x4 xr[16];
#pragma unroll
    for (int i = 0; i < MF_LA; ++i) xr[i] = rd(i);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int c = 4 * kb + q;
      const uint32_t msk = (FULL || c < SC) ? 0xFFFFFFFFu : 0u;
      const float sg = e8m0_scale(tile_scale(b.s[0], kb));
      const float su = e8m0_scale(tile_scale(b.s[1], kb));
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int i = 4 * kb + d;
        if (i + MF_LA < 16) xr[i + MF_LA] = rd(i + MF_LA);
        const bf16x8 xv = __builtin_bit_cast(bf16x8, (live && (FULL || c < SC)) ? xr[i] : z);
        ag = mfma_bf16(fp4x8_bf16(b.q[0][kb][d] & msk, sg), xv, ag);
        au = mfma_bf16(fp4x8_bf16(b.q[1][kb][d] & msk, su), xv, au);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = s * 128 + 32 * j + 8 * q < p.H;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(xb + xoff + (ok ? (32 * j + 8 * q) * 2 : 0));
      const bf16x8 xv = __builtin_bit_cast(bf16x8, (live && ok) ? raw : z);
      ag = mfma_bf16(__builtin_bit_cast(bf16x8, ok ? b.q[0][j] : z), xv, ag);
      au = mfma_bf16(__builtin_bit_cast(bf16x8, ok ? b.q[1][j] : z), xv, au);
    }
  }
}

// FC1 + SwiGLU of rows [64 t, 64 t + 64) (wave w: row group 4 t + w) of the
// routed expert a (FP4) or the shared expert (bf16, a < 0), column group cg.
template <bool FP4, bool FULL>
__device__ __forceinline__ void mf_fc1_unit(const LayerParams& p, WgState& st, Lds& L, char* mfb, int a, int cg, int t) {
  constexpr int KS = FP4 ? 512 : 128, XS = KS * 2 + 16;
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int N = FP4 ? p.I : p.Is;
  const int g = 4 * t + w;
  const uint8_t* blob = FP4 ? p.experts + (size_t)st.s_active[a] * p.blob_bytes : nullptr;
  const int S = FP4 ? (p.H / 32 + 15) / 16 : (p.H + 127) / 128;
  const int gl = min(g, (N + 15) / 16 - 1);  // waves past the last row group load a valid group, store nothing
  f32x4 ag{0.f, 0.f, 0.f, 0.f}, au{0.f, 0.f, 0.f, 0.f};
  MfBuf ba, bb;
  mf1_load<FP4, FULL>(p, blob, gl, 0, ba, 0.f);
  if (S > 1) mf1_load<FP4, FULL>(p, blob, gl, 1, bb, 0.f);
  load_cols(p, st, L, a, cg);  // after the first weight loads: its barriers overlap them
  const int nc = L.nrows;
  const int XF = p.H * 2 + 16;  // column stride of whole-K staging
  if (nc * XF <= MF_STAGE_BYTES) {
    // Narrow column group: all of K for every column in LDS at once, then
    // the weights stream with no barrier (the common case at small batch).
    constexpr int PER = 8;
    const int CPC = p.H / 8, total = nc * CPC;
    for (int base = tidx(); base < total; base += 256 * PER) {
      u32x4 v[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ch = min(base + 256 * i, total - 1), c = ch / CPC, j = ch - c * CPC;
        const int b = a >= 0 ? L.slot[c] / p.k : L.slot[c];
        v[i] = *reinterpret_cast<const u32x4*>(p.x + (size_t)b * p.H + 8 * j);
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ch = base + 256 * i, c = ch / CPC, j = ch - c * CPC;
        if (ch < total) *reinterpret_cast<u32x4*>(mfb + c * XF + 16 * j) = v[i];
      }
    }
    __syncthreads();
    const bool live = r < nc;
    const char* xcol = mfb + (live ? r : 0) * XF;
    for (int s = 0; s < S; s += 2) {
      mf1_math<FP4, FULL>(p, s, ba, xcol, s * KS * 2, live, ag, au);
      if (s + 2 < S) mf1_load<FP4, FULL>(p, blob, gl, s + 2, ba, ag[0] + au[0]);
      if (s + 1 < S) {
        mf1_math<FP4, FULL>(p, s + 1, bb, xcol, (s + 1) * KS * 2, live, ag, au);
        if (s + 3 < S) mf1_load<FP4, FULL>(p, blob, gl, s + 3, bb, ag[0] + au[0]);
      }
    }
  } else {
    {
      XSeg<KS> x0;
      x0.load(p, L, a >= 0, 0, nc);
      x0.store(mfb);
    }
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ss = s + h;
        if (ss < S) {
          XSeg<KS> xn;
          if (ss + 1 < S) xn.load(p, L, a >= 0, ss + 1, nc);
          MfBuf& b = h ? bb : ba;
          mf1_math<FP4, FULL>(p, ss, b, mfb + (ss & 1) * MF_COLS * XS + r * XS, 0, true, ag, au);
          if (ss + 2 < S) mf1_load<FP4, FULL>(p, blob, gl, ss + 2, b, ag[0] + au[0]);
          if (ss + 1 < S) xn.store(mfb + ((ss + 1) & 1) * MF_COLS * XS);
          __syncthreads();
        }
      }
    }
  }
  // h = silu(gate) * up: rows 16 g + 4 q + i of column r, as fp32 (one 16-byte coherent store)
  float* hout = FP4 ? reinterpret_cast<float*>(p.hr_p) : reinterpret_cast<float*>(p.hs_p);
  const int n0 = 16 * g + 4 * q;
  if (n0 < N && r < nc) {  // N is a multiple of 8: rows n0 .. n0+3 all exist
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_f(ag[i]) * au[i];
    st_f32x4_coh(hout, (size_t)L.slot[r] * N + n0, hv);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every lane's h stores have completed
  __syncthreads();
  if (tidx() == 0) st_coh(hflag_at(p, a < 0 ? p.umax : a, cg, t), make_pair(1u, st.tag));
}

// Shared-expert FC1 + SwiGLU at batch > 1 (bf16 weights): one 16-row group g
// of Is for column group cg.  The four waves split K -- wave w takes the
// 128-element segments w, w + 4, ... -- so a unit is one row group's 458 KB
// (at K3's shape) like a routed unit, not four; the B operand (8 x values of
// the lane's column and k-slot) is read straight from global memory, where
// the B rows of x stay in L2, so no staging or barrier interrupts the
// stream.  Partial sums meet in LDS; h goes out as fp32 with coherent stores,
// then the group's "done" flag (after every store has completed).
template <bool FULL>
__device__ __forceinline__ void mf_sh1_unit(const LayerParams& p, WgState& st, Lds& L, char* mfb, int cg, int g) {
  load_cols(p, st, L, -1, cg);
  const int nc = L.nrows;
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int S = (p.H + 127) / 128;
  const int P = w < S ? (S - w + 3) / 4 : 0;
  const bool live = r < nc;
  const uint16_t* xrow = p.x + (size_t)L.slot[live ? r : 0] * p.H;
  const u32x4 z{0u, 0u, 0u, 0u};
  f32x4 ag{0.f, 0.f, 0.f, 0.f}, au{0.f, 0.f, 0.f, 0.f};
  MfBuf ba, bb;
  u32x4 xa[4], xb[4];
  auto load = [&](MfBuf& b, u32x4 (&xv)[4], int pp, float dep) {
    const int s = w + 4 * pp;
    mf1_load<false, FULL>(p, nullptr, g, s, b, dep);
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = ld16(xrow + min(s * 128 + 32 * j + 8 * q, p.H - 8) + after(0, dep));
  };
  auto math = [&](const MfBuf& b, const u32x4 (&xv)[4], int pp) {
    const int s = w + 4 * pp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = s * 128 + 32 * j + 8 * q < p.H;
      const bf16x8 x8 = __builtin_bit_cast(bf16x8, (live && ok) ? xv[j] : z);
      ag = mfma_bf16(__builtin_bit_cast(bf16x8, ok ? b.q[0][j] : z), x8, ag);
      au = mfma_bf16(__builtin_bit_cast(bf16x8, ok ? b.q[1][j] : z), x8, au);
    }
  };
  if (P > 0) load(ba, xa, 0, 0.f);
  if (P > 1) load(bb, xb, 1, 0.f);
  for (int pp = 0; pp < P; pp += 2) {
    math(ba, xa, pp);
    if (pp + 2 < P) load(ba, xa, pp + 2, ag[0] + au[0]);
    if (pp + 1 < P) {
      math(bb, xb, pp + 1);
      if (pp + 3 < P) load(bb, xb, pp + 3, ag[0] + au[0]);
    }
  }
  // waves' partial sums: lane (q, r) holds rows 4 q + i of column r
  float* red = reinterpret_cast<float*>(mfb);  // [4 waves][2][16 rows][16 columns]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[((w * 2 + 0) * 16 + 4 * q + i) * 16 + r] = ag[i];
    red[((w * 2 + 1) * 16 + 4 * q + i) * 16 + r] = au[i];
  }
  __syncthreads();
  {
    const int row = tidx() >> 4, col = tidx() & 15, n = 16 * g + row;
    float vg = 0.f, vu = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      vg += red[((ww * 2 + 0) * 16 + row) * 16 + col];
      vu += red[((ww * 2 + 1) * 16 + row) * 16 + col];
    }
    if (col < nc && n < p.Is)
      st_coh(reinterpret_cast<uint32_t*>(p.hs_p) + (size_t)L.slot[col] * p.Is + n, __float_as_uint(silu_f(vg) * vu));
  }
  __builtin_amdgcn_s_waitcnt(0);  // every thread's h stores have completed
  __syncthreads();
  if (tidx() == 0) st_coh(hflag_at(p, p.umax, cg, g), make_pair(1u, st.tag));
}

// One FC2 segment of a wave: two 16-row A tiles of the down matrix.
//   FP4:  q[t][kb] = packed slab kb of tile t, s[t] its scales
//   bf16: q[t][j]  = 8 elements of row r of tile t at s*128 + 32 j + 8 q
template <bool FP4, bool FULL>
__device__ __forceinline__ void mf2_load(const LayerParams& p, const uint8_t* down, const int (&gt)[2], int s,
                                         MfBuf& b, float dep) {
  const int lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  if (FP4) {
    const int C2 = p.I / 32;
    const int SC = FULL ? 16 : min(16, C2 - 16 * s);
#pragma unroll
    for (int t = 0; t < 2; ++t) load_tile<FULL, true>(down + tile_off(gt[t], s, C2) + after(0, dep), SC, b.q[t], b.s[t]);
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int m = min(16 * gt[t] + r, p.H - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = min(s * 128 + 32 * j + 8 * q, p.Is - 8) + after(0, dep);
        b.q[t][j] = ld_weight16(p.sd + (size_t)m * p.Is + k0);
      }
    }
  }
}

// hb / lob: this lane's column of the staged h hi / lo halves (column stride
// applied); hoff: byte offset of segment s inside the column; live: the
// column exists (else the B fragments are zero).  PK (at most 8 columns):
// the B operand carries the hi half of column c in column c and the lo half
// in column c + 8 -- hb is then the lane's own half, lob unused -- so one
// MFMA a step does what the hi + lo pair does, and column c's result is
// column c plus column c + 8 of the product (added at the end of the unit).
template <bool FP4, bool FULL, bool PK = false>
__device__ __forceinline__ void mf2_math(const LayerParams& p, int s, const MfBuf& b, const char* hb, const char* lob,
                                         int hoff, bool live, f32x4 (&acc)[2]) {
  const int lane = tidx() & 63, q = lane >> 4;
  const u32x4 z{0u, 0u, 0u, 0u};
  if (FP4) {
    const int C2 = p.I / 32;
    const int SC = FULL ? 16 : min(16, C2 - 16 * s);
    // h fragments are read from LDS MF_LA steps ahead (see mf1_math)
    u32x4 rh[16], rl[16];
    auto rd = [&](int i) {
      const int kb = i >> 2, d = i & 3, c = 4 * kb + q;
      const bool bv = live && (FULL || c < SC);
      const int off = after(hoff + (bv ? (128 * kb + 32 * q + 8 * d) * 2 : 0), acc[0][0] + acc[1][0]);
      rh[i] = *reinterpret_cast<const u32x4*>(hb + off);
      if (!PK) rl[i] = *reinterpret_cast<const u32x4*>(lob + off);
    };
#pragma unroll
    for (int i = 0; i < MF_LA; ++i) rd(i);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int c = 4 * kb + q;
      const uint32_t msk = (FULL || c < SC) ? 0xFFFFFFFFu : 0u;
      float sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t] = e8m0_scale(tile_scale(b.s[t], kb));
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int i = 4 * kb + d;
        if (i + MF_LA < 16) rd(i + MF_LA);
        const bool bv = live && (FULL || c < SC);
        const bf16x8 hi = __builtin_bit_cast(bf16x8, bv ? rh[i] : z);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 wv = fp4x8_bf16(b.q[t][kb][d] & msk, sc[t]);
          acc[t] = mfma_bf16(wv, hi, acc[t]);
          if (!PK) acc[t] = mfma_bf16(wv, __builtin_bit_cast(bf16x8, bv ? rl[i] : z), acc[t]);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = s * 128 + 32 * j + 8 * q < p.Is;
      const int off = hoff + (ok ? (32 * j + 8 * q) * 2 : 0);
      const u32x4 rh = *reinterpret_cast<const u32x4*>(hb + off);
      const bf16x8 hi = __builtin_bit_cast(bf16x8, (live && ok) ? rh : z);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 wv = __builtin_bit_cast(bf16x8, ok ? b.q[t][j] : z);
        acc[t] = mfma_bf16(wv, hi, acc[t]);
        if (!PK) {
          const u32x4 rl = *reinterpret_cast<const u32x4*>(lob + off);
          acc[t] = mfma_bf16(wv, __builtin_bit_cast(bf16x8, (live && ok) ? rl : z), acc[t]);
        }
      }
    }
  }
}

// Columns [0, ncols) x elements [k0, k0 + KE) of h (fp32, written by this
// launch's FC1 units: 8-byte coherent loads, PER per thread per batch) into
// LDS as bf16 hi halves (column c at hb + c * XS) and lo halves (at
// hb + lo_off + c * XS).  Elements at or past K, and absent columns, are 0.
template <int PER>
__device__ __forceinline__ void mf_stage_h(const LayerParams& p, const Lds& L, const float* hsrc, int K, int k0,
                                           int KE, int nc, int ncols, char* hb, int XS, int lo_off) {
  const int HP = KE / 2, total = ncols * HP;  // element pairs
  for (int base = tidx(); base < total; base += 256 * PER) {
    uint64_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = base + 256 * i, c = e / HP, j = e - c * HP;
      const int k = k0 + 2 * j;
      const bool ok = e < total && c < nc && k < K;
      v[i] = ok ? __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(hsrc) + (size_t)L.slot[c] * K + k),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : 0ull;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = base + 256 * i, c = e / HP, j = e - c * HP;
      if (e < total) {
        uint32_t hi2 = 0, lo2 = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float f = __uint_as_float((uint32_t)(v[i] >> (32 * h)));
          const uint16_t hb16 = f32_to_bf16(f);
          const float rem = f - __uint_as_float((uint32_t)hb16 << 16);
          hi2 |= (uint32_t)hb16 << (16 * h);
          lo2 |= (uint32_t)f32_to_bf16(rem) << (16 * h);
        }
        *reinterpret_cast<uint32_t*>(hb + c * XS + 4 * j) = hi2;
        *reinterpret_cast<uint32_t*>(hb + lo_off + c * XS + 4 * j) = lo2;
      }
    }
  }
}

// FC2 of rows [512 t, 512 t + 512) of H -- four 128-row tiles; in tile mt
// wave w takes row groups 8 (4 t + mt) + w and + 4 -- of routed expert a
// (FP4) or the shared expert (a < 0), column group cg, once every FC1 tile of
// that column group is done.  A narrow column group stages all of h once and
// runs one pipelined pass per (tile, segment) with no barrier; a wide one
// stages h 512 elements at a time.
template <bool FP4, bool FULL>
__device__ __forceinline__ void mf_fc2_unit(const LayerParams& p, WgState& st, Lds& L, char* mfb, int a, int cg, int t) {
  const int nc = unit_ncols(p, st, a, cg);
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int K = FP4 ? p.I : p.Is;
  const int G = p.H / 16;
  const uint8_t* down =
      FP4 ? p.experts + (size_t)st.s_active[a] * p.blob_bytes + (size_t)2 * p.I * (p.H / 32) * 17 : nullptr;
  const int S = FP4 ? (K / 32 + 15) / 16 : (K + 127) / 128;
  constexpr int MT2 = FP4 ? MF_MT2 : 1;  // 128-row tiles per unit (shared expert: one, 393 KB of bf16)
  const int MT = min(MT2, (G - 8 * MT2 * t + 7) / 8);  // 128-row tiles of this unit that exist
  auto groups = [&](int mt, int (&gt)[2]) {
    gt[0] = min(8 * (MT2 * t + mt) + w, G - 1);
    gt[1] = min(8 * (MT2 * t + mt) + w + 4, G - 1);
  };
  uint64_t* out = FP4 ? p.or_p : p.os_p;
  auto emit = [&](int mt, const f32x4 (&acc)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int g = 8 * (MT2 * t + mt) + w + 4 * tt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float a, b;
        regroup_rows(acc[tt], h, a, b);
        if (r < nc && g < G) st_pair2_f32(out, (size_t)L.slot[r] * p.H + 16 * g + 8 * h + 2 * q, a, b, st.tag);
      }
    }
  };
  MfBuf ba, bb;
  const int XF = K * 2 + 16;  // column stride of whole-K staging
  // narrow: all of K staged once, at most 8 columns (the packed hi + lo of
  // mf2_math); 1024 columns never fit (written as a select: the plain
  // conjunction made the compiler spill 31 VGPRs)
  const bool narrow = 2 * (nc <= 8 ? nc : 1024) * XF <= MF_STAGE_BYTES;
  {  // the weights do not depend on FC1.  The second pass is tile 1 at
     // segment 0 on the wide FP4 path (chunk order), else tile 0 at segment 1.
    int gt[2];
    groups(0, gt);
    mf2_load<FP4, FULL>(p, down, gt, 0, ba, 0.f);
    const bool by_tile = FP4 && !narrow;
    if (by_tile ? MT > 1 : MT * S > 1) {
      groups(by_tile ? 1 : 1 / S, gt);
      mf2_load<FP4, FULL>(p, down, gt, by_tile ? 0 : 1 % S, bb, 0.f);
    }
  }
  load_cols(p, st, L, a, cg);  // after the first weight loads: its barriers overlap them
  {  // wait until every FC1 tile (shared expert: 16-row group) of this column group has published its h
    const int ntile = FP4 ? (K + MF_NT1 - 1) / MF_NT1 : (K + 15) / 16;
    bool ok = true;
    if (tidx() < ntile) {
      uint64_t f[1];
      const int ti = tidx();
      ok = poll_pairs<1>(hflag_at(p, a < 0 ? p.umax : a, cg, 0), 1, [&](int) { return ti; }, st.tag, f, SPIN_LIMIT,
                         p.ctrl + CTRL_ERR);
    }
    if (!ok) set_error(p);
  }
  const float* hsrc = FP4 ? reinterpret_cast<const float*>(p.hr_p) : reinterpret_cast<const float*>(p.hs_p);
  const f32x4 zero4{0.f, 0.f, 0.f, 0.f};
  if (narrow) {  // all of h staged once; passes tile by tile; hi and lo in one MFMA
    constexpr int KS = FP4 ? 512 : 128;
    const int P = MT * S;
    const int cc = r & 7;  // lane r < 8: hi half of column r; lane r >= 8: lo half of column r - 8
    const bool live = cc < nc;
    f32x4 acc[2] = {zero4, zero4};
    __syncthreads();
    mf_stage_h<16>(p, L, hsrc, K, 0, K, nc, nc, mfb, XF, nc * XF);
    __syncthreads();
    const char* hcol = mfb + (live ? cc : 0) * XF + (r >= 8 ? nc * XF : 0);
    for (int pp = 0; pp < P; pp += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ps = pp + h;
        if (ps < P) {
          MfBuf& b = h ? bb : ba;
          const int mt = ps / S, sg = ps - mt * S;
          mf2_math<FP4, FULL, true>(p, sg, b, hcol, nullptr, sg * KS * 2, live, acc);
          if (ps + 2 < P) {
            int gt[2];
            groups((ps + 2) / S, gt);
            mf2_load<FP4, FULL>(p, down, gt, (ps + 2) % S, b, acc[0][0] + acc[1][0]);
          }
          if (sg == S - 1) {
            f32x4 sum[2];  // column c + column c + 8: lanes r and r + 8 of a 16-lane row (rotate by 8)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sum[tt][i] = acc[tt][i] + __uint_as_float(dpp_u32<0x128>(__float_as_uint(acc[tt][i])));
            emit(mt, sum);
            acc[0] = zero4;
            acc[1] = zero4;
          }
        }
      }
    }
  } else {
    // Wide column group: h goes through LDS 512 elements at a time (hi and lo
    // halves fill the staging region), and every pass that reads a chunk runs
    // while it is staged, so a unit stages h K / 512 times instead of once per
    // (tile, segment).  Pass (c, j) is FP4 tile j at segment c, or bf16 tile 0
    // at segment 4 c + j; four passes a chunk keep the two weight buffers
    // alternating.
    constexpr int XS = 512 * 2 + 16;
    const int NCH = (K + 511) / 512;
    const bool pk = nc <= 8;
    f32x4 accs[MT2][2];
#pragma unroll
    for (int i = 0; i < MT2; ++i) accs[i][0] = accs[i][1] = zero4;
    auto seg_of = [&](int c, int j) { return FP4 ? c : 4 * c + j; };
    auto pass_ok = [&](int c, int j) { return c < NCH && seg_of(c, j) < S && (FP4 ? j < MT : true); };
    for (int c = 0; c < NCH; ++c) {
      __syncthreads();  // the previous chunk's h is no longer read
      mf_stage_h<16>(p, L, hsrc, K, c * 512, 512, nc, MF_COLS, mfb, XS, MF_COLS * XS);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        MfBuf& b = (j & 1) ? bb : ba;
        f32x4 (&acc_j)[2] = accs[FP4 ? j % MT2 : 0];
        if (pass_ok(c, j)) {
          if (pk)  // at most 8 columns: hi and lo in one MFMA (see mf2_math)
            mf2_math<FP4, FULL, true>(p, seg_of(c, j), b, mfb + (r & 7) * XS + (r >= 8 ? MF_COLS * XS : 0), nullptr,
                                      FP4 ? 0 : j * 256, true, acc_j);
          else
            mf2_math<FP4, FULL>(p, seg_of(c, j), b, mfb + r * XS, mfb + MF_COLS * XS + r * XS, FP4 ? 0 : j * 256, true,
                                acc_j);
        }
        const int c2 = j + 2 < 4 ? c : c + 1, j2 = j + 2 < 4 ? j + 2 : j - 2;
        if (pass_ok(c2, j2)) {
          int gt[2];
          groups(FP4 ? j2 : 0, gt);
          mf2_load<FP4, FULL>(p, down, gt, seg_of(c2, j2), b, acc_j[0][0] + acc_j[1][0]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MT2; ++i) {
      if (i < MT) {
        if (pk) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              accs[i][tt][e] += __uint_as_float(dpp_u32<0x128>(__float_as_uint(accs[i][tt][e])));
        }
        emit(i, accs[i]);
      }
    }
  }
}

// ---- FP4 x MXFP8 routed experts (opt-in: moe_decode_layer_mxfp8) ----------------
//
// The expert kernel of "Kimi K3 on GB300: 13 kernels a layer" (section "Why
// batch 1 on a rack is not only a bandwidth problem") multiplies FP4 weights
// by MXFP8 activations.  On gfx950 that product is one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16 rows x 128 elements x 16 columns,
// which takes both operands as stored and their E8M0 block scales:
//   A (FP4 weights): lane 16 q + r holds row r, elements 32 q .. 32 q + 31 of
//     the 128-element step as 16 bytes -- exactly slab kb of a packed tile --
//     and supplies the scale of (row r, block q): byte kb of the tile's scale
//     dword, which the instruction's byte select picks;
//   B (E4M3 activations): lane 16 q + r holds column r, elements 16 q ..
//     16 q + 15 in its first 16 bytes and 64 + 16 q .. 64 + 16 q + 15 in its
//     last 16, and supplies the scale of (column r, block q);
//   D: lane 16 q + r holds rows 4 q .. 4 q + 3 of column r, as for the bf16
//     instruction.
// No FP4 decode runs on the vector ALU, and FC2 needs one product per step
// instead of the bf16 path's hi + lo pair.  The activations are quantised to
// MXFP8 inside the unit while they are staged: per block of 32 the E8M0 scale
// 2^(floor(log2 amax) - 8) (8: the exponent of E4M3's largest power of two),
// each element the nearest E4M3 value of v / scale, ties to even, magnitudes
// past 448 clamped to 448 (OCP Microscaling Formats v1.0).
// LDS of a unit: column c's codes at c * XQ (whole 512-element segments, zero
// past K), then the scales: dword (c, s, q) holds in byte kb the scale of
// block 16 s + 4 kb + q of column c (127, i.e. 1.0, past K).

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Nearest E4M3 code of v (ties to even), clamped to +-448; v finite.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 464.0f) return s | 0x7Eu;  // past the largest finite value; 464 itself ties to 448 (the even code)
  if (a < 0.015625f) return s | (uint32_t)__builtin_rintf(a * 512.0f);  // subnormals: multiples of 2^-9 (8: 2^-6)
  uint32_t u = __float_as_uint(a);
  u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;  // significand to 3 bits, nearest even
  return s | ((((u >> 23) - 120u) << 3) | ((u >> 20) & 7u));  // exponent bias 127 -> 7
}

// MXFP8 of one block of 32 values: the codes (byte j = element j) and the
// E8M0 scale byte.
__device__ __forceinline__ uint32_t mx8_block(const float (&v)[32], u32x4& c0, u32x4& c1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = ef == 0 ? -127 : min(127, max(-127, ef - 127 - 8));  // floor(log2 amax) - 8
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);      // 2^-e (e <= 119: a normal number)
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d)
    w[d] = e4m3_code(v[4 * d] * inv) | (e4m3_code(v[4 * d + 1] * inv) << 8) | (e4m3_code(v[4 * d + 2] * inv) << 16) |
           (e4m3_code(v[4 * d + 3] * inv) << 24);
  c0 = u32x4{w[0], w[1], w[2], w[3]};
  c1 = u32x4{w[4], w[5], w[6], w[7]};
  return (uint32_t)(e + 127);
}

template <int KB>
__device__ __forceinline__ f32x4 mfma_fp4_mx8(const u32x4& a, const u32x4& b0, const u32x4& b1, uint32_t sa,
                                              uint32_t sb, f32x4 c) {
  const i32x8 av{(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 bv{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, KB, (int)sa, KB, (int)sb);
}

// Columns (a unit's rows of activations) and their MXFP8 staging: codes of
// column c at c * xq, scale dwords at sc + ((c * S + s) * 4 + q) * 4.
struct MxCols {
  char* buf;
  int xq;   // column stride of the codes (bytes)
  int sc;   // byte offset of the scale dwords
  int S;    // segments of 512 elements covered
};

// Stores the MXFP8 of block b (element 32 b ...) of column c; blocks past
// the operand's K hold zero codes and scale 1.
__device__ __forceinline__ void mx8_put(const MxCols& m, int c, int b, int seg0, u32x4 c0, u32x4 c1, uint32_t scale) {
  char* col = m.buf + c * m.xq + 32 * (b - 16 * seg0);
  *reinterpret_cast<u32x4*>(col) = c0;
  *reinterpret_cast<u32x4*>(col + 16) = c1;
  const int s = b / 16 - seg0, w = b % 16;
  m.buf[m.sc + ((c * m.S + s) * 4 + (w & 3)) * 4 + (w >> 2)] = (char)scale;
}

// The 32 bf16 activations of block b of batch row `row` (zero past H).
__device__ __forceinline__ void x_block(const LayerParams& p, int row, int b, float (&v)[32]) {
  if (32 * b < p.H) {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (size_t)row * p.H + 32 * b);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 q = src[g];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[8 * g + 2 * d] = bf16_lo(q[d]);
        v[8 * g + 2 * d + 1] = bf16_hi(q[d]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
}

// One 128-element step kb of segment s for a lane: its B fragment (column
// col) and B scale dword.
__device__ __forceinline__ void mx8_frag(const MxCols& m, int col, int s_local, int kb, int q, u32x4& b0, u32x4& b1,
                                         uint32_t& sb) {
  const char* base = m.buf + col * m.xq + 512 * s_local + 128 * kb + 16 * q;
  b0 = *reinterpret_cast<const u32x4*>(base);
  b1 = *reinterpret_cast<const u32x4*>(base + 64);
  sb = *reinterpret_cast<const uint32_t*>(m.buf + m.sc + ((col * m.S + s_local) * 4 + q) * 4);
}

// A operand data and scale of one FP4 tile slab for a lane; on a partial
// segment, blocks past the tile's SC are zeroed with scale 1.
template <bool FULL>
__device__ __forceinline__ void mx8_a(const u32x4& slab, uint32_t sv, int SC, int kb, int q, u32x4& a, uint32_t& sa) {
  const bool ok = FULL || 4 * kb + q < SC;
  a = ok ? slab : u32x4{0u, 0u, 0u, 0u};
  sa = ok ? sv : 0x7F7F7F7Fu;
}

// FC1 + SwiGLU of rows [64 t, 64 t + 64) of routed expert a, column group cg,
// with MXFP8 activations.  A narrow column group (all of K for every column
// fits the staging region) quantises x once and streams with no barrier; a
// wide one quantises segment by segment into two alternating buffers.
template <bool FULL>
__device__ __forceinline__ void mx_fc1_unit(const LayerParams& p, WgState& st, Lds& L, char* mfb, int a, int cg,
                                            int t) {
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int N = p.I, g = 4 * t + w;
  const uint8_t* blob = p.experts + (size_t)st.s_active[a] * p.blob_bytes;
  const int C1 = p.H / 32, S = (C1 + 15) / 16;
  const int gl = min(g, (N + 15) / 16 - 1);
  f32x4 ag{0.f, 0.f, 0.f, 0.f}, au{0.f, 0.f, 0.f, 0.f};
  MfBuf ba, bb;
  mf1_load<true, FULL>(p, blob, gl, 0, ba, 0.f);
  if (S > 1) mf1_load<true, FULL>(p, blob, gl, 1, bb, 0.f);
  load_cols(p, st, L, a, cg);
  const int nc = L.nrows;
  const bool live = r < nc;
  const int col = live ? r : 0;
  auto math = [&](const MxCols& m, int s, int s_local, const MfBuf& b) {
    const int SC = FULL ? 16 : min(16, C1 - 16 * s);
    auto step = [&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      u32x4 b0, b1, ga, ua;
      uint32_t sb, sg, su;
      mx8_frag(m, col, s_local, kb, q, b0, b1, sb);
      mx8_a<FULL>(b.q[0][kb], b.s[0], SC, kb, q, ga, sg);
      mx8_a<FULL>(b.q[1][kb], b.s[1], SC, kb, q, ua, su);
      ag = mfma_fp4_mx8<kb>(ga, b0, b1, sg, sb, ag);
      au = mfma_fp4_mx8<kb>(ua, b0, b1, su, sb, au);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
  };
  const int XQ = S * 512 + 16;
  if (nc * (XQ + S * 16) <= MF_STAGE_BYTES) {
    const MxCols m{mfb, XQ, nc * XQ, S};
    for (int i = tidx(); i < nc * S * 16; i += 256) {
      const int c = i / (S * 16), b = i - c * (S * 16);
      float v[32];
      x_block(p, L.slot[c] / p.k, b, v);
      u32x4 c0, c1;
      const uint32_t sc = mx8_block(v, c0, c1);
      mx8_put(m, c, b, 0, c0, c1, 32 * b < p.H ? sc : 127u);
    }
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
      math(m, s, s, ba);
      if (s + 2 < S) mf1_load<true, FULL>(p, blob, gl, s + 2, ba, ag[0] + au[0]);
      if (s + 1 < S) {
        math(m, s + 1, s + 1, bb);
        if (s + 3 < S) mf1_load<true, FULL>(p, blob, gl, s + 3, bb, ag[0] + au[0]);
      }
    }
  } else {
    // two buffers of one segment each: 16 columns x (512 + 16) code bytes, then 16 x 16 scale bytes
    constexpr int XQS = 512 + 16, BUF = MF_COLS * XQS + MF_COLS * 16;
    auto buf = [&](int s) { return MxCols{mfb + (s & 1) * BUF, XQS, MF_COLS * XQS, 1}; };
    const int c_me = tidx() >> 4, j_me = tidx() & 15;  // this thread's (column, block) of a segment
    auto quant_put = [&](int s, const float (&v)[32]) {
      u32x4 c0, c1;
      const uint32_t sc = mx8_block(v, c0, c1);
      mx8_put(buf(s), c_me, 16 * s + j_me, s, c0, c1, 32 * (16 * s + j_me) < p.H ? sc : 127u);
    };
    {
      float v[32];
      x_block(p, c_me < nc ? L.slot[c_me] / p.k : 0, j_me, v);
      if (c_me < nc) quant_put(0, v);
    }
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ss = s + h;
        if (ss < S) {
          float v[32];
          if (ss + 1 < S) x_block(p, c_me < nc ? L.slot[c_me] / p.k : 0, 16 * (ss + 1) + j_me, v);
          MfBuf& b = h ? bb : ba;
          math(buf(ss), ss, 0, b);
          if (ss + 2 < S) mf1_load<true, FULL>(p, blob, gl, ss + 2, b, ag[0] + au[0]);
          if (ss + 1 < S && c_me < nc) quant_put(ss + 1, v);
          __syncthreads();
        }
      }
    }
  }
  // h = silu(gate) * up: rows 16 g + 4 q + i of column r, as fp32 (one 16-byte coherent store)
  float* hout = reinterpret_cast<float*>(p.hr_p);
  const int n0 = 16 * g + 4 * q;
  if (n0 < N && r < nc) {
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_f(ag[i]) * au[i];
    st_f32x4_coh(hout, (size_t)L.slot[r] * N + n0, hv);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every lane's h stores have completed
  __syncthreads();
  if (tidx() == 0) st_coh(hflag_at(p, a, cg, t), make_pair(1u, st.tag));
}

// FC2 of rows [512 t, 512 t + 512) of H of routed expert a, column group cg,
// with the SwiGLU output quantised to MXFP8: all of K (I) for every column is
// staged once (the envelope of the variant), then one pass per (128-row
// tile, segment), one scaled MFMA per tile and step.
template <bool FULL>
__device__ __forceinline__ void mx_fc2_unit(const LayerParams& p, WgState& st, Lds& L, char* mfb, int a, int cg,
                                            int t) {
  const int nc = unit_ncols(p, st, a, cg);
  const int w = tidx() >> 6, lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int K = p.I, G = p.H / 16;
  const uint8_t* down = p.experts + (size_t)st.s_active[a] * p.blob_bytes + (size_t)2 * p.I * (p.H / 32) * 17;
  const int C2 = K / 32, S = (C2 + 15) / 16;
  const int MT = min(MF_MT2, (G - 8 * MF_MT2 * t + 7) / 8);
  auto groups = [&](int mt, int (&gt)[2]) {
    gt[0] = min(8 * (MF_MT2 * t + mt) + w, G - 1);
    gt[1] = min(8 * (MF_MT2 * t + mt) + w + 4, G - 1);
  };
  MfBuf ba, bb;
  const int P = MT * S;
  {
    int gt[2];
    groups(0, gt);
    mf2_load<true, FULL>(p, down, gt, 0, ba, 0.f);
    if (P > 1) {
      groups(1 / S, gt);
      mf2_load<true, FULL>(p, down, gt, 1 % S, bb, 0.f);
    }
  }
  load_cols(p, st, L, a, cg);
  {  // wait until every FC1 tile of this column group has published its h
    const int ntile = (K + MF_NT1 - 1) / MF_NT1;
    bool ok = true;
    if (tidx() < ntile) {
      uint64_t f[1];
      const int ti = tidx();
      ok = poll_pairs<1>(hflag_at(p, a, cg, 0), 1, [&](int) { return ti; }, st.tag, f, SPIN_LIMIT,
                         p.ctrl + CTRL_ERR);
    }
    if (!ok) set_error(p);
  }
  const int XQ = S * 512 + 16;
  const MxCols m{mfb, XQ, nc * XQ, S};
  const float* hsrc = reinterpret_cast<const float*>(p.hr_p);
  __syncthreads();
  for (int i = tidx(); i < nc * S * 16; i += 256) {
    const int c = i / (S * 16), b = i - c * (S * 16);
    float v[32];
    if (32 * b < K) {
      const uint64_t* src = reinterpret_cast<const uint64_t*>(hsrc + (size_t)L.slot[c] * K + 32 * b);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint64_t pr = ld_coh(src + j);
        v[2 * j] = __uint_as_float((uint32_t)pr);
        v[2 * j + 1] = __uint_as_float((uint32_t)(pr >> 32));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = 0.0f;
    }
    u32x4 c0, c1;
    const uint32_t sc = mx8_block(v, c0, c1);
    mx8_put(m, c, b, 0, c0, c1, 32 * b < K ? sc : 127u);
  }
  __syncthreads();
  const int col = r < nc ? r : 0;
  const f32x4 zero4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc[2] = {zero4, zero4};
  for (int pp = 0; pp < P; pp += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ps = pp + h;
      if (ps < P) {
        MfBuf& b = h ? bb : ba;
        const int mt = ps / S, sg = ps - mt * S;
        const int SC = FULL ? 16 : min(16, C2 - 16 * sg);
        auto step = [&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
          u32x4 b0, b1;
          uint32_t sb;
          mx8_frag(m, col, sg, kb, q, b0, b1, sb);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            u32x4 av;
            uint32_t sa;
            mx8_a<FULL>(b.q[tt][kb], b.s[tt], SC, kb, q, av, sa);
            acc[tt] = mfma_fp4_mx8<kb>(av, b0, b1, sa, sb, acc[tt]);
          }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        if (ps + 2 < P) {
          int gt[2];
          groups((ps + 2) / S, gt);
          mf2_load<true, FULL>(p, down, gt, (ps + 2) % S, b, acc[0][0] + acc[1][0]);
        }
        if (sg == S - 1) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int gg = 8 * (MF_MT2 * t + mt) + w + 4 * tt;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float a, b;
              regroup_rows(acc[tt], h, a, b);
              if (r < nc && gg < G)
                st_pair2_f32(p.or_p, (size_t)L.slot[r] * p.H + 16 * gg + 8 * h + 2 * q, a, b, st.tag);
            }
          }
          acc[0] = zero4;
          acc[1] = zero4;
        }
      }
    }
  }
}

// ---- the kernel ------------------------------------------------------------------

// FULL: the layer's shape makes every weight-stream segment and FC2 row group
// complete (H % 7168 == 0, I % 1536 == 0, Is % 384 == 0), so the streams need
// no clamping or masking.
template <int RG, bool FULL, int TPL, bool MX8>
__global__ __launch_bounds__(256, 2) void k_moe_layer(LayerParams p) {
  extern __shared__ u32x4 lds_raw[];
  u32x4* xs = lds_raw;
  u32x4* hs = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(lds_raw) + p.lds_h_off);
  constexpr bool MF = RG > 1;  // batch > 1: routed and shared experts on the matrix cores
  char* mfb = reinterpret_cast<char*>(lds_raw);  // MFMA staging (aliases the x region: one unit at a time)
  int* sched_lds = reinterpret_cast<int*>(reinterpret_cast<char*>(lds_raw) + p.lds_sched_off);
  __shared__ Lds L;
  // Every thread loads the call epoch itself (no barrier before the first
  // unit).  A tag computed lazily at its first use, after the first unit's
  // loads, measured no faster: the wait it saves hides in the set-up code.
  const uint32_t epoch = ld_coh(p.ctrl + CTRL_EPOCH);
  const uint32_t tag = (epoch == 0xFFFFFFFFu) ? 1u : epoch + 1u;  // never 0: a cleared workspace holds no valid pair
  WgState st{false, false, 0, tag, nullptr, nullptr, nullptr, nullptr};
  // The first units (router, routing, shared FC1) go by workgroup index, so
  // the launch ramp does not queue on the head counter.
  int u = (int)blockIdx.x < p.n_static ? (int)blockIdx.x : -1;
  unsigned nxt = 0;
  if (u < 0) {
    if (threadIdx.x == 0) L.next = queue_unit(p, claim_next(p));
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(L.next);
  }
  int it = 0;
  if constexpr (!MF && FULL) {
    // Batch 1: a workgroup whose first unit is a router unit (by workgroup
    // index) runs it ahead of the unit loop, so the router rows -- the start
    // of the layer's critical path -- are requested before the loop's set-up
    // code (what the compiler hoists out of the loop for every unit type,
    // ~2 us at launch) instead of after it: router units 7 -> 6 us, the layer
    // ~1 us faster.  Running the shared-FC1 workgroups' first units ahead too
    // measured slower: their reads then compete with the router's from the
    // first microsecond.
    if (u >= 0 && u < p.n_rt) {
      if (threadIdx.x == 0) nxt = claim_next(p);
      router_unit(p, st, u);
      if (threadIdx.x == 0) L.nxt[0] = queue_unit(p, nxt);
      __syncthreads();
      u = __builtin_amdgcn_readfirstlane(L.nxt[0]);
      it = 1;
    }
  }
  for (;;) {
    // Batch > 1 (and partial tiles): the shape is taken through an empty asm
    // at every unit, so the compiler computes what each unit derives from it
    // inside that unit instead of hoisting all of it, for every unit type, to
    // the kernel's start (where it held every workgroup ~2 us at launch and
    // spilled registers): no vector registers spill then, and batch 8 / 64
    // run ~1% faster.  The batch-1 kernel at full tiles keeps the hoisting:
    // there recomputing per unit costs more than the set-up saves (78.5
    // against 75 us a layer).
    if constexpr (MF || !FULL) asm volatile("" : "+s"(p.H), "+s"(p.I), "+s"(p.E), "+s"(p.k), "+s"(p.Is), "+s"(p.B));
    if (p.n_total > 0 && u >= p.n_total) break;  // batch 1: past the end, claim nothing more
    // the next unit is claimed now; its index is only needed after this one
    if (threadIdx.x == 0) nxt = claim_next(p);
    int rel = u;
    if (rel < p.n_rt) {
      if constexpr (MF) {
        if (p.rt_f64) router_f64_unit(p, st, mfb, rel);
        else router_mf_unit(p, st, L, rel);
      } else {
        router_unit(p, st, rel);
      }
    } else if ((rel -= p.n_rt) < p.n_ro) {
      routing_unit<TPL>(p, st, L, reinterpret_cast<int*>(xs), rel);
    } else if ((rel -= p.n_ro) < p.n_sch) {
      __syncthreads();
      build_schedule<MF>(p, st, reinterpret_cast<int*>(xs), L.wtot);
      st.x_cached = false;
    } else if ((rel -= p.n_sch) < p.n_s1) {
      if constexpr (MF) mf_sh1_unit<FULL>(p, st, L, mfb, rel / p.mf_t1s, rel % p.mf_t1s);
      else shared_fc1_unit<RG, FULL>(p, st, L, xs, rel);
    } else {
      rel -= p.n_s1;
      if (!st.route_seen) {
        __syncthreads();
        cache_schedule<MF>(p, st, L, sched_lds);
      }
      const int U = st.U;
      if constexpr (MF) {
        const int NCG = st.s_cg_off[U];  // column groups of all active experts
        if (rel < NCG * p.mf_t1) {
          const int gc = rel / p.mf_t1, ae = find_expert(st, gc);
          if constexpr (MX8) mx_fc1_unit<FULL>(p, st, L, mfb, ae, min(gc - st.s_cg_off[ae], 3), rel % p.mf_t1);
          else mf_fc1_unit<true, FULL>(p, st, L, mfb, ae, min(gc - st.s_cg_off[ae], 3), rel % p.mf_t1);
        } else if ((rel -= NCG * p.mf_t1) < p.n_s2) {
          mf_fc2_unit<false, FULL>(p, st, L, mfb, -1, rel / p.mf_t2s, rel % p.mf_t2s);
        } else if ((rel -= p.n_s2) < NCG * p.mf_t2) {
          const int gc = rel / p.mf_t2, ae = find_expert(st, gc);
          if constexpr (MX8) mx_fc2_unit<FULL>(p, st, L, mfb, ae, min(gc - st.s_cg_off[ae], 3), rel % p.mf_t2);
          else mf_fc2_unit<true, FULL>(p, st, L, mfb, ae, min(gc - st.s_cg_off[ae], 3), rel % p.mf_t2);
        } else if ((rel -= NCG * p.mf_t2) < p.B * p.n_tile) {
          combine_unit<MF>(p, st, L, rel / p.n_tile, rel % p.n_tile, nxt);
        } else {
          break;
        }
      } else {
        if (rel < U * p.T1) {
          // a run of routed FC1 units, ending with the loop's protocol done
          // for each; u is then the next unit, claimed but not started
          u = routed_fc1_run<FULL>(p, st, L, xs, u, it, nxt);
          continue;
        } else if ((rel -= U * p.T1) < p.n_s2) {
          shared_fc2_unit<RG, FULL>(p, st, L, hs, rel);
        } else if ((rel -= p.n_s2) < U * p.n_r2) {
          // a run of routed FC2 units, as for FC1
          u = routed_fc2_run<FULL>(p, st, L, hs, u, it, nxt);
          continue;
        } else if ((rel -= U * p.n_r2) < p.B * p.n_tile) {
          combine_unit<MF>(p, st, L, rel / p.n_tile, rel % p.n_tile, nxt);
        } else {
          break;
        }
      }
    }
    // One barrier per unit: it ends this unit's use of LDS and publishes the
    // next index.  The index word alternates between two slots, so thread 0
    // cannot overwrite one that a slower wave has yet to read.
    if (threadIdx.x == 0) L.nxt[it & 1] = queue_unit(p, nxt);
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(L.nxt[it & 1]);  // uniform: unit arithmetic stays scalar
    ++it;
  }
  // Exit: the last workgroup to count itself out resets the queue and
  // advances the epoch (every other workgroup has made its final claim and
  // read the epoch long before).  At batch 1 most count out during their
  // last unit (count_out_early), the rest here.
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = st.exited ? st.exit_old
                                   : __hip_atomic_fetch_add(p.ctrl + CTRL_EXIT, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      st_coh(p.ctrl + CTRL_HEAD, 0u);
      st_coh(p.ctrl + CTRL_HEAD1, 0u);
      st_coh(p.ctrl + CTRL_EXIT, 0u);
      st_coh(p.ctrl + CTRL_EPOCH, st.tag);  // the next call's tag is this one's + 1
    }
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

// mf: the matrix-core kernel (every batch > 1, and the FP4 x MXFP8 variant
// at every batch); else the batch-1 kernel.
static LaunchShape launch_shape(int H, int I, int E, int k, int Is, int B, bool mf) {
  LaunchShape s;
  s.rg = mf ? 4 : 1;
  // FULL: every packed tile holds 16 blocks (H, I multiples of 512), every
  // bf16 shared-expert stream segment is complete, and every unit's rows exist
  s.full = (H % 512 == 0) && (I % 512 == 0) && (H % (32 * 8 * CPL1) == 0) && (Is % (8 * 8 * CPL2) == 0) &&
           (Is % NTS1 == 0) && (H % NTR2 == 0) && (H % NTS2 == 0);
  if (mf) s.full = (H % 512 == 0) && (I % 512 == 0);  // the MFMA path: every packed tile is complete
  s.xstride = ((H / 8 + 7) / 8) * 8;
  int K2 = I > Is ? I : Is;
  s.hstride = ((K2 / 4 + 7) / 8) * 8;  // fp32 h rows (shared expert FC2)
  if (!mf && 2 * h_lo_offset(I) > s.hstride) s.hstride = 2 * h_lo_offset(I);  // bf16 hi + lo rows (routed FC2)
  size_t x_bytes = mf ? 0 : (size_t)s.rg * s.xstride * 16;  // matrix-core kernel: no x rows in LDS
  // routing reuses this region: top-k survivors and slots, then the
  // schedule's row sets (8 bytes an expert), starts (E) and slot ids (B*k)
  size_t keys_bytes = (size_t)topk_lds_words(E <= 1024 ? 4 : 16) * 4, cnt_bytes = (size_t)(3 * E + B * k) * 4;
  size_t sched_bytes = keys_bytes > cnt_bytes ? keys_bytes : cnt_bytes;
  size_t xr = x_bytes > sched_bytes ? x_bytes : sched_bytes;
  // batch > 1: the MFMA staging buffers (two 16-column segments) alias this
  // region, and no h rows are staged
  const size_t mf_bytes = MF_STAGE_BYTES;
  if (mf && mf_bytes > xr) xr = mf_bytes;
  xr = align256(xr);
  s.lds_h_off = (int)xr;
  // batch 1: two h rows (routed FC2 units alternate between them)
  size_t hr = mf ? 0 : align256((size_t)2 * s.hstride * 16);
  s.lds_sched_off = (int)(xr + hr);
  const size_t slots = (size_t)B * k, umax = slots < (size_t)E ? slots : (size_t)E;
  s.lds = xr + hr + align256(4 * (3 * umax + 2 + slots));
  return s;
}

static std::atomic<int> g_grid_cap{0};
void set_layer_grid_cap(int n) { g_grid_cap.store(n); }

template <int RG, bool FULL, int TPL, bool MX8 = false>
static hipError_t launch_t(LayerParams p, size_t lds, hipStream_t s) {
  auto kern = k_moe_layer<RG, FULL, TPL, MX8>;
  static thread_local int cached[2] = {-1, -1};  // (lds bytes, blocks per CU)
  int per_cu = 0;
  if (cached[0] == (int)lds) {
    per_cu = cached[1];
  } else {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess || per_cu < 1) per_cu = 1;
    cached[0] = (int)lds;
    cached[1] = per_cu;
  }
  const int cap = g_grid_cap.load();
  const int grid = cap > 0 ? std::min(cap, num_cus() * per_cu) : num_cus() * per_cu;
  p.n_static = std::min(grid, p.n_front);
  p.nq = grid >= 16 ? 2 : 1;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

bool mx8_supported(int H, int I) {
  // FC2 stages all of I for 16 columns at once (codes and scales)
  const int S2 = (I / 32 + 15) / 16;
  return MF_COLS * (S2 * 512 + 16 + S2 * 16) <= MF_STAGE_BYTES && H > 0;
}

hipError_t launch_layer(const LayerArgs& a, const float* bias, const uint16_t* wr, int32_t* idx, hipStream_t s,
                        bool mx8) {
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
  p.logits_p = a.ws.logits_p;
  p.idx_p = a.ws.idx_p;
  p.gate_p = a.ws.gate_p;
  p.active = a.ws.sched.active;
  p.row_off = a.ws.sched.row_off;
  p.rows = a.ws.sched.rows;
  p.hs_p = a.ws.hs_p;
  p.hr_p = a.ws.hr_p;
  p.os_p = a.ws.os_p;
  p.or_p = a.ws.or_p;
  p.ctrl = a.ws.ctrl;
  p.umax = a.ws.umax;
  const bool mf = a.B > 1 || mx8;
  const LaunchShape sh = launch_shape(a.H, a.I, a.E, a.k, a.Is, a.B, mf);
  p.rt_f64 = a.B > RT_F64_MIN_BATCH;
  p.n_rt_e = p.rt_f64 ? (a.E + 15) / 16 : (a.E + 3) / 4;  // router units per row block: 16 or 4 experts each
  p.xstride = sh.xstride;
  p.hstride = sh.hstride;
  p.n_rb = p.rt_f64 ? (a.B + 15) / 16 : (mf ? (a.B + 7) / 8 : 1);  // row blocks: 16 rows, 8 rows, or the one row
  p.n_rt = p.n_rt_e * p.n_rb;
  p.n_ro = a.B;
  p.n_sch = mf ? 1 : 0;
  p.n_s1 = a.Is > 0 ? (a.Is + NTS1 - 1) / NTS1 : 0;
  p.T1 = (a.I + NT1 - 1) / NT1;
  p.n_s2 = a.Is > 0 ? (a.H + NTS2 - 1) / NTS2 : 0;
  p.n_r2 = (a.H + NTR2 - 1) / NTR2;
  p.n_tile = (a.H + NT2 - 1) / NT2;
  p.mf_t1 = (a.I + MF_NT1 - 1) / MF_NT1;
  p.mf_t1s = (a.Is + 15) / 16;
  p.mf_t2 = (a.H + MF_NT2 - 1) / MF_NT2;
  p.mf_t2s = (a.H + 127) / 128;
  p.mf_cgs = (a.B + MF_COLS - 1) / MF_COLS;
  if (mf) {  // MFMA path: shared expert units per column group
    p.n_s1 = a.Is > 0 ? p.mf_cgs * p.mf_t1s : 0;
    p.n_s2 = a.Is > 0 ? p.mf_cgs * p.mf_t2s : 0;
  }
  p.cg_off = a.ws.sched.cg_off;
  p.hflag = a.ws.hflag;
  p.hflag_tiles = a.ws.hflag_tiles;
  p.n_front = p.n_rt + p.n_ro + p.n_sch + p.n_s1;
  // batch 1: the one row picks k distinct experts, so the queue's length is known here
  p.n_total = mf ? 0 : p.n_front + a.k * p.T1 + p.n_s2 + a.k * p.n_r2 + a.B * p.n_tile;
  p.lds_h_off = sh.lds_h_off;
  p.lds_sched_off = sh.lds_sched_off;
  // top-k keys per lane in the first selection phase: E <= 1024 -> 4, else 16
  if (mx8) {
    if (a.E <= 1024) return sh.full ? launch_t<4, true, 4, true>(p, sh.lds, s) : launch_t<4, false, 4, true>(p, sh.lds, s);
    return sh.full ? launch_t<4, true, 16, true>(p, sh.lds, s) : launch_t<4, false, 16, true>(p, sh.lds, s);
  }
  if (a.E <= 1024) {
    if (sh.rg == 1) return sh.full ? launch_t<1, true, 4>(p, sh.lds, s) : launch_t<1, false, 4>(p, sh.lds, s);
    return sh.full ? launch_t<4, true, 4>(p, sh.lds, s) : launch_t<4, false, 4>(p, sh.lds, s);
  }
  if (sh.rg == 1) return sh.full ? launch_t<1, true, 16>(p, sh.lds, s) : launch_t<1, false, 16>(p, sh.lds, s);
  return sh.full ? launch_t<4, true, 16>(p, sh.lds, s) : launch_t<4, false, 16>(p, sh.lds, s);
}

}  // namespace moe
