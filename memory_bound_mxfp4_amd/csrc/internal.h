// internal.h -- host-side launchers and the workspace layout shared by the
// library's translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mxfp4.h"

namespace moe {

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Offsets of the six sub-arrays of an expert blob (layout documented in
// moe_mxfp4.h): gate codes, up codes, down codes, gate/up/down scales.
struct BlobLayout {
  size_t off[6];
  size_t bytes;
};
BlobLayout blob_layout(int H, int I);

// Expert-gathered schedule built on the device from the top-k indices.
//   active[U]         the U distinct experts any row selected, ascending
//   row_off[U+1]      rows of active expert a are rows[row_off[a] .. row_off[a+1])
//   rows[B*k]         slot ids s = b * k + j
//   cg_off[U+1]       batch > 1: active expert a has column groups (up to 16
//                     of its rows each) cg_off[a] .. cg_off[a+1]
struct Sched {
  int* cg_off;
  int* active;
  int* row_off;
  int* rows;
};

// Control block at the start of the workspace: uint32 words, each counter on
// a 128-byte line of its own (line i starts at word CTRL_STRIDE * i) so that
// polls of different counters never share a cache line.
//   line 0, word 0   head of work queue 0           (zero between calls)
//   line 0, word 7   sticky error word (byte offset MOE_WS_STATUS_OFFSET)
//   line 1           workgroups that have exited    (zero between calls)
//   line 2           call epoch: bumped by the last workgroup of every call
//   line 3           schedule-ready word pair (batch > 1): U | tag << 32
//   line 4           head of work queue 1           (zero between calls)
// Data handed between workgroups inside a call travels as 8-byte pairs
// (32-bit value | 32-bit tag << 32), tag = epoch + 1 of the call, written and
// read with single 8-byte coherent accesses: a consumer polls the data itself
// until every pair carries its call's tag, so no producer ever has to drain
// its stores and bump a counter.
constexpr int CTRL_STRIDE = 32;
constexpr int CTRL_HEAD = 0, CTRL_ERR = 7, CTRL_EXIT = 1 * CTRL_STRIDE, CTRL_EPOCH = 2 * CTRL_STRIDE,
              CTRL_READY = 3 * CTRL_STRIDE, CTRL_HEAD1 = 4 * CTRL_STRIDE, CTRL_WORDS = 5 * CTRL_STRIDE;

// Workspace of moe_decode_layer.
struct Workspace {
  unsigned* ctrl;
  int umax;
  uint64_t* logits_p;  // [B][E]      router logits
  uint64_t* idx_p;     // [B*k]       expert of slot s = b*k + j
  uint64_t* gate_p;    // [B*k]       gate of slot s
  Sched sched;         // batch > 1: expert-gathered schedule (plain ints, published by READY)
  uint64_t* hs_p;      // [B][Is]     shared-expert SwiGLU output
  uint64_t* hr_p;      // [B*k][I]    routed SwiGLU output, by slot
  uint64_t* os_p;      // [B][H]      shared-expert output
  uint64_t* or_p;      // [B*k][H]    routed expert outputs, by slot
  uint64_t* hflag;     // batch > 1: [umax + 1][4][hflag_tiles] "FC1 tile done" tags
  int hflag_tiles;
  size_t bytes;
};
Workspace ws_layout(void* base, int H, int I, int E, int k, int Is, int B);

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_router_logits(const uint16_t* x, int B, int H, const uint16_t* wr, const float* bias, int E,
                                float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int B, int E, int k, int32_t* idx, float* gate, hipStream_t s);

struct LayerArgs {
  int H, I, E, k, Is, B;
  const uint16_t* x;
  const uint16_t *sg, *su, *sd;
  const uint8_t* experts;
  BlobLayout blob;
  const float* gate;
  Workspace ws;
  float* residual;
};
// mx8: the routed experts' FP4 x MXFP8 variant (the matrix-core kernel at
// every batch); mx8_supported: the shapes that variant covers.
hipError_t launch_layer(const LayerArgs& a, const float* bias, const uint16_t* wr, int32_t* idx, hipStream_t s,
                        bool mx8 = false);
bool mx8_supported(int H, int I);
// Cap on the layer kernel's grid (0: two workgroups per compute unit).
void set_layer_grid_cap(int n);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_pack_experts(uint8_t* experts, int E, int H, int I, uint8_t* scratch, bool to_packed,
                               hipStream_t s);

hipError_t launch_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, const void* x, bool x_f32,
                             int B, float* y, hipStream_t s);

hipError_t launch_rmsnorm(const float* in, int B, int H, float eps, uint16_t* out, hipStream_t s);
hipError_t launch_dense_gemv(const uint16_t* w, int N, int K, const uint16_t* x, int B, uint16_t* y, hipStream_t s);
hipError_t launch_residual_add(float* h, const uint16_t* t, int B, int H, hipStream_t s);
hipError_t launch_residual_add_rmsnorm(float* h, const uint16_t* t, int B, int H, float eps, uint16_t* out,
                                       hipStream_t s);

hipError_t launch_stream_read(const void* buf, size_t bytes, int blocks_per_cu, uint32_t* sink, hipStream_t s);
hipError_t launch_prefetch(const moe_range* ranges, int n, int blocks, hipStream_t s);

int num_cus();

}  // namespace moe
