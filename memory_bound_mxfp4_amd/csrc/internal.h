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
//   n_active          number U of distinct experts any row selected
//   active[U]         their ids, ascending
//   row_off[U+1]      rows of active expert a are rows[row_off[a] .. row_off[a+1])
//   rows[B*k]         slot ids s = b * k + j
struct Sched {
  int* n_active;
  int* active;
  int* row_off;
  int* rows;
};

// Control block at the start of the workspace: counters of uint32, each on a
// 128-byte line of its own (counter i at word CTRL_STRIDE * i), so that polls
// of different counters never share a cache line.  Zeroed once by
// moe_workspace_init; every layer call leaves it zeroed again, except the
// sticky error word.
constexpr int CTRL_STRIDE = 32;
enum {
  CTRL_HEAD = 0,     // work-queue head
  CTRL_ROUTER = 1,   // (unused)
  CTRL_ROUTING = 2,  // rows routed (batch > 1)
  CTRL_READY = 3,    // schedule published (0/1, batch > 1)
  CTRL_U = 4,        // number of distinct experts (batch > 1)
  CTRL_SH1 = 5,      // shared FC1 units done
  CTRL_EXIT = 6,     // workgroups that have exited
  CTRL_ERR = 7,      // sticky: a bounded wait expired (byte offset 28: in the first line)
  CTRL_FC1 = 8       // first of the per-launch arrays below
};
// Counter lines after CTRL_FC1: [umax] routed FC1 units done per active expert
// (per slot at batch 1), [T2] FC2 tile tickets, [MOE_MAX_BATCH] router
// row-block tickets, [MOE_MAX_TOPK] published expert + 1 of each slot (batch 1).
__host__ __device__ constexpr int ctrl_lines(int umax, int T2) {
  return CTRL_FC1 + umax + T2 + MOE_MAX_BATCH + MOE_MAX_TOPK;
}
// Word index of counter i (the error word stays at word 7 of the first line).
__host__ __device__ constexpr int ctrl_word(int i) { return i == CTRL_ERR ? CTRL_ERR : i * CTRL_STRIDE; }

// Workspace of moe_decode_layer.
struct Workspace {
  unsigned* ctrl;
  int ctrl_words;
  int umax;
  float* logits;    // [B][E]
  Sched sched;
  float* h_shared;  // [B][Is]
  float* h_routed;  // [B*k][I]
  float* o_shared;  // [B][H]
  float* o_routed;  // [B*k][H]
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
hipError_t launch_layer(const LayerArgs& a, const float* bias, const uint16_t* wr, int32_t* idx, hipStream_t s);
int layer_tiles_fc2(int H);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, const void* x, bool x_f32,
                             int B, float* y, hipStream_t s);

hipError_t launch_rmsnorm(const float* in, int B, int H, float eps, uint16_t* out, hipStream_t s);
hipError_t launch_dense_gemv(const uint16_t* w, int N, int K, const uint16_t* x, int B, uint16_t* y, hipStream_t s);
hipError_t launch_residual_add(float* h, const uint16_t* t, int B, int H, hipStream_t s);

int num_cus();

}  // namespace moe
