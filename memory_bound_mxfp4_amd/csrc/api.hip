// api.hip -- the C ABI of libmoe_mxfp4.so: argument validation, workspace
// layout and kernel launches.  Semantics are documented in moe_mxfp4.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"
#include "moe_mxfp4.h"

namespace moe {

BlobLayout blob_layout(int H, int I) {
  size_t h = (size_t)H, i = (size_t)I;
  size_t sz[6] = {i * h / 2, i * h / 2, h * i / 2, i * h / 32, i * h / 32, h * i / 32};
  BlobLayout L;
  size_t o = 0;
  for (int m = 0; m < 6; ++m) {
    L.off[m] = o;
    o += align256(sz[m]);
  }
  L.bytes = o;
  return L;
}

Workspace ws_layout(void* base, int H, int I, int E, int k, int Is, int B) {
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + o : nullptr;
    o += align256(bytes);
    return r;
  };
  Workspace w;
  const size_t slots = (size_t)B * k;
  const size_t umax = slots < (size_t)E ? slots : (size_t)E;
  w.umax = (int)umax;
  w.ctrl = reinterpret_cast<unsigned*>(take(sizeof(unsigned) * CTRL_WORDS));
  w.logits_p = reinterpret_cast<uint64_t*>(take(8 * (size_t)B * E));
  w.idx_p = reinterpret_cast<uint64_t*>(take(8 * slots));
  w.gate_p = reinterpret_cast<uint64_t*>(take(8 * slots));
  w.sched.active = reinterpret_cast<int*>(take(sizeof(int) * umax));
  w.sched.row_off = reinterpret_cast<int*>(take(sizeof(int) * (umax + 1)));
  w.sched.rows = reinterpret_cast<int*>(take(sizeof(int) * slots));
  w.hs_p = reinterpret_cast<uint64_t*>(take(8 * (size_t)B * (Is > 0 ? Is : 1)));
  w.hr_p = reinterpret_cast<uint64_t*>(take(8 * slots * I));
  w.os_p = reinterpret_cast<uint64_t*>(take(8 * (size_t)B * H));
  w.or_p = reinterpret_cast<uint64_t*>(take(8 * slots * H));
  w.sched.cg_off = reinterpret_cast<int*>(take(sizeof(int) * (umax + 1)));
  const int n1 = I > Is ? I : Is;
  w.hflag_tiles = (n1 + 15) / 16;  // routed FC1 flags per 64-row tile, shared ones per 16-row group
  w.hflag = reinterpret_cast<uint64_t*>(take(8 * (umax + 1) * 4 * (size_t)w.hflag_tiles));
  w.bytes = o;
  return w;
}

int num_cus() {
  static std::atomic<int> cached{0};
  int v = cached.load();
  if (v > 0) return v;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached.store(n);
  return n;
}

}  // namespace moe

using namespace moe;

static inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static moe_status check_layer(const moe_layer_weights* w, int batch) {
  if (!w) return MOE_ERR_INVALID_ARGUMENT;
  const int H = w->hidden, I = w->inter, E = w->num_experts, k = w->top_k, Is = w->shared_inter;
  if (H <= 0 || I <= 0 || E <= 0 || k <= 0 || Is < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 32 || I % 32 || Is % 8) return MOE_ERR_INVALID_ARGUMENT;
  if (batch < 1 || batch > MOE_MAX_BATCH) return MOE_ERR_INVALID_ARGUMENT;
  if (k > E || k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARGUMENT;
  if (!w->router_w || !w->experts) return MOE_ERR_INVALID_ARGUMENT;
  if (Is > 0 && (!w->shared_gate || !w->shared_up || !w->shared_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (Is == 0 && (w->shared_gate || w->shared_up || w->shared_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (w->expert_layout != MOE_EXPERTS_CANONICAL && w->expert_layout != MOE_EXPERTS_PACKED)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(w->router_w, 16) || !aligned(w->experts, 256) || (w->router_bias && !aligned(w->router_bias, 4)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (Is > 0 && (!aligned(w->shared_gate, 16) || !aligned(w->shared_up, 16) || !aligned(w->shared_down, 16)))
    return MOE_ERR_INVALID_ARGUMENT;
  // kernel envelope: activation rows staged in 64 KB of LDS, keys per lane
  if (H > 16384 || I > 16384 || Is > 16384 || E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

extern "C" {

size_t moe_expert_bytes(int hidden, int inter) {
  if (hidden <= 0 || inter <= 0 || hidden % 32 || inter % 32) return 0;
  return blob_layout(hidden, inter).bytes;
}

moe_status moe_workspace_size(const moe_layer_weights* w, int batch, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_layer(w, batch);
  if (st != MOE_OK) return st;
  *bytes = ws_layout(nullptr, w->hidden, w->inter, w->num_experts, w->top_k, w->shared_inter, batch).bytes;
  return MOE_OK;
}

size_t moe_router_workspace_size(int batch, int num_experts) {
  if (batch < 1 || num_experts < 1) return 0;
  return align256(sizeof(float) * (size_t)batch * num_experts);
}

moe_status router_topk(const uint16_t* x, int batch, int hidden, const uint16_t* router_w, const float* bias,
                       int num_experts, int top_k, int32_t* topk_idx, float* topk_gate, float* logits, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!x || !router_w || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARGUMENT;
  if (batch < 1 || batch > MOE_MAX_BATCH || hidden <= 0 || hidden % 32 || num_experts < 1 || top_k < 1 ||
      top_k > num_experts || top_k > MOE_MAX_TOPK)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(router_w, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (hidden > 16384 || num_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  float* lg = logits;
  if (!lg) {
    if (!ws) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < moe_router_workspace_size(batch, num_experts)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    lg = static_cast<float*>(ws);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_router_logits(x, batch, hidden, router_w, bias, num_experts, lg, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_topk(lg, batch, num_experts, top_k, topk_idx, topk_gate, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status expert_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int n, int k, const void* x,
                             moe_dtype x_dtype, int batch, float* y, void* stream) {
  if (!codes || !scales || !x || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (n < 1 || k < 32 || k % 32 || batch < 1 || batch > MOE_MAX_BATCH) return MOE_ERR_INVALID_ARGUMENT;
  if (x_dtype != MOE_DTYPE_BF16 && x_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 16384) return MOE_ERR_UNSUPPORTED;
  if (launch_gemv_mxfp4(codes, scales, n, k, x, x_dtype == MOE_DTYPE_F32, batch, y, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

}  // extern "C"

// The kernels moe_decode_layer launches, in launch order.
static const char* const kLayerKernels[] = {"k_moe_layer"};
static const int kNumLayerKernels = 1;

static moe_status run_layer(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                            int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, hipStream_t s,
                            void* const* events, bool mx8 = false) {
  moe_status st = check_layer(w, batch);
  if (st != MOE_OK) return st;
  if (mx8 && !mx8_supported(w->hidden, w->inter)) return MOE_ERR_UNSUPPORTED;
  if (!x || !residual || !topk_idx || !topk_gate || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(ws, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (w->expert_layout != MOE_EXPERTS_PACKED) return MOE_ERR_UNSUPPORTED;
  const int H = w->hidden, I = w->inter, E = w->num_experts, k = w->top_k, Is = w->shared_inter;
  Workspace wsl = ws_layout(ws, H, I, E, k, Is, batch);
  if (ws_bytes < wsl.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  LayerArgs a;
  a.H = H;
  a.I = I;
  a.E = E;
  a.k = k;
  a.Is = Is;
  a.B = batch;
  a.x = x;
  a.sg = w->shared_gate;
  a.su = w->shared_up;
  a.sd = w->shared_down;
  a.experts = w->experts;
  a.blob = blob_layout(H, I);
  a.gate = topk_gate;
  a.ws = wsl;
  a.residual = residual;
  int ev = 0;
  auto mark = [&]() {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[ev++]), s) == hipSuccess;
  };
  if (!mark()) return MOE_ERR_HIP;
  if (launch_layer(a, w->router_bias, w->router_w, topk_idx, s, mx8) != hipSuccess || !mark()) return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" {

moe_status moe_decode_layer(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                            int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(w, x, residual, batch, topk_idx, topk_gate, ws, ws_bytes, static_cast<hipStream_t>(stream),
                   nullptr);
}

}  // extern "C"

// ---- the entry point that allocates nothing ---------------------------------
//
// Its workspace is this file-scope device array: every GPU the library runs
// on holds its own copy from the first call until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address of each GPU's copy is looked up once, with that GPU current, and
// only that address is ever handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];  // per device: device address of `scratch`, once set up

// The current device's copy of `scratch`, set up on its first use: address
// looked up, then the whole array cleared by a fill kernel on `s` (the
// control block at its start must begin at zero, and no stale pair may
// carry a tag a later call could take for its own).  That first use must not
// be under stream capture, where the fill would be recorded into the graph.
static moe_status noalloc_scratch(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return MOE_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    if (launch_zero(ptr, MOE_NOALLOC_SCRATCH_BYTES, s) != hipSuccess) return MOE_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

extern "C" {

moe_status moe_decode_layer_noalloc(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                    int32_t* topk_idx, float* topk_gate, uint32_t* status, void* stream) {
  moe_status st = check_layer(w, batch);
  if (st != MOE_OK) return st;
  if (status && !aligned(status, 4)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = ws_layout(nullptr, w->hidden, w->inter, w->num_experts, w->top_k, w->shared_inter, batch).bytes;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!x || !residual || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = noalloc_scratch(s, &ws);
  if (st != MOE_OK) return st;
  st = run_layer(w, x, residual, batch, topk_idx, topk_gate, ws, MOE_NOALLOC_SCRATCH_BYTES, s, nullptr);
  if (st != MOE_OK || !status) return st;
  if (hipMemcpyAsync(status, static_cast<const char*>(ws) + MOE_WS_STATUS_OFFSET, sizeof(uint32_t),
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_decode_layer_mxfp8(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(w, x, residual, batch, topk_idx, topk_gate, ws, ws_bytes, static_cast<hipStream_t>(stream),
                   nullptr, true);
}

int moe_decode_layer_kernel_count(void) { return kNumLayerKernels; }

const char* moe_decode_layer_kernel_name(int i) {
  return (i >= 0 && i < kNumLayerKernels) ? kLayerKernels[i] : nullptr;
}

moe_status moe_decode_layer_timed(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream,
                                  void* const* events, int n_events) {
  if (!events || n_events < kNumLayerKernels + 1) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i <= kNumLayerKernels; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARGUMENT;
  return run_layer(w, x, residual, batch, topk_idx, topk_gate, ws, ws_bytes, static_cast<hipStream_t>(stream),
                   events);
}

static moe_status pack_common(uint8_t* experts, int E, int H, int I, void* scratch, size_t scratch_bytes,
                              void* stream, bool to_packed) {
  if (!experts || !scratch || E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(experts, 256) || !aligned(scratch, 16)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t nb = blob_layout(H, I).bytes;
  if (scratch_bytes < nb) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const uint8_t* sc = static_cast<const uint8_t*>(scratch);
  if (sc < experts + (size_t)E * nb && experts < sc + nb) return MOE_ERR_INVALID_ARGUMENT;  // overlap
  if (launch_pack_experts(experts, E, H, I, static_cast<uint8_t*>(scratch), to_packed,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_pack_experts(uint8_t* experts, int num_experts, int hidden, int inter, void* scratch,
                            size_t scratch_bytes, void* stream) {
  return pack_common(experts, num_experts, hidden, inter, scratch, scratch_bytes, stream, true);
}

moe_status moe_unpack_experts(uint8_t* experts, int num_experts, int hidden, int inter, void* scratch,
                              size_t scratch_bytes, void* stream) {
  return pack_common(experts, num_experts, hidden, inter, scratch, scratch_bytes, stream, false);
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned(ws, 256) || ws_bytes % 16) return MOE_ERR_INVALID_ARGUMENT;
  if (launch_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status, void* stream) {
  if (!ws || !status || !aligned(ws, 256) || !aligned(status, 4) || ws_bytes < sizeof(unsigned) * CTRL_WORDS)
    return MOE_ERR_INVALID_ARGUMENT;
  const char* word = static_cast<const char*>(ws) + MOE_WS_STATUS_OFFSET;
  if (hipMemcpyAsync(status, word, sizeof(uint32_t), hipMemcpyDefault, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_set_max_workgroups(int n) {
  if (n < 0) return MOE_ERR_INVALID_ARGUMENT;
  set_layer_grid_cap(n);
  return MOE_OK;
}

moe_status moe_stream_read_probe(const void* buf, size_t bytes, int blocks_per_cu, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || bytes < 16 || bytes % 16 || blocks_per_cu < 1 || blocks_per_cu > 32)
    return MOE_ERR_INVALID_ARGUMENT;
  if (launch_stream_read(buf, bytes, blocks_per_cu, sink, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_prefetch(const moe_range* ranges, int n_ranges, int blocks, void* stream) {
  if (!ranges || n_ranges < 1 || n_ranges > MOE_PREFETCH_MAX_RANGES || blocks < 1 || blocks > 65536)
    return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < n_ranges; ++i)
    if (!ranges[i].ptr || !aligned(ranges[i].ptr, 16) || ranges[i].bytes % 16) return MOE_ERR_INVALID_ARGUMENT;
  if (launch_prefetch(ranges, n_ranges, blocks, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status rmsnorm_bf16(const float* in, int batch, int hidden, float eps, uint16_t* out, void* stream) {
  if (!in || !out || batch < 1 || batch > MOE_MAX_BATCH || hidden < 1 || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARGUMENT;
  if (launch_rmsnorm(in, batch, hidden, eps, out, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status dense_gemv_bf16(const uint16_t* w, int n, int k, const uint16_t* x, int batch, uint16_t* y,
                           void* stream) {
  if (!w || !x || !y || n < 1 || k < 8 || k % 8 || batch < 1 || batch > MOE_MAX_BATCH) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(w, 16) || !aligned(x, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (k > 32768) return MOE_ERR_UNSUPPORTED;
  if (launch_dense_gemv(w, n, k, x, batch, y, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status residual_add_bf16(float* h, const uint16_t* t, int batch, int hidden, void* stream) {
  if (!h || !t || batch < 1 || batch > MOE_MAX_BATCH || hidden < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (launch_residual_add(h, t, batch, hidden, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status residual_add_rmsnorm_bf16(float* h, const uint16_t* t, int batch, int hidden, float eps, uint16_t* out,
                                     void* stream) {
  if (!h || !t || !out || batch < 1 || batch > MOE_MAX_BATCH || hidden < 1 || !(eps >= 0.0f))
    return MOE_ERR_INVALID_ARGUMENT;
  if (launch_residual_add_rmsnorm(h, t, batch, hidden, eps, out, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

}  // extern "C"
