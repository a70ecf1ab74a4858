/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 mixture-of-experts
 * decode-layer library (libmoe_mxfp4.so).
 *
 * The operation.  One decode step of one mixture-of-experts layer of the kind
 * described in "Kimi K3 on GB300: 13 kernels a layer, and what 842 and 423
 * tokens a second measure" (ai.thesatyajit.com), section "What one decode
 * step of Kimi K3 does": per token a router scores 896 experts, 16 are routed
 * to, a shared expert runs beside them, and the experts are stored in MXFP4
 * (17,547,264 bytes each at hidden 7168, expert intermediate 1536).  For each
 * activation row b of a batch of 1..64 (the decode envelope of "vLLM reports
 * 842 tokens per second for Kimi decoding with NVIDIA DSpark", ai-primer.com,
 * list of the supported envelope):
 *
 *   logit[e] = fp32( sum_h x[b][h] * Wr[e][h] + bias[e] )
 *   S        = the top_k experts by (logit descending, index ascending)
 *   gate[j]  = exp(logit[S_j] - logit[S_0]) / sum_i exp(logit[S_i] - logit[S_0])
 *   FFN_W(x) = W_down ( silu(W_gate x) * (W_up x) ),   silu(z) = z / (1 + e^-z)
 *   residual[b] += FFN_shared(x[b]) + sum_j gate[j] * FFN_{S_j}(x[b])
 *
 * MXFP4 (OCP Microscaling Formats v1.0): each weight is a 4-bit E2M1 code
 * (sign, 2-bit exponent with bias 1, 1-bit mantissa: magnitudes 0, .5, 1,
 * 1.5, 2, 3, 4, 6), and each block of 32 consecutive elements along the
 * contraction dimension K of one output row shares an E8M0 scale byte
 * (2^(byte-127); 0xFF is NaN).  Codes are packed two per byte, element 2i in
 * bits 3:0 and element 2i+1 in bits 7:4.  A matrix [N][K] is stored as codes
 * [N][K/2] bytes and scales [N][K/32] bytes, both row-major.
 *
 * Expert blob.  Routed expert e occupies moe_expert_bytes(H, I) bytes at
 * experts + e * moe_expert_bytes(H, I), holding, each sub-array starting at a
 * multiple of 256 bytes (no padding occurs at H 7168, I 1536):
 *     gate codes [I][H/2] | up codes [I][H/2] | down codes [H][I/2] |
 *     gate scales [I][H/32] | up scales [I][H/32] | down scales [H][I/32]
 *
 * Precision.  Router products bf16 x bf16 are exact; they are summed in fp64
 * and rounded once to fp32 (so expert selection is reproducible bit for bit).
 * Expert and shared-expert dot products are accumulated in fp32; the SwiGLU
 * intermediate is kept in fp32; the combine is fp32.
 *
 * Conventions for every entry point.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises, and keeps no state
 *     between calls.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and runs asynchronously; results are visible after the
 *     caller synchronises that stream.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and return MOE_ERR_INVALID_ARGUMENT; shapes outside the kernels'
 *     envelope return MOE_ERR_UNSUPPORTED (the caller runs something else);
 *     a failed launch returns MOE_ERR_HIP.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Buffers must not alias unless stated.  Device pointers must be aligned
 *     to 16 bytes (bf16/fp32 tensors) and 256 bytes (expert blobs, workspace).
 *   - Concurrent calls are safe when they use distinct workspaces and
 *     outputs.  Non-finite inputs are not checked; a 0xFF scale byte makes
 *     NaN every output that depends on its block.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1,    /* NULL pointer, bad size, bad alignment   */
  MOE_ERR_UNSUPPORTED = -2,         /* valid, but beyond the kernels' envelope */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3, /* ws_bytes < moe_workspace_size(...)      */
  MOE_ERR_HIP = -4                  /* a HIP runtime call or launch failed     */
} moe_status;

typedef enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 } moe_dtype;

/* Largest batch (activation rows) any entry point accepts. */
#define MOE_MAX_BATCH 64
/* Largest top_k and number of experts the router/top-k kernels accept. */
#define MOE_MAX_TOPK 64
#define MOE_MAX_EXPERTS 4096

/* Layout of the experts buffer (moe_layer_weights.expert_layout). */
#define MOE_EXPERTS_CANONICAL 0 /* the blob layout described above             */
#define MOE_EXPERTS_PACKED 1    /* rewritten by moe_pack_experts (see below)    */

/*
 * One layer's weights: a host struct of device pointers.
 *   hidden H, inter I (routed expert intermediate), num_experts E, top_k k,
 *   shared_inter Is (0 = no shared expert).  H and I multiples of 32,
 *   Is a multiple of 8.
 *   router_w     bf16 [E][H] (row e scores expert e)
 *   router_bias  fp32 [E], added to the logits before selection and gates;
 *                NULL for none
 *   shared_gate, shared_up  bf16 [Is][H];  shared_down  bf16 [H][Is];
 *                all three NULL iff Is == 0
 *   experts      E blobs of moe_expert_bytes(H, I) bytes
 *   expert_layout  MOE_EXPERTS_CANONICAL or MOE_EXPERTS_PACKED: which layout
 *                the experts buffer holds (moe_decode_layer needs PACKED)
 * bf16 tensors are raw bfloat16 bit patterns (uint16_t).
 */
typedef struct {
  int32_t hidden, inter, num_experts, top_k, shared_inter;
  const uint16_t* router_w;
  const float* router_bias;
  const uint16_t* shared_gate;
  const uint16_t* shared_up;
  const uint16_t* shared_down;
  const uint8_t* experts;
  int32_t expert_layout;
} moe_layer_weights;

/* Bytes of one expert blob (17,547,264 at H 7168, I 1536); 0 if H or I is
 * not a positive multiple of 32. */
size_t moe_expert_bytes(int hidden, int inter);

/* Workspace bytes moe_decode_layer needs for this layer at this batch.
 * Returns MOE_ERR_INVALID_ARGUMENT for the same shape errors as
 * moe_decode_layer. */
moe_status moe_workspace_size(const moe_layer_weights* w, int batch, size_t* bytes);

/*
 * moe_pack_experts / moe_unpack_experts -- rewrite experts [0, num_experts)
 * of an experts buffer IN PLACE from the canonical blob layout into the
 * packed layout moe_decode_layer streams, or back.  Done once, when the
 * weights are loaded; not part of a decode step.  Each blob keeps its size
 * (moe_expert_bytes) and position; the rewrite is an exact byte permutation.
 *
 * Packed layout.  Each MXFP4 matrix [N][K] of a blob is cut into tiles of 16
 * rows x 16 scale blocks (16 x 512 elements; the last tile of a row group
 * holds the remaining K/32 mod 16 blocks).  A tile of SC blocks holds its
 * codes as [SC][16 rows] x 16 bytes followed by its scales as [16 rows][SC]
 * bytes (in a full tile, SC = 16, a row's scale of block 4 kb + q sits at
 * byte 4 q + kb of the row's 16); a row group's tiles are consecutive.  The blob holds, for every
 * 16-row group of the gate/up rows and every segment along H, the gate tile
 * then the up tile; then the down tiles (16-row groups of H, segments along
 * I); then zero padding up to moe_expert_bytes.  So a wave of 64 lanes reads
 * 16 rows x 128 elements of codes as one contiguous kilobyte, with the tile's
 * scales right behind it.
 *
 *   experts  device buffer of num_experts * moe_expert_bytes(H, I) bytes,
 *            256-byte aligned
 *   scratch  device buffer of >= moe_expert_bytes(H, I) bytes, not
 *            overlapping experts (one expert is staged through it at a time)
 * Enqueued on `stream`; the buffer must not be used by other work until the
 * stream has passed the call.
 */
moe_status moe_pack_experts(uint8_t* experts, int num_experts, int hidden, int inter, void* scratch,
                            size_t scratch_bytes, void* stream);
moe_status moe_unpack_experts(uint8_t* experts, int num_experts, int hidden, int inter, void* scratch,
                              size_t scratch_bytes, void* stream);

/*
 * router_topk -- router GEMV, top-k selection and renormalised gates.
 *   x          bf16 [batch][hidden]
 *   router_w   bf16 [num_experts][hidden]; bias fp32 [num_experts] or NULL
 *   topk_idx   out int32 [batch][top_k], experts in (logit desc, index asc)
 *              order -- ties resolve to the lower index
 *   topk_gate  out fp32 [batch][top_k], gates in the same order, sum 1
 *   logits     out fp32 [batch][num_experts] (the router scores), or NULL
 *   ws         device workspace of >= moe_router_workspace_size(...) bytes
 *              (may be NULL when that size is 0)
 * 1 <= batch <= 64, 1 <= top_k <= min(num_experts, 64),
 * num_experts <= 4096, hidden a multiple of 32 and <= 16384.
 */
size_t moe_router_workspace_size(int batch, int num_experts);
moe_status router_topk(const uint16_t* x, int batch, int hidden, const uint16_t* router_w, const float* bias,
                       int num_experts, int top_k, int32_t* topk_idx, float* topk_gate, float* logits, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * expert_gemv_mxfp4 -- y[b][n] = sum_k dequant(W)[n][k] * x[b][k], fp32.
 *   codes   [n][k/2] bytes, scales [n][k/32] bytes (one MXFP4 matrix)
 *   x       [batch][k], bf16 (x_dtype MOE_DTYPE_BF16) or fp32
 *   y       out fp32 [batch][n]; must not alias x
 * k a multiple of 32 (<= 16384), 1 <= n, 1 <= batch <= 64.
 */
moe_status expert_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int n, int k, const void* x,
                             moe_dtype x_dtype, int batch, float* y, void* stream);

/*
 * moe_workspace_init -- clear a workspace before its first use.
 * The first bytes of a layer workspace are a control block that
 * moe_decode_layer's single persistent kernel synchronises through: the
 * counters of its two work queues (zero between calls) and a call epoch that
 * every call advances.  Data that workgroups of one call hand to each other is tagged
 * with that call's epoch, so stale data of an earlier call is never taken
 * for the current call's.  A workspace therefore needs this (or any zero
 * fill of the whole buffer) once after allocation, and again after a call
 * that did not complete (a device fault).  Enqueued on `stream`.  ws
 * 256-byte aligned, ws_bytes a multiple of 16.
 * The uint32 at byte offset MOE_WS_STATUS_OFFSET of the workspace is a sticky
 * status word: nonzero means a synchronisation wait inside a call timed out
 * (about a second), which only happens if the workspace was not initialised
 * or the launch could not keep all of its workgroups resident; the outputs
 * of such a call are not valid.  It is cleared by moe_workspace_init.
 * Tags repeat after 2^32 calls on one workspace.
 */
#define MOE_WS_STATUS_OFFSET 28
moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * moe_workspace_status -- enqueue on `stream` a copy of the workspace's
 * sticky status word (above) into *status, a uint32 in device memory or in
 * pinned host memory; the value is there once the stream has passed the
 * call.  0: every synchronisation wait of every call since
 * moe_workspace_init completed, so their outputs are valid; nonzero: a wait
 * gave up and the outputs of that call (and of later calls on the
 * workspace, whose waits then give up at once) are not valid.  A call whose
 * wait gives up still runs to completion without reading or writing outside
 * its buffers.  ws 256-byte aligned with ws_bytes covering the control block
 * (512 bytes); status 4-byte aligned; else MOE_ERR_INVALID_ARGUMENT.
 */
moe_status moe_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status, void* stream);

/* Batch > 1: the 8 bytes at this workspace offset hold, in their low 32 bits,
 * the number of distinct experts the last call routed its rows to (counted
 * on the device from the top-k indices) and, in their high 32 bits, that
 * call's tag.  Read it after the stream has passed the call. */
#define MOE_WS_ACTIVE_EXPERTS_OFFSET 384

/*
 * moe_decode_layer -- the whole layer for `batch` rows, as one kernel launch.
 *   x          bf16 [batch][hidden], the layer input (normalised activations)
 *   residual   fp32 [batch][hidden], read and overwritten with
 *              residual + shared + sum_j gate_j * expert_j; must not alias x
 *   topk_idx   out int32 [batch][top_k]; topk_gate out fp32 [batch][top_k]
 *   w          weights with expert_layout == MOE_EXPERTS_PACKED (a canonical
 *              experts buffer returns MOE_ERR_UNSUPPORTED: pack it once first)
 *   ws         workspace of >= moe_workspace_size(w, batch) bytes, 256-byte
 *              aligned, owned by the caller, cleared once by
 *              moe_workspace_init; calls that share a workspace must be
 *              ordered on one stream (they must not overlap)
 * Routing never leaves the device: no host synchronisation happens inside.
 */
moe_status moe_decode_layer(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                            int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_decode_layer_mxfp8 -- opt-in variant of moe_decode_layer whose routed
 * experts multiply their FP4 weights by MXFP8 activations, the precision the
 * expert kernel of "Kimi K3 on GB300: 13 kernels a layer, and what 842 and
 * 423 tokens a second measure" uses (section "Why batch 1 on a rack is not
 * only a bandwidth problem": FP4 x MXFP8 FC1/FC2 products).  The row entering
 * a routed expert's FC1 and the SwiGLU output entering its FC2 are each
 * quantised to MXFP8 (OCP Microscaling Formats v1.0: per block of 32
 * consecutive elements an E8M0 scale 2^(floor(log2 amax) - 8), elements the
 * nearest E4M3 value, ties to even, clamped to +-448) and the products run on
 * gfx950's scaled FP4 x FP8 matrix instruction with the dot products summed
 * in fp32.  The router, top-k, gates, the bf16 shared expert and the combine
 * are exactly those of moe_decode_layer, so expert indices and gates are
 * identical; the layer output differs from moe_decode_layer's by the
 * activation quantisation (a few 1e-2 relative on the experts' part).
 * Arguments, workspace and errors as moe_decode_layer; additionally
 * MOE_ERR_UNSUPPORTED when 16 columns of the FC2 input (inter rounded up to
 * 512, as E4M3 codes and scales) exceed 33,280 bytes of staging (inter above
 * 1536).
 */
moe_status moe_decode_layer_mxfp8(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_decode_layer_noalloc -- moe_decode_layer for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no workspace: the library's
 * own static device array of MOE_NOALLOC_SCRATCH_BYTES serves instead, one
 * per GPU, held from the first call on that GPU until the process ends; the
 * call itself allocates nothing.  x, residual, topk_idx, topk_gate and w are
 * as for moe_decode_layer.
 *   status   device pointer to a uint32 (or NULL): after the layer, the
 *            array's sticky status word is copied there on `stream` (0: every
 *            wait of every no-allocation call on this GPU completed, see
 *            moe_workspace_status)
 * Errors: MOE_ERR_WORKSPACE_TOO_SMALL, before anything is enqueued, when
 * moe_workspace_size(w, batch) exceeds MOE_NOALLOC_SCRATCH_BYTES (24 MiB:
 * the K3 shape fits up to batch 20); MOE_ERR_UNSUPPORTED when the first call
 * on a GPU is made while `stream` is being captured (that call clears the
 * array once with a fill kernel, which must not be recorded into a graph);
 * otherwise as moe_decode_layer.
 * Every call on one GPU shares that GPU's array and leaves its contents for
 * the next (each call's data carries that call's tag, so nothing stale is
 * ever taken as current): calls on one GPU must be ordered -- two that
 * overlap, on different streams or threads, race on the array and their
 * results are undefined.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (24u << 20)
moe_status moe_decode_layer_noalloc(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                    int32_t* topk_idx, float* topk_gate, uint32_t* status, void* stream);

/*
 * Per-kernel timing of moe_decode_layer (for profiling and benchmarks).
 * moe_decode_layer_kernel_count() is the number K of kernels one call
 * launches; moe_decode_layer_kernel_name(i) the name of the i-th (NULL out
 * of range).  moe_decode_layer_timed() is moe_decode_layer that also records
 * K+1 caller-created hipEvent_t `events` on `stream`: events[0] before the
 * first kernel and events[i+1] right after kernel i, so the elapsed time
 * between events[i] and events[i+1] brackets kernel i.  n_events must be at
 * least K+1 and no entry may be NULL (else MOE_ERR_INVALID_ARGUMENT).
 */
int moe_decode_layer_kernel_count(void);
const char* moe_decode_layer_kernel_name(int i);
moe_status moe_decode_layer_timed(const moe_layer_weights* w, const uint16_t* x, float* residual, int batch,
                                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream,
                                  void* const* events, int n_events);

/*
 * Dense-block pieces used between MoE layers of a decode-step stack.
 * rmsnorm_bf16:    out[b] = bf16( in[b] / sqrt(mean(in[b]^2) + eps) ), gain 1;
 *                  in fp32 [batch][hidden], out bf16 [batch][hidden].
 * dense_gemv_bf16: y[b][n] = bf16( sum_k W[n][k] * x[b][k] ) with fp32
 *                  accumulation; W bf16 [n][k], x bf16 [batch][k], y bf16
 *                  [batch][n]; y must not alias x.  k a multiple of 8.
 * residual_add_bf16: h[b][i] += float(t[b][i]) (h fp32, t bf16).
 * residual_add_rmsnorm_bf16: residual_add_bf16 then rmsnorm_bf16 of the
 *                  updated h into out, as one launch (same sums, same order).
 */
moe_status rmsnorm_bf16(const float* in, int batch, int hidden, float eps, uint16_t* out, void* stream);
moe_status dense_gemv_bf16(const uint16_t* w, int n, int k, const uint16_t* x, int batch, uint16_t* y,
                           void* stream);
moe_status residual_add_bf16(float* h, const uint16_t* t, int batch, int hidden, void* stream);
moe_status residual_add_rmsnorm_bf16(float* h, const uint16_t* t, int batch, int hidden, float eps, uint16_t* out,
                                     void* stream);

/*
 * moe_set_max_workgroups -- test and diagnostic knob, not needed for decoding:
 * caps the number of workgroups of the layer kernel (every moe_decode_layer*
 * entry point) launched after it returns, process-wide, at n; n = 0 restores
 * the default (two workgroups per compute unit).  The layer's work queue is
 * built to finish on any grid of at least one workgroup (a unit waits only
 * on units before it in the queue), and its results do not depend on the
 * grid; a small grid runs it in a different interleaving, which is what
 * the knob is for.  n < 0: MOE_ERR_INVALID_ARGUMENT.  Not synchronised
 * with launches in flight on other host threads.
 */
moe_status moe_set_max_workgroups(int n);

/*
 * moe_stream_read_probe -- measurement aid, not part of a decode step: one
 * kernel that reads `bytes` of `buf` once with 16-byte non-temporal loads
 * (blocks_per_cu 256-thread workgroups per compute unit, grid-stride), the
 * access pattern of a plain streaming read.  Timing it gives the device's
 * HBM read ceiling that the layer's weight streams are compared with.
 * `sink` (device, 4 bytes) is written only in the (never expected) case
 * that the xor of all data equals 0x9E3779B9, so nothing else is stored.
 * buf 16-byte aligned, bytes a positive multiple of 16, 1 <= blocks_per_cu
 * <= 32; else MOE_ERR_INVALID_ARGUMENT.
 */
moe_status moe_stream_read_probe(const void* buf, size_t bytes, int blocks_per_cu, uint32_t* sink, void* stream);

/*
 * moe_prefetch -- read a table of weight ranges once with ordinary
 * (allocating) loads, so that they sit in the device's memory-side
 * last-level cache (256 MB on MI355X) when a later kernel streams them: the
 * "prefetch on a third stream" of "Kimi K3 on GB300: 13 kernels a layer"
 * (section "What the fused path changes"), where a small kernel walks a
 * table of upcoming weight ranges.  Meant for a side stream, beside kernels
 * that leave HBM idle (norms, launch gaps); it writes nothing and its
 * results are not needed by anyone, so nothing has to wait for it.
 *   ranges   host array of n_ranges (1..MOE_PREFETCH_MAX_RANGES) device
 *            ranges, each 16-byte aligned with a size multiple of 16; the
 *            table is copied into the launch, so it need not outlive the call
 *   blocks   256-thread workgroups of the kernel (1..65536): how much of the
 *            device it occupies beside the other stream's work
 * Safe under stream capture (one kernel node, arguments by value).
 */
#define MOE_PREFETCH_MAX_RANGES 8
typedef struct {
  const void* ptr;
  size_t bytes;
} moe_range;
moe_status moe_prefetch(const moe_range* ranges, int n_ranges, int blocks, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
