// mx_common.h -- device helpers shared by the library's kernels (gfx950).
// Internal to libmoe_mxfp4.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define WAVE 64

// Streaming (non-temporal) 16-byte load: used ONLY for static weights, never
// for data that another wave of the same launch writes.
__device__ __forceinline__ u32x4 ld_weight16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Coherent (agent-scope) scalar loads and stores.  Data one workgroup of a
// launch writes and another reads goes through these: on gfx950 they carry
// the sc1 cache policy, i.e. they are performed at the device coherence point
// instead of in an XCD's non-coherent L2, so no L2 write-back or invalidate
// (which serialise device-wide) is ever needed to hand data between
// workgroups on different XCDs.
template <typename T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// E8M0 scale byte -> an fp32 power of two for the gfx950 scaled FP4
// conversions, which take the exponent of their scale operand: 2^(b-127),
// with 2^-127 (byte 0) as a subnormal and NaN for byte 0xFF.
__device__ __forceinline__ float e8m0_scale(uint32_t b) {
  uint32_t bits = (b == 0u) ? 0x00400000u : ((b == 255u) ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

// 4 FP4 byte pairs of one dword -> 4 bf16 pairs (exact: E2M1 x 2^k fits bf16).
// Pair j holds elements 2j (low nibble of byte j) and 2j+1 (high nibble).
__device__ __forceinline__ void dq4_bf16(uint32_t w, float s, bf16x2 out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
}

__device__ __forceinline__ void dq4_f32(uint32_t w, float s, f32x2 out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// fp32 -> bf16 round to nearest even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Butterfly sums across `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ double sum_lanes_f64(double v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, WAVE);
  hi = __shfl_xor(hi, m, WAVE);
  return ((uint64_t)hi << 32) | lo;
}
