// probe.hip -- a plain streaming read of a device buffer: the HBM read
// ceiling that the decode layer's own streams are compared against.  Every
// lane reads 16-byte granules with non-temporal loads, eight in flight per
// iteration, grid-stride over the buffer; the granules are folded by xor and
// stored only if the fold takes one particular value, so no load can be
// dropped by the compiler and (almost) nothing is written.
#include "internal.h"
#include "mx_common.h"

namespace moe {

constexpr int PROBE_UNROLL = 8;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * PROBE_UNROLL;
  for (size_t base = (size_t)blockIdx.x * 256 * PROBE_UNROLL + threadIdx.x; base < n16; base += stride) {
    u32x4 v[PROBE_UNROLL];
#pragma unroll
    for (int i = 0; i < PROBE_UNROLL; ++i) {
      const size_t g = base + 256 * (size_t)i;
      v[i] = g < n16 ? ld_weight16(p + g) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < PROBE_UNROLL; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int blocks_per_cu, uint32_t* sink, hipStream_t s) {
  const int grid = num_cus() * blocks_per_cu;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
