// qmoe_stream_read: a plain streaming read of a device buffer, for measuring
// the HBM read rate this part sustains with the decode kernels' access
// pattern (16-byte nontemporal vector loads, consecutive lanes on
// consecutive 16-byte chunks, several loads in flight per lane).  Decode is a
// weight stream ([P3] "RTX 3090 Llama 70B three-tier cache" section 4.4:
// every weight is read once per token), so this rate is the practical
// ceiling of the decode GEMVs, reported beside the 8 TB/s vendor peak.
#include "common.hpp"

namespace qmoe {

constexpr int kStreamBlock = 256;
constexpr int kStreamDepth = 4;  // loads in flight per lane

__global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(const uint4* p, size_t n16,
                                                                   uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kStreamBlock;
  size_t i = (size_t)blockIdx.x * kStreamBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamDepth - 1) * stride < n16; i += kStreamDepth * stride) {
    uint4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) v[d] = load_stream(p + i + d * stride);
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a store the compiler cannot rule out keeps every load alive; it almost
  // never happens
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" int qmoe_stream_read(const void* buf, size_t bytes, int blocks_per_cu,
                                uint32_t* sink, void* stream) {
  if (bytes == 0) return QMOE_OK;
  if (!buf || !sink) return fail(QMOE_ERR_INVALID_ARG, "qmoe_stream_read: null pointer");
  if (!QMOE_ALIGNED(buf, 16) || bytes % 16)
    return fail(QMOE_ERR_INVALID_ARG, "qmoe_stream_read: buffer not 16-byte aligned/sized");
  if (blocks_per_cu < 1 || blocks_per_cu > 64)
    return fail(QMOE_ERR_INVALID_ARG, "qmoe_stream_read: blocks_per_cu=%d", blocks_per_cu);
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const dim3 grid((unsigned)(cus * blocks_per_cu));
  return QMOE_LAUNCH("stream_read", stream_read_kernel, grid, kStreamBlock, 0,
                     (hipStream_t)stream, (const uint4*)buf, bytes / 16, sink);
}
