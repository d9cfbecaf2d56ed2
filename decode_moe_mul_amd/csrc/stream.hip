// qmoe_stream_read: a plain streaming read of a device buffer, for measuring
// the HBM read rate this part sustains (16-byte nontemporal vector loads,
// each block on a contiguous chunk of its own, consecutive lanes on
// consecutive 16-byte pieces, eight loads in flight per lane).  Decode is a
// weight stream ([P3] "RTX 3090 Llama 70B three-tier cache" section 4.4:
// every weight is read once per token), so this rate is the practical
// ceiling of the decode GEMVs, reported beside the 8 TB/s vendor peak.
// Per-block chunks with eight loads in flight per lane gave the highest rate
// of the patterns tried on MI355X and varied least with the block count; a
// grid-stride read with four loads per lane stayed near 6 TB/s at 4 to 16
// blocks per CU.
//
// qmoe_wave_latency: the dependent-issue latencies one wave sees on this part
// (shader clock cycles), and the cost of the routing's wave top-k on one row,
// the steps that bound the decode routing's tail, where a single wave per row
// works through k dependent rounds.
#include "route.hpp"

namespace qmoe {

constexpr int kStreamBlock = 256;
constexpr int kStreamDepth = 8;  // loads in flight per lane

// Block b reads the b-th of gridDim.x equal chunks, each a whole number of
// steps of kStreamDepth x 256 x 16 bytes; the remainder past the chunks is
// read grid-stride, one load per lane at a time.
__global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(const uint4* p, size_t n16,
                                                                   uint32_t* sink) {
  constexpr size_t kStep = (size_t)kStreamDepth * kStreamBlock;
  const size_t chunk = n16 / gridDim.x / kStep * kStep;
  const uint4* q = p + (size_t)blockIdx.x * chunk;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < chunk; i += kStep) {
    uint4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) v[d] = load_stream(q + i + d * kStreamBlock);
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (size_t i = chunk * gridDim.x + (size_t)blockIdx.x * kStreamBlock + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kStreamBlock) {
    const uint4 v = load_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a store the compiler cannot rule out keeps every load alive; it almost
  // never happens
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Keys of the measured top-k: a fixed hash of (lane, slot, call) mapped to
// floats in [-1, 1), with a 1/8 chance of a value shared by many experts.
QMOE_D float lat_key(int lane, int i, int call) {
  uint32_t h = (uint32_t)(lane * 64 + i) * 0x9E3779B1u + (uint32_t)call * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  if ((h & 7u) == 0u) return 0.5f;
  return (float)(h >> 8) * (1.f / 8388608.f) - 1.f;
}

// One wave.  out[0] cycles per dependent VALU op, out[1] per DPP wave max
// with its read-back, out[2] per ballot round trip (compare, ballot, first
// lane, read-lane), out[3] per wave_topk of 512 keys with k = 10, out[4] per
// lane_sort of 8 keys, out[5] the shader clock in MHz (shader cycles over
// the 100 MHz real-time counter across the kernel).
__global__ __launch_bounds__(64) void wave_latency_kernel(uint64_t* out, uint32_t seed) {
  const int lane = threadIdx.x & 63;
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime(), k0 = __builtin_amdgcn_s_memtime();
  uint32_t v = seed * (uint32_t)(lane + 1);
  constexpr int kN = 256;
  uint64_t c0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < kN; ++i) v = max(v, v ^ (uint32_t)i) + 1u;
  uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t valu = (c1 - c0) / kN;
  c0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < kN / 4; ++i) {
    const uint32_t m = wave_max_u32(v);
    v = v == m ? 0u : v + 1u;
  }
  c1 = __builtin_amdgcn_s_memtime();
  const uint64_t wmax = (c1 - c0) / (kN / 4);
  c0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < kN; ++i) {
    const uint64_t m = __builtin_amdgcn_ballot_w64((v & 7u) == (uint32_t)(lane & 7));
    const int l = m ? (int)__builtin_ctzll(m) : 0;
    v += (uint32_t)__builtin_amdgcn_readlane((int)v, l) & 3u;
  }
  c1 = __builtin_amdgcn_s_memtime();
  const uint64_t ballot = (c1 - c0) / kN;
  constexpr int kCalls = 16;
  int acc = 0;
  c0 = __builtin_amdgcn_s_memtime();
  for (int c = 0; c < kCalls; ++c) {
    float raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = lat_key(lane, i, c + acc);
    int id;
    float lg;
    wave_topk<8>(raw, 512, 10, id, lg);
    acc += __builtin_amdgcn_readlane(id, 9) & 1;
  }
  c1 = __builtin_amdgcn_s_memtime();
  const uint64_t topk = (c1 - c0) / kCalls;
  c0 = __builtin_amdgcn_s_memtime();
  for (int c = 0; c < kCalls; ++c) {
    uint32_t key[8], kk[8], ss[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = order_key(lat_key(lane, i, c + acc));
    lane_sort<8>(key, kk, ss);
    acc += __builtin_amdgcn_readlane((int)(kk[0] ^ ss[7]), 0) & 1;
  }
  c1 = __builtin_amdgcn_s_memtime();
  const uint64_t sort = (c1 - c0) / kCalls;
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime(), k1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    out[0] = valu;
    out[1] = wmax;
    out[2] = ballot;
    out[3] = topk;
    out[4] = sort;
    out[5] = r1 > r0 ? (k1 - k0) * 100 / (r1 - r0) : 0;  // cycles per 10 ns -> MHz
    out[6] = (uint64_t)(v & 1u) + (uint64_t)(acc & 1);   // keeps the chains alive
  }
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

extern "C" int qmoe_wave_latency(uint64_t* out, void* stream) {
  if (!out) return fail(QMOE_ERR_INVALID_ARG, "qmoe_wave_latency: null pointer");
  return QMOE_LAUNCH("wave_latency", wave_latency_kernel, dim3(1), 64, 0, (hipStream_t)stream,
                     out, 0x2545F491u);
}
