// moe_combine: y[t] = sum_i p[t,i] * o[inv_perm[t*k+i]] (+ shared[t]), in
// fixed slot order, no atomics.  The weighted sum of the selected experts of
// [P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析.
#include <algorithm>

#include "common.hpp"

namespace qmoe {

// Block (x, b): float4 columns [256 x, 256 x + 256) of rows t = b, b + gridDim.y, ...
// A row's slot positions and weights are block-uniform (scalar loads); the o
// rows of up to kSlots slots are requested together before the fmaf chain
// adds them in slot order, so a row waits for memory twice per kSlots slots,
// not once per slot.
constexpr int kSlots = 16;
__global__ __launch_bounds__(256) void combine_kernel(const float* o, const int32_t* inv,
                                                      const float* p, int T, int k, int H,
                                                      const float* shared, float* y) {
  const int H4 = H >> 2;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H4) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < k; s0 += kSlots) {
      int pos[kSlots];
      float w[kSlots];
      float4 v[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {  // unconditional loads: no branch between them
        const size_t a = (size_t)t * k + min(s0 + j, k - 1);
        pos[j] = inv[a];
        w[j] = p[a];
      }
#pragma unroll
      for (int j = 0; j < kSlots; ++j)
        if (s0 + j >= k) pos[j] = -1;
#pragma unroll
      for (int j = 0; j < kSlots; ++j)  // invalid slots read row 0 and add nothing
        v[j] = ((const float4*)(o + (size_t)(pos[j] < 0 ? 0 : pos[j]) * H))[c];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        if (pos[j] < 0) continue;
        acc.x = fmaf(w[j], v[j].x, acc.x);
        acc.y = fmaf(w[j], v[j].y, acc.y);
        acc.z = fmaf(w[j], v[j].z, acc.z);
        acc.w = fmaf(w[j], v[j].w, acc.w);
      }
    }
    if (shared) {
      const float4 v = ((const float4*)(shared + (size_t)t * H))[c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    ((float4*)(y + (size_t)t * H))[c] = acc;
  }
}

}  // namespace qmoe

using namespace qmoe;

extern "C" int moe_combine(const float* o, const int32_t* inv_perm, const float* p, int T,
                           int k, int H, const float* shared, float* y, void* stream) {
  if (T < 0 || k < 0 || H <= 0 || H % 4)
    return fail(QMOE_ERR_INVALID_ARG, "moe_combine: bad sizes T=%d k=%d H=%d", T, k, H);
  if (T == 0) return QMOE_OK;
  if (!y || (k > 0 && (!o || !inv_perm || !p)))
    return fail(QMOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  if (!QMOE_ALIGNED(y, 16) || (o && !QMOE_ALIGNED(o, 16)) || (shared && !QMOE_ALIGNED(shared, 16)))
    return fail(QMOE_ERR_INVALID_ARG, "moe_combine: misaligned pointer");
  const dim3 grid((unsigned)((H / 4 + 255) / 256), (unsigned)std::min(T, 65535));
  return QMOE_LAUNCH("combine", combine_kernel, grid, 256, 0, (hipStream_t)stream, o, inv_perm,
                     p, T, k, H, shared, y);
}
