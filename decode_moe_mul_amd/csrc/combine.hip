// moe_combine: y[t] = sum_i p[t,i] * o[inv_perm[t*k+i]] (+ shared[t]), in
// fixed slot order, no atomics.  The weighted sum of the selected experts of
// [P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析.
#include "common.hpp"

namespace qmoe {

__global__ __launch_bounds__(256) void combine_kernel(const float* o, const int32_t* inv,
                                                      const float* p, int T, int k, int H,
                                                      const float* shared, float* y) {
  const int H4 = H >> 2;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * H4) return;
  const int t = (int)(i / H4), c = (int)(i - (size_t)t * H4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < k; ++s) {
    const int pos = inv[(size_t)t * k + s];
    if (pos < 0) continue;
    const float w = p[(size_t)t * k + s];
    const float4 v = ((const float4*)(o + (size_t)pos * H))[c];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  if (shared) {
    const float4 v = ((const float4*)(shared + (size_t)t * H))[c];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  ((float4*)(y + (size_t)t * H))[c] = acc;
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
  const size_t n = (size_t)T * (H / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  return QMOE_LAUNCH("combine", combine_kernel, grid, 256, 0, (hipStream_t)stream, o, inv_perm,
                     p, T, k, H, shared, y);
}
