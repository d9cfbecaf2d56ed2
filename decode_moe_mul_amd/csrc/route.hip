// moe_route: router logits, top-k with ties to the lower id, renormalised
// softmax over the kept logits, always-on shared experts appended.
// ([P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析: a light
// router picks 10 of 512 experts per token; [P4] "DwarfStar on 8x L40S",
// section 快速上手: a shared expert beside the routed ones.)
//
// Kernels:
//  router_gemv_kernel  rows <= 16: each wave streams one expert row of Wr over
//                      a K-slice against all rows staged in LDS; split-K
//                      partials go to the workspace (no atomics).
//  router_gemm_kernel  longer chunks: 64x64 output tiles, LDS-staged K steps.
//  topk_kernel         one wave per row: sums the split-K partials in fixed
//                      order, adds the bias, selects k by repeated wave
//                      arg-max, softmax over the kept logits.
#include "common.hpp"

namespace qmoe {

constexpr int kRouteBlock = 256;
constexpr int kGemvRowsMax = 16;

struct RouteParams {
  const void* x;
  int x_dtype, T, H;
  const float* Wr;
  const float* bias;
  int E, k, n_shared;
  int32_t* ids;
  float* p;
  float* logits;
  float* part;  // [KS][T][E]
  int KS, ks_len;
};

// 4 consecutive activations (fp32 or bf16) starting at element i (i % 4 == 0)
template <int DT>
QMOE_D float4 load_act4(const void* x, size_t i) {
  if constexpr (DT == QMOE_F32) {
    return *(const float4*)((const float*)x + i);
  } else {
    const uint2 b = *(const uint2*)((const uint16_t*)x + i);
    return make_float4(bf16_bits_to_f32(b.x & 0xFFFFu), bf16_bits_to_f32(b.x >> 16),
                       bf16_bits_to_f32(b.y & 0xFFFFu), bf16_bits_to_f32(b.y >> 16));
  }
}

// x[:, k0:k0+len] -> xsl [T][ks_len], float4 granules, 4 loads in flight
template <int DT>
QMOE_D void stage_x_slice(const RouteParams& P, int k0, int len, float* xsl) {
  const int l4 = len >> 2, n4 = P.T * l4;
  for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * kRouteBlock) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + u * kRouteBlock, n4 - 1);  // unconditional loads
      const int t = i / l4, j = 4 * (i - t * l4);
      v[u] = load_act4<DT>(P.x, (size_t)t * P.H + k0 + j);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kRouteBlock;
      if (i < n4) {
        const int t = i / l4, j = 4 * (i - t * l4);
        *(float4*)(xsl + t * P.ks_len + j) = v[u];
      }
    }
  }
}

// Grid (E/4, KS); wave w of block b handles expert 4b+w over values
// [ks*ks_len, (ks+1)*ks_len) of the hidden dimension (ks_len <= 1024, a
// multiple of 256).  Loads are issued in batches before they are used.
__global__ __launch_bounds__(kRouteBlock) void router_gemv_kernel(RouteParams P) {
  extern __shared__ __align__(16) float xsl[];  // [T][ks_len]
  const int ks = blockIdx.y;
  const int k0 = ks * P.ks_len;
  const int len = min(P.ks_len, P.H - k0);
  if (P.x_dtype == QMOE_F32)
    stage_x_slice<QMOE_F32>(P, k0, len, xsl);
  else
    stage_x_slice<QMOE_BF16>(P, k0, len, xsl);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= P.E) return;
  const float* wrow = P.Wr + (size_t)e * P.H + k0;
  float4 w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = 4 * lane + 256 * u;
    w[u] = j < len ? *(const float4*)(wrow + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc[kGemvRowsMax];
#pragma unroll
  for (int t = 0; t < kGemvRowsMax; ++t) {
    acc[t] = 0.f;
    if (t < P.T) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 4 * lane + 256 * u;
        if (j < len) {
          const float4 xv = *(const float4*)(xsl + t * P.ks_len + j);
          acc[t] += w[u].x * xv.x + w[u].y * xv.y + w[u].z * xv.z + w[u].w * xv.w;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvRowsMax; ++t) {
    if (t < P.T) {
      float v = acc[t];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) P.part[((size_t)ks * P.T + t) * P.E + e] = v;
    }
  }
}

// 64 x 64 tile of logits (rows x experts), 256 threads x (4 x 4) outputs.
constexpr int kGT = 64, kGE = 64, kGK = 32;
__global__ __launch_bounds__(kRouteBlock) void router_gemm_kernel(RouteParams P) {
  __shared__ float xs[kGK][kGT + 4];
  __shared__ float wsm[kGK][kGE + 4];
  const int t0 = blockIdx.y * kGT, e0 = blockIdx.x * kGE;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 16 x 16 threads
  float acc[4][4] = {};
  for (int k0 = 0; k0 < P.H; k0 += kGK) {
    for (int i = threadIdx.x; i < kGT * kGK; i += kRouteBlock) {
      const int r = i / kGK, c = i - r * kGK;
      const int t = t0 + r, kk = k0 + c;
      xs[c][r] = (t < P.T && kk < P.H) ? load_act(P.x, P.x_dtype, (size_t)t * P.H + kk) : 0.f;
      const int e = e0 + r;
      wsm[c][r] = (e < P.E && kk < P.H) ? P.Wr[(size_t)e * P.H + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kGK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[c][ty + 16 * i]; b[i] = wsm[c][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
      if (t < P.T && e < P.E) P.part[(size_t)t * P.E + e] = acc[i][j];
    }
}

// (key, id) order: larger key first, then smaller id.  NaN keys rank below
// every number.
QMOE_D bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int PER>  // values per lane: E <= 64 * PER
__global__ __launch_bounds__(kRouteBlock) void topk_kernel(RouteParams P) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= P.T) return;
  float raw[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    raw[i] = 0.f;
    if (e < P.E) {
      // split-K partials in order, 8 loads in flight at a time
      float v = 0.f;
      for (int s0 = 0; s0 < P.KS; s0 += 8) {
        float pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[u] = s0 + u < P.KS ? P.part[((size_t)(s0 + u) * P.T + t) * P.E + e] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < P.KS) v += pv[u];
      }
      if (P.bias) v += P.bias[e];
      raw[i] = v;
      if (P.logits) P.logits[(size_t)t * P.E + e] = v;
    }
  }
  uint64_t taken = 0;
  int my_id = 0;
  float my_raw = 0.f;
  for (int s = 0; s < P.k; ++s) {
    float bk = -INFINITY, br = 0.f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < P.E && !((taken >> i) & 1)) {
        const float key = raw[i] != raw[i] ? -INFINITY : raw[i];
        if (better(key, e, bk, bi)) { bk = key; bi = e; br = raw[i]; }
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ok = __shfl_xor(bk, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      const float orw = __shfl_xor(br, off, 64);
      if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; br = orw; }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == s) { my_id = bi; my_raw = br; }
  }
  const int kt = P.k + P.n_shared;
  // softmax over the kept logits, relative to the largest (slot 0)
  const float l0 = __shfl(my_raw, 0, 64);
  const float w = lane < P.k ? expf(my_raw - l0) : 0.f;
  float sum = w;
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < P.k) {
    P.ids[(size_t)t * kt + lane] = my_id;
    P.p[(size_t)t * kt + lane] = w / sum;
  }
  for (int s = lane; s < P.n_shared; s += 64) {
    P.ids[(size_t)t * kt + P.k + s] = P.E + s;
    P.p[(size_t)t * kt + P.k + s] = 1.f;
  }
}

static void route_split(int T, int H, int& KS, int& ks_len) {
  if (T > kGemvRowsMax) { KS = 1; ks_len = H; return; }
  // K-slices of 1024 values (multiple of 256), capped so T*ks_len*4 <= 32 KiB
  ks_len = 1024;
  while (ks_len > 256 && (size_t)T * ks_len * 4 > 32768) ks_len /= 2;
  KS = (H + ks_len - 1) / ks_len;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

size_t moe_route_workspace_size(int T, int H, int E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  return round_up256((size_t)KS * T * E * sizeof(float)) + 256;
}

int moe_route(const void* x, int x_dtype, int T, int H, const float* Wr, const float* bias,
              int E, int k, int n_shared, int32_t* ids, float* p, float* logits, void* ws,
              size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || k > 64 || n_shared < 0)
    return fail(QMOE_ERR_INVALID_ARG, "moe_route: bad sizes T=%d H=%d E=%d k=%d n_shared=%d",
                T, H, E, k, n_shared);
  if (E > 4096) return fail(QMOE_ERR_UNSUPPORTED, "moe_route: E=%d > 4096", E);
  if (H % 4) return fail(QMOE_ERR_INVALID_ARG, "moe_route: H %% 4 != 0");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_route: unknown x_dtype %d", x_dtype);
  if (T == 0) return QMOE_OK;
  if (!x || !Wr || !ids || !p) return fail(QMOE_ERR_INVALID_ARG, "moe_route: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(Wr, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_route: misaligned x/Wr");
  const size_t need = moe_route_workspace_size(T, H, E);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu (or misaligned)", ws_bytes,
                need);
  RouteParams P{x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids, p, logits, (float*)ws, 0, 0};
  route_split(T, H, P.KS, P.ks_len);
  hipStream_t s = (hipStream_t)stream;
  int st;
  if (T <= kGemvRowsMax) {
    const dim3 grid((E + 3) / 4, P.KS);
    st = QMOE_LAUNCH("router_gemv", router_gemv_kernel, grid, kRouteBlock,
                     (size_t)T * P.ks_len * sizeof(float), s, P);
  } else {
    const dim3 grid((E + kGE - 1) / kGE, (T + kGT - 1) / kGT);
    st = QMOE_LAUNCH("router_gemm", router_gemm_kernel, grid, kRouteBlock, 0, s, P);
  }
  if (st) return st;
  const dim3 tgrid((T + 3) / 4);
  const int per = (E + 63) / 64;
  if (per <= 1) return QMOE_LAUNCH("topk", topk_kernel<1>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 2) return QMOE_LAUNCH("topk", topk_kernel<2>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 4) return QMOE_LAUNCH("topk", topk_kernel<4>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 8) return QMOE_LAUNCH("topk", topk_kernel<8>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 16) return QMOE_LAUNCH("topk", topk_kernel<16>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 32) return QMOE_LAUNCH("topk", topk_kernel<32>, tgrid, kRouteBlock, 0, s, P);
  return QMOE_LAUNCH("topk", topk_kernel<64>, tgrid, kRouteBlock, 0, s, P);
}

}  // extern "C"
