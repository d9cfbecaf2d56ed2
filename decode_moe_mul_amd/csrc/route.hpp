// Internal header: device pieces of the router shared by moe_route,
// moe_route_decode and the one-launch decode layer -- the split-K router
// partials, the wave top-k with its softmax, the coherent hand-over of values
// between blocks of one launch -- and the host-side K split.
//
// The router's sums keep the default floating-point contraction; include this
// header before any header that switches contraction off.
#pragma once
#include "permute.hpp"

namespace qmoe {

constexpr int kRouteBlock = 256;
constexpr int kGemvRowsMax = 16;
// split-K router for <= 16 rows: 16 waves, one expert row of Wr per wave, so
// that each staged x slice serves 16 experts
constexpr int kGemvBlock = 1024;
constexpr int kGemvExperts = kGemvBlock / 64;

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

// x[:, k0:k0+len] -> xsl [T][ks_len], float4 granules, 4 loads in flight.
// Loads and stores are unconditional: a granule index past the end is
// clamped to the last granule, whose value it then writes again.  (With the
// stores under a condition the compiler moves each load into its store's
// branch, and the loads no longer fly together.)
template <int DT, int NT>
QMOE_D void stage_x_slice(const RouteParams& P, int k0, int len, float* xsl) {
  const int l4 = len >> 2, n4 = P.T * l4;
  for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * NT) {
    float4 v[4];
    int at[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + u * NT, n4 - 1);
      const int t = i / l4, j = 4 * (i - t * l4);
      v[u] = load_act4<DT>(P.x, (size_t)t * P.H + k0 + j);
      at[u] = t * P.ks_len + j;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) *(float4*)(xsl + at[u]) = v[u];
  }
}

// Sum over the wave of acc[r] for 16 rows at once: each exchange step halves
// the rows a lane carries (xor 32, 16, 8, 4), then xor 2 and 1 finish the
// sums.  17 lane exchanges instead of 16 separate 6-step reductions.  Lane L
// ends with the total of row ((L>>5)&1)*8 + ((L>>4)&1)*4 + ((L>>3)&1)*2 + ((L>>2)&1).
QMOE_D float wave_sum16(float (&acc)[kGemvRowsMax]) {
  const int lane = threadIdx.x & 63;
  float a8[8], a4[4], a2[2];
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float keep = b5 ? acc[8 + j] : acc[j], give = b5 ? acc[j] : acc[8 + j];
    a8[j] = keep + __shfl_xor(give, 32, 64);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float keep = b4 ? a8[4 + j] : a8[j], give = b4 ? a8[j] : a8[4 + j];
    a4[j] = keep + __shfl_xor(give, 16, 64);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b3 ? a4[2 + j] : a4[j], give = b3 ? a4[j] : a4[2 + j];
    a2[j] = keep + __shfl_xor(give, 8, 64);
  }
  float v = (b2 ? a2[1] : a2[0]) + __shfl_xor(b2 ? a2[0] : a2[1], 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

// The weight-row half of router_partials: wave w's expert row over the slice,
// 4 float4 per lane (zero past the slice).
template <int NT>
QMOE_D void router_wrow(const RouteParams& P, int b, int ks, float4 (&w)[4]) {
  const int k0 = ks * P.ks_len;
  const int len = min(P.ks_len, P.H - k0);
  const int lane = threadIdx.x & 63;
  const int e = b * (NT / 64) + (threadIdx.x >> 6);
  const float* wrow = P.Wr + (size_t)min(e, P.E - 1) * P.H + k0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = 4 * lane + 256 * u;
    w[u] = j < len ? *(const float4*)(wrow + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int NT>
QMOE_D void router_stage(const RouteParams& P, float* xsl, int ks) {
  const int k0 = ks * P.ks_len;
  const int len = min(P.ks_len, P.H - k0);
  if (P.x_dtype == QMOE_F32)
    stage_x_slice<QMOE_F32, NT>(P, k0, len, xsl);
  else
    stage_x_slice<QMOE_BF16, NT>(P, k0, len, xsl);
}

template <bool COH, int NT>
QMOE_D void router_dots(const RouteParams& P, const float* xsl, int b, int ks,
                        const float4 (&w)[4]);

// Block (b, ks) of the split-K router, NT threads: wave w handles expert
// (NT/64) b + w over values
// [ks*ks_len, (ks+1)*ks_len) of the hidden dimension (ks_len <= 1024, a
// multiple of 256) and writes its partial dot products for all T rows to
// part[ks][t][e] (written through when COH).  The weight row is requested
// before x is staged, so both loads are in flight together.  Every thread
// returns (no early exit), so callers may synchronise afterwards.
template <bool COH, int NT>
QMOE_D void router_partials(const RouteParams& P, float* xsl, int b, int ks) {
  float4 w[4];
  router_wrow<NT>(P, b, ks, w);
  router_stage<NT>(P, xsl, ks);
  __syncthreads();
  router_dots<COH, NT>(P, xsl, b, ks, w);
}

// The dot products of router_partials against the staged slice (every
// thread returns, so callers may synchronise afterwards).
template <bool COH, int NT>
QMOE_D void router_dots(const RouteParams& P, const float* xsl, int b, int ks,
                        const float4 (&w)[4]) {
  const int k0 = ks * P.ks_len;
  const int len = min(P.ks_len, P.H - k0);
  const int lane = threadIdx.x & 63;
  const int e = b * (NT / 64) + (threadIdx.x >> 6);
  const bool has_e = e < P.E;
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
  const float v = wave_sum16(acc);
  const int t = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 +
                ((lane >> 2) & 1);
  if (has_e && (lane & 3) == 0 && t < P.T) {
    float* dst = P.part + ((size_t)ks * P.T + t) * P.E + e;
    if constexpr (COH) store_coherent(dst, v);
    else *dst = v;
  }
}
// Order-preserving unsigned image of a logit (NaN ranks as -inf); every
// number maps above 0, which marks taken / absent slots.
QMOE_D uint32_t order_key(float f) {
  if (f != f) f = -INFINITY;
  const uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The lane's PER (key, slot) pairs sorted by key descending, equal keys by
// slot ascending: Batcher's odd-even merge network on 64-bit values
// key << 32 | ~slot, which are all distinct, so the order is unique.
template <int PER>
QMOE_D void lane_sort(const uint32_t (&key)[PER], uint32_t (&kk)[PER], uint32_t (&ss)[PER]) {
  uint64_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = ((uint64_t)key[i] << 32) | (uint32_t)~i;
#pragma unroll
  for (int p = 1; p < PER; p *= 2)
#pragma unroll
    for (int q = p; q >= 1; q /= 2)
#pragma unroll
      for (int j = q % p; j + q < PER; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q; ++i) {
          const int a = i + j, b = i + j + q;
          if (a / (2 * p) == b / (2 * p)) {
            // bitwise blends, not selects of array elements: the compiler
            // would turn those into dynamically indexed register arrays
            const uint64_t m = 0ull - (uint64_t)(v[b] > v[a]);
            const uint64_t va = v[a], vb = v[b];
            v[a] = (vb & m) | (va & ~m);
            v[b] = (va & m) | (vb & ~m);
          }
        }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kk[i] = (uint32_t)(v[i] >> 32);
    ss[i] = ~(uint32_t)v[i];
  }
}

// Top-k of one row of E logits held by one wave (lane l holds expert
// l + 64 i in raw[i], E <= 64 * PER, PER a power of two).  Each lane sorts
// its keys once (order key: NaN ranks as -inf; absent experts 0).  A round
// takes the wave max of the lanes' leading keys; when one lane holds it
// (the common case, found with one ballot) that lane wins, otherwise a DPP
// min over slot * 64 + lane picks the lowest id among the tied lanes (a
// lane's equal keys are in slot order).  The winner drops its leading key.
// Lane s < k gets the s-th id and its logit (read from the owning lane at
// the end).
template <int PER>
QMOE_D void wave_topk(const float (&raw)[PER], int E, int k, int& my_id, float& my_raw) {
  static_assert((PER & (PER - 1)) == 0, "PER must be a power of two");
  const int lane = threadIdx.x & 63;
  uint32_t key[PER], kk[PER], ss[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = lane + 64 * i < E ? order_key(raw[i]) : 0u;
  lane_sort<PER>(key, kk, ss);
  int src_lane = 0, src_slot = 0;
  for (int s = 0; s < k; ++s) {
    const uint32_t kmax = wave_max_u32(kk[0]);  // > 0 while s < k <= E
    const uint64_t m = __builtin_amdgcn_ballot_w64(kk[0] == kmax);
    int wl, ws;
    if (__builtin_popcountll(m) == 1) {
      wl = (int)__builtin_ctzll(m);
      ws = __builtin_amdgcn_readlane((int)ss[0], wl);
    } else {
      const uint32_t wid =
          wave_min_u32(kk[0] == kmax ? ss[0] * 64u + (uint32_t)lane : 0xFFFFFFFFu);
      wl = (int)(wid & 63u);
      ws = (int)(wid >> 6);
    }
    if (lane == s) { src_lane = wl; src_slot = ws; }
    const uint32_t w = lane == wl ? ~0u : 0u;  // the winner shifts its list
#pragma unroll
    for (int i = 0; i + 1 < PER; ++i) {
      kk[i] = (kk[i + 1] & w) | (kk[i] & ~w);
      ss[i] = (ss[i + 1] & w) | (ss[i] & ~w);
    }
    kk[PER - 1] &= ~w;
  }
  float g = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float v = __shfl(raw[i], src_lane, 64);
    g = i == src_slot ? v : g;
  }
  my_id = lane < k ? src_slot * 64 + src_lane : 0;
  my_raw = lane < k ? g : 0.f;
}

// ids/p of row t from its top-k (softmax over the kept logits relative to
// the largest), shared experts appended with weight 1
QMOE_D void write_topk(const RouteParams& P, int t, int my_id, float my_raw, int32_t* ids_copy) {
  const int lane = threadIdx.x & 63;
  const int kt = P.k + P.n_shared;
  const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_raw), 0));
  const float w = lane < P.k ? expf(my_raw - l0) : 0.f;
  float sum = w;
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < P.k) {
    P.ids[(size_t)t * kt + lane] = my_id;
    P.p[(size_t)t * kt + lane] = w / sum;
    if (ids_copy) ids_copy[t * kt + lane] = my_id;
  }
  for (int s = lane; s < P.n_shared; s += 64) {
    P.ids[(size_t)t * kt + P.k + s] = P.E + s;
    P.p[(size_t)t * kt + P.k + s] = 1.f;
    if (ids_copy) ids_copy[t * kt + P.k + s] = P.E + s;
  }
}
// Final logits of row t for the lane's experts e = lane + 64 i: the KS
// partials summed in slice order, then the bias (moe_route's top-k kernel and
// the fused decode routing both take their logits from here, so they agree
// bit for bit).  Up to 32 loads per lane in flight; row and slice offsets are
// wave-uniform (scalar), expert offsets per lane.
template <int PER>
QMOE_D void row_logits(const RouteParams& P, int t, float (&v)[PER]) {
  constexpr int SC = PER >= 16 ? 1 : 32 / PER;  // K-slices per batch of loads
  const int lane = threadIdx.x & 63;
  const float* rowp = P.part + (size_t)t * P.E;
  const size_t slice = (size_t)P.T * P.E;
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = 0.f;
  for (int s0 = 0; s0 < P.KS; s0 += SC) {
    float pv[SC][PER];
#pragma unroll
    for (int u = 0; u < SC; ++u) {
      const float* sp = rowp + (size_t)min(s0 + u, P.KS - 1) * slice;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        pv[u][i] = load_coherent(sp + (uint32_t)min(lane + 64 * i, P.E - 1));
    }
#pragma unroll
    for (int u = 0; u < SC; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (s0 + u < P.KS) v[i] += pv[u][i];
  }
  if (P.bias) {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] += P.bias[min(lane + 64 * i, P.E - 1)];
  }
}

inline void route_split(int T, int H, int& KS, int& ks_len) {
  if (T > kGemvRowsMax) { KS = 1; ks_len = H; return; }
  // K-slices of 1024 values (multiple of 256), capped so T*ks_len*4 <= 64 KiB
  // (the staged slice of every row fits a block's default LDS limit)
  ks_len = 1024;
  while (ks_len > 256 && (size_t)T * ks_len * 4 > 65536) ks_len /= 2;
  KS = (H + ks_len - 1) / ks_len;
}

}  // namespace qmoe
