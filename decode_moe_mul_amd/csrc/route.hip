// moe_route: router logits, top-k with ties to the lower id, renormalised
// softmax over the kept logits, always-on shared experts appended.
// ([P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析: a light
// router picks 10 of 512 experts per token; [P4] "DwarfStar on 8x L40S",
// section 快速上手: a shared expert beside the routed ones.)
//
// Kernels:
//  router_gemv_kernel  rows <= 16: 16 waves per block, each streaming one
//                      expert row of Wr over a K-slice against all rows
//                      staged in LDS; split-K partials go to the workspace.
//  router_gemm_kernel  longer chunks: 64x64 output tiles on the matrix cores
//                      (fp32 operands and sums).
//  topk_kernel         one wave per row: sums the split-K partials in fixed
//                      order, adds the bias, selects k by repeated wave
//                      arg-max, softmax over the kept logits.
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

// x[:, k0:k0+len] -> xsl [T][ks_len], float4 granules, 4 loads in flight
template <int DT, int NT>
QMOE_D void stage_x_slice(const RouteParams& P, int k0, int len, float* xsl) {
  const int l4 = len >> 2, n4 = P.T * l4;
  for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * NT) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + u * NT, n4 - 1);  // unconditional loads
      const int t = i / l4, j = 4 * (i - t * l4);
      v[u] = load_act4<DT>(P.x, (size_t)t * P.H + k0 + j);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT;
      if (i < n4) {
        const int t = i / l4, j = 4 * (i - t * l4);
        *(float4*)(xsl + t * P.ks_len + j) = v[u];
      }
    }
  }
}

// Device-coherent scalar access for values handed between blocks of one
// launch: agent-scope relaxed atomics, i.e. stores written through and loads
// served past the per-XCD L2, so that no cache-wide write-back or invalidate
// (what a device fence costs) is needed.
QMOE_D void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
QMOE_D float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This thread's outstanding vector-memory operations have completed (its
// written-through stores are visible device-wide) before it goes on.
QMOE_D void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Block (b, ks) of the split-K router: wave w handles expert 16b+w over values
// [ks*ks_len, (ks+1)*ks_len) of the hidden dimension (ks_len <= 1024, a
// multiple of 256) and writes its partial dot products for all T rows to
// part[ks][t][e] (written through when COH).  The weight row is requested
// before x is staged, so both loads are in flight together.  Every thread
// returns (no early exit), so callers may synchronise afterwards.
template <bool COH>
QMOE_D void router_partials(const RouteParams& P, float* xsl) {
  const int ks = blockIdx.y;
  const int k0 = ks * P.ks_len;
  const int len = min(P.ks_len, P.H - k0);
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kGemvExperts + (threadIdx.x >> 6);
  const bool has_e = e < P.E;
  const float* wrow = P.Wr + (size_t)min(e, P.E - 1) * P.H + k0;
  float4 w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = 4 * lane + 256 * u;
    w[u] = j < len ? *(const float4*)(wrow + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (P.x_dtype == QMOE_F32)
    stage_x_slice<QMOE_F32, kGemvBlock>(P, k0, len, xsl);
  else
    stage_x_slice<QMOE_BF16, kGemvBlock>(P, k0, len, xsl);
  __syncthreads();
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

__global__ __launch_bounds__(kGemvBlock) void router_gemv_kernel(RouteParams P) {
  extern __shared__ __align__(16) float xsl[];  // [T][ks_len]
  router_partials<false>(P, xsl);
}

// 64 x 64 tile of logits (rows x experts) on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32, fp32 products and sums).  Wave w computes rows
// 32 (w >> 1) .. and experts 32 (w & 1) .. of the tile as 2 x 2 blocks of
// 16 x 16.  Per 16-wide chunk of H each lane loads 4 consecutive values of
// its row of x and of its expert's row of Wr; op s of the chunk takes value s
// of every lane group, so both operands walk the chunk's 16 indices in the
// same interleaved order.  Four chunks of loads are in flight.
constexpr int kGT = 64, kGE = 64, kGDepth = 4;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
QMOE_D void rg_load(const RouteParams& P, const int (&trow)[2], const int (&erow)[2], int k,
                    float4 (&a)[2], float4 (&b)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = load_act4<DT>(P.x, (size_t)trow[i] * P.H + k);
    b[i] = *(const float4*)(P.Wr + (size_t)erow[i] * P.H + k);
  }
}

template <int DT>
__global__ __launch_bounds__(kRouteBlock) void router_gemm_kernel(RouteParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int tb = blockIdx.y * kGT + 32 * (wave >> 1), eb = blockIdx.x * kGE + 32 * (wave & 1);
  // operand rows, clamped: rows past the end re-read the last one (dropped)
  int trow[2], erow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    trow[i] = min(tb + 16 * i + r, P.T - 1);
    erow[i] = min(eb + 16 * i + r, P.E - 1);
  }
  const int nch = (P.H + 15) / 16;
  // this lane's 4 values of chunk c start at k; past H (when H % 16 != 0)
  // the load re-reads the last 4 and the values are zeroed
  auto k_of = [&](int c) { return min(16 * c + 4 * kg, P.H - 4); };
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float4 ra[kGDepth][2], rb[kGDepth][2];
#pragma unroll
  for (int u = 0; u < kGDepth; ++u) rg_load<DT>(P, trow, erow, k_of(min(u, nch - 1)), ra[u], rb[u]);
  for (int c0 = 0; c0 < nch; c0 += kGDepth) {
#pragma unroll
    for (int u = 0; u < kGDepth; ++u) {
      const int c = c0 + u;
      const bool valid = c < nch && 16 * c + 4 * kg < P.H;
      float4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = valid ? ra[u][i] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[i] = rb[u][i];
      }
      rg_load<DT>(P, trow, erow, k_of(min(c + kGDepth, nch - 1)), ra[u], rb[u]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].x, b[j].x, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].y, b[j].y, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].z, b[j].z, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].w, b[j].w, acc[i][j], 0, 0, 0);
        }
    }
  }
  // lane holds rows 4 kg + q of each 16 x 16 block, column r
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = tb + 16 * i + 4 * kg + q, e = eb + 16 * j + r;
        if (t < P.T && e < P.E) P.part[(size_t)t * P.E + e] = acc[i][j][q];
      }
}

// Order-preserving unsigned image of a logit (NaN ranks as -inf); every
// number maps above 0, which marks taken / absent slots.
QMOE_D uint32_t order_key(float f) {
  if (f != f) f = -INFINITY;
  const uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Top-k of one row of E logits held by one wave (lane l holds experts
// l + 64 i in raw[i]): k rounds of a wave arg-max (DPP max of the keys, then
// DPP min of the ids that hold it, so ties go to the lower id).  Lane s < k
// gets the s-th id and its logit.
template <int PER>  // E <= 64 * PER
QMOE_D void wave_topk(const float (&raw)[PER], int E, int k, int& my_id, float& my_raw) {
  const int lane = threadIdx.x & 63;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = lane + 64 * i < E ? order_key(raw[i]) : 0u;
  my_id = 0;
  my_raw = 0.f;
  for (int s = 0; s < k; ++s) {
    uint32_t kb = 0u, ib = 0xFFFFFFFFu;
    float rb = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)  // ascending ids, strict: lowest id on ties
      if (key[i] > kb) { kb = key[i]; ib = (uint32_t)(lane + 64 * i); rb = raw[i]; }
    const uint32_t kmax = wave_max_u32(kb);
    const uint32_t wid = wave_min_u32(kb == kmax ? ib : 0xFFFFFFFFu);
    const float rsel = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rb), (int)(wid & 63u)));
    if ((int)(wid & 63u) == lane) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == (int)(wid >> 6)) key[i] = 0u;
    }
    if (lane == s) { my_id = (int)wid; my_raw = rsel; }
  }
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

// Final logits of row t, expert e: split-K partials summed in order + bias.
QMOE_D float final_logit(const RouteParams& P, int t, int e) {
  float v = 0.f;
  for (int s0 = 0; s0 < P.KS; s0 += 8) {
    float pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      pv[u] = s0 + u < P.KS
                  ? P.part[((size_t)(s0 + u) * P.T + t) * P.E + e]
                  : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < P.KS) v += pv[u];
  }
  if (P.bias) v += P.bias[e];
  return v;
}

template <int PER>  // values per lane: E <= 64 * PER
__global__ __launch_bounds__(kRouteBlock) void topk_kernel(RouteParams P) {
  __shared__ float row[4][64 * PER];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= P.T) return;
  constexpr int C = PER < 8 ? PER : 8;  // experts per lane whose loads fly together
#pragma unroll
  for (int i0 = 0; i0 < PER; i0 += C) {
    float v[C];
#pragma unroll
    for (int i = 0; i < C; ++i) v[i] = final_logit(P, t, min(lane + 64 * (i0 + i), P.E - 1));
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int e = lane + 64 * (i0 + i);
      if (e < P.E) {
        row[wave][e] = v[i];
        if (P.logits) P.logits[(size_t)t * P.E + e] = v[i];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  float raw[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) raw[i] = lane + 64 * i < P.E ? row[wave][lane + 64 * i] : 0.f;
  int my_id;
  float my_raw;
  wave_topk<PER>(raw, P.E, P.k, my_id, my_raw);
  write_topk(P, t, my_id, my_raw, nullptr);
}

// ------------------------------------------- fused decode routing -------
// router_partials -> final logits -> top-k -> permutation in one launch for
// up to 16 rows.  The block that completes last (a device-scope counter in
// the workspace decides) gives one wave to each row: the wave sums that row's
// split-K partials in order (as final_logit does), takes its top-k and
// writes ids/p; the block then sorts the assignments.  Partials are written
// through and read past L2 (store_coherent/load_coherent) and each thread
// drains its stores before the block's counter increment, so no device-wide
// fence (an L2 write-back plus invalidate per wave) is needed.  The finishing
// block resets the counter, so it starts and ends at zero.
struct RouteDecodeParams {
  RouteParams r;
  unsigned* ctr;       // [1]
  int32_t* offsets;    // [E_total + 1]
  int32_t* perm;       // [T * kt]
  int32_t* inv;        // [T * kt]
  int E_total, W, nbits;
};

constexpr int kDecodeLdsInts = 8192;  // LDS ints of the fused kernel (32 KiB)

// Final logits of row t for the lane's experts e = lane + 64 i: the KS
// partials summed in slice order, then the bias (final_logit's order, so the
// values equal moe_route's bit for bit).  Up to 32 loads per lane in flight;
// row and slice offsets are wave-uniform (scalar), expert offsets per lane.
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

template <int PER>
__global__ __launch_bounds__(kGemvBlock) void route_decode_kernel(RouteDecodeParams D) {
  extern __shared__ __align__(16) float smem[];
  __shared__ int last;
  const RouteParams& P = D.r;
  router_partials<true>(P, smem);
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0)
    last = atomicAdd(&D.ctr[0], 1u) == gridDim.x * gridDim.y - 1u;
  __syncthreads();
  if (!last) return;
  const int kt = P.k + P.n_shared, A = P.T * kt;
  int32_t* ids_l = (int32_t*)smem;  // [A]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = wave; t < P.T; t += kGemvBlock / 64) {  // one row per wave
    float raw[PER];
    row_logits<PER>(P, t, raw);
    if (P.logits) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (lane + 64 * i < P.E) P.logits[(size_t)t * P.E + lane + 64 * i] = raw[i];
    }
    int my_id;
    float my_raw;
    wave_topk<PER>(raw, P.E, P.k, my_id, my_raw);
    write_topk(P, t, my_id, my_raw, ids_l);
  }
  __syncthreads();
  int* hist = (int*)smem + ((A + 63) & ~63);
  permute_block<kGemvBlock>(ids_l, A, D.E_total, D.W, D.nbits, D.offsets, D.perm, D.inv, hist,
                             hist + D.W * D.E_total);
  if (threadIdx.x == 0)
    __hip_atomic_store(&D.ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    const dim3 grid((E + kGemvExperts - 1) / kGemvExperts, P.KS);
    st = QMOE_LAUNCH("router_gemv", router_gemv_kernel, grid, kGemvBlock,
                     (size_t)T * P.ks_len * sizeof(float), s, P);
  } else {
    const dim3 grid((E + kGE - 1) / kGE, (T + kGT - 1) / kGT);
    st = x_dtype == QMOE_F32
             ? QMOE_LAUNCH("router_gemm", router_gemm_kernel<QMOE_F32>, grid, kRouteBlock, 0, s, P)
             : QMOE_LAUNCH("router_gemm", router_gemm_kernel<QMOE_BF16>, grid, kRouteBlock, 0, s, P);
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

// Fused decode routing: the block counter, then the split-K partials
constexpr size_t kDecodeCtrBytes = 256;

size_t moe_route_decode_workspace_size(int T, int H, int E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  return kDecodeCtrBytes + round_up256((size_t)KS * T * E * sizeof(float));
}

int moe_route_decode(const void* x, int x_dtype, int T, int H, const float* Wr,
                     const float* bias, int E, int k, int n_shared, int32_t* ids, float* p,
                     float* logits, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                     size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || k > 64 || n_shared < 0)
    return fail(QMOE_ERR_INVALID_ARG,
                "moe_route_decode: bad sizes T=%d H=%d E=%d k=%d n_shared=%d", T, H, E, k,
                n_shared);
  if (T > kGemvRowsMax)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_route_decode: T=%d > %d rows", T, kGemvRowsMax);
  if (E > 512) return fail(QMOE_ERR_UNSUPPORTED, "moe_route_decode: E=%d > 512", E);
  if (H % 4) return fail(QMOE_ERR_INVALID_ARG, "moe_route_decode: H %% 4 != 0");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_route_decode: unknown x_dtype %d", x_dtype);
  const int kt = k + n_shared, E_total = E + n_shared, A = T * kt;
  const int hist_ints = kDecodeLdsInts - ((A + 63) & ~63) - kGemvBlock / 64;
  if (hist_ints < E_total)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_route_decode: T*(k+n_shared)=%d with %d experts "
                "does not fit the fused permutation", A, E_total);
  if (!offsets) return fail(QMOE_ERR_INVALID_ARG, "moe_route_decode: null offsets");
  if (T == 0)  // nothing to route; the empty permutation still zeroes offsets
    return moe_permute(nullptr, 0, kt, E_total, offsets, nullptr, nullptr, stream);
  if (!x || !Wr || !ids || !p || !perm || !inv_perm)
    return fail(QMOE_ERR_INVALID_ARG, "moe_route_decode: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(Wr, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_route_decode: misaligned x/Wr");
  const size_t need = moe_route_decode_workspace_size(T, H, E);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_route_decode: workspace %zu < %zu (or misaligned)",
                ws_bytes, need);
  uint8_t* w = (uint8_t*)ws;
  RouteDecodeParams D{};
  D.r = RouteParams{x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids, p, logits, nullptr, 0, 0};
  route_split(T, H, D.r.KS, D.r.ks_len);
  D.ctr = (unsigned*)w;
  D.r.part = (float*)(w + kDecodeCtrBytes);
  D.offsets = offsets;
  D.perm = perm;
  D.inv = inv_perm;
  D.E_total = E_total;
  D.W = permute_waves(A, E_total, hist_ints, kGemvBlock / 64);
  D.nbits = id_bits(E_total);
  const dim3 grid((E + kGemvExperts - 1) / kGemvExperts, D.r.KS);
  const size_t lds = (size_t)kDecodeLdsInts * 4;
  hipStream_t s = (hipStream_t)stream;
  const int per = (E + 63) / 64;
#define QMOE_ROUTE_DECODE(PERV) \
  return QMOE_LAUNCH("route_decode", route_decode_kernel<PERV>, grid, kGemvBlock, lds, s, D)
  if (per <= 1) QMOE_ROUTE_DECODE(1);
  if (per <= 2) QMOE_ROUTE_DECODE(2);
  if (per <= 4) QMOE_ROUTE_DECODE(4);
  QMOE_ROUTE_DECODE(8);
#undef QMOE_ROUTE_DECODE
}

}  // extern "C"

