// Decode-side quantized GEMV: qgemv_<fmt> (dense, [P3] "RTX 3090 Llama 70B
// three-tier cache" section 4.4) and the two phases of moe_ffn_tiered (routed
// experts in mixed-precision tiers, [P2] "Three RTX 3090 Qwen3.8-Flash-Next
// guide" sections 优化策略二/三 and bug item 4; many session rows per launch,
// [P4] "DwarfStar on 8x L40S" section "120 t/s 的秘密微批次分组解码").
//
// Work decomposition (one block = 4 waves):
//  * a weight row is reduced by G lanes (G = largest power of two <= 64 that
//    divides the row's 32-value unit count), so every lane owns whole
//    32-value units and a wave covers 64/G rows;
//  * each lane streams its units straight from HBM (16 B of codes per unit
//    for 4-bit formats), decodes them to exact fp16 pairs and dots them with
//    activations staged once per block in LDS (fp16, in the format's pair
//    order); the unit scale is applied once per unit in fp32;
//  * the rows of a token chunk (up to 16 rows) share one pass over the
//    weights; longer row lists loop over chunks;
//  * gate and up rows of the same output are computed by the same lanes, so
//    SiLU(g) * u is applied in registers before anything is stored.
#include "common.hpp"

namespace qmoe {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kXCap = 16384;  // fp16 activation values staged per block

struct Mat {
  const uint8_t* p0;
  const uint8_t* p1;
  const uint8_t* p2;
  const uint8_t* p3;
};

QMOE_D Mat mat_of(const void* base, int fmt, int N, int K) {
  const Layout L = layout_of(fmt, N, K);
  const uint8_t* b = (const uint8_t*)base;
  return {b + L.off[0], b + L.off[1], b + L.off[2], b + L.off[3]};
}

// Load unit u (values 32u..32u+31) of row `row` and decode it: 16 fp16-pair
// code words plus the fp32 coefficients of the unit.
//   Q8_0/Q4_0/MXFP4: value = c0 * code
//   Q4_K: value = c0 * code - c1          (c1 multiplies the sum of x)
//   Q6_K: value = c0 * code (first 16), c1 * code (last 16)
template <int FMT>
QMOE_D void load_unit(const Mat& M, int row, int u, int K, uint32_t codes[16], float& c0,
                      float& c1) {
  const size_t nb32 = (size_t)(K >> 5);
  if constexpr (FMT == QMOE_Q8_0) {
    const uint4* q = (const uint4*)(M.p0 + (size_t)row * K + 32 * (size_t)u);
    const uint4 a = q[0], b = q[1];
    const uint32_t d = ((const uint16_t*)M.p1)[row * nb32 + u];
    bytes_to_h2(a, b, codes);
    c0 = f16_bits_to_f32(d);
    c1 = 0.f;
  } else if constexpr (FMT == QMOE_Q4_0) {
    const uint4 q = *(const uint4*)(M.p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const uint32_t d = ((const uint16_t*)M.p1)[row * nb32 + u];
    nibbles_to_h2(q, H2_NEG_1032, codes);
    c0 = f16_bits_to_f32(d);
    c1 = 0.f;
  } else if constexpr (FMT == QMOE_MXFP4) {
    const uint4 q = *(const uint4*)(M.p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const uint32_t e = M.p1[row * nb32 + u];
    e2m1_to_h2(q, codes);
    c0 = e8m0_to_f32(e);
    c1 = 0.f;
  } else if constexpr (FMT == QMOE_Q4_K) {
    const uint4 q = *(const uint4*)(M.p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const uint4 meta = ((const uint4*)M.p1)[(size_t)row * (K >> 8) + (u >> 3)];
    const int j = u & 7;
    const uint64_t lo = (uint64_t)meta.y | ((uint64_t)meta.z << 32);
    const uint64_t hi = (uint64_t)meta.z | ((uint64_t)meta.w << 32);
    const float sc = (float)((lo >> (6 * j)) & 63u);
    const float mn = (float)((hi >> (16 + 6 * j)) & 63u);
    nibbles_to_h2(q, H2_NEG_1024, codes);
    c0 = f16_bits_to_f32(meta.x & 0xFFFFu) * sc;
    c1 = f16_bits_to_f32(meta.x >> 16) * mn;
  } else {  // Q6_K
    const uint4 ql = *(const uint4*)(M.p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const uint2 qh = *(const uint2*)(M.p1 + (size_t)row * (K >> 2) + 8 * (size_t)u);
    const size_t sb = (size_t)row * (K >> 8) + (u >> 3);
    const uint32_t sc2 = ((const uint16_t*)(M.p2 + 16 * sb))[u & 7];
    const float d = f16_bits_to_f32(((const uint16_t*)M.p3)[sb]);
    q6_to_h2(ql, qh, codes);
    c0 = d * (float)(int8_t)(sc2 & 0xFFu);
    c1 = d * (float)(int8_t)(sc2 >> 8);
  }
}

// acc[r] += <unit u of the row, staged activations of row r>
template <int FMT, int RC>
QMOE_D void unit_mac(const uint32_t codes[16], float c0, float c1, const uint32_t* xs,
                     const float* sx, int ul, int U, float (&acc)[RC]) {
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const uint4* xp = (const uint4*)(xs + ((size_t)r * U + ul) * 16);
    const uint4 v0 = xp[0], v1 = xp[1], v2 = xp[2], v3 = xp[3];
    const uint32_t xv[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                             v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
    float s0 = 0.f, s1 = 0.f;
    if constexpr (FMT == QMOE_Q6_K) {
#pragma unroll
      for (int p = 0; p < 8; ++p) s0 = fdot2(codes[p], xv[p], s0);
#pragma unroll
      for (int p = 8; p < 16; ++p) s1 = fdot2(codes[p], xv[p], s1);
      acc[r] += c0 * s0 + c1 * s1;
    } else {
#pragma unroll
      for (int p = 0; p < 16; p += 2) {
        s0 = fdot2(codes[p], xv[p], s0);
        s1 = fdot2(codes[p + 1], xv[p + 1], s1);
      }
      acc[r] += c0 * (s0 + s1);
      if constexpr (FMT == QMOE_Q4_K) acc[r] -= c1 * sx[r * U + ul];
    }
  }
}

// Stage activation rows into LDS: for rows r < rc and units ul < U of the
// chunk starting at value k0, 16 fp16-pair words in the format's pair order,
// plus the fp32 sum of the unit's 32 values.  `src(r)` gives the row pointer
// (element 0 of the full-length row) and its dtype is `dtype`.
template <bool BYTE_PAIRS, class Src>
QMOE_D void stage_rows(uint32_t* xs, float* sx, int rc, int U, int k0, Src src, int dtype) {
  for (int idx = threadIdx.x; idx < rc * U; idx += kBlock) {
    const int r = idx / U, ul = idx - r * U;
    const void* row = src(r);
    float v[32];
    if (dtype == QMOE_F32) {
      const float4* p = (const float4*)((const float*)row + k0 + 32 * ul);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = p[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
      const uint4* p = (const uint4*)((const uint16_t*)row + k0 + 32 * ul);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 b = p[i];
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
          v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        }
      }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += v[i];
    sx[idx] = s;
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int e0 = BYTE_PAIRS ? pair_elem_byte(p, 0) : pair_elem_nibble(p, 0);
      const int e1 = BYTE_PAIRS ? pair_elem_byte(p, 1) : pair_elem_nibble(p, 1);
      w[p] = pack_h2(v[e0], v[e1]);
    }
    uint4* dst = (uint4*)(xs + (size_t)idx * 16);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    dst[2] = make_uint4(w[8], w[9], w[10], w[11]);
    dst[3] = make_uint4(w[12], w[13], w[14], w[15]);
  }
}

QMOE_D float group_sum_rt(float v, int G) {
  for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One block computes `rows` (row0 .. row0 + rows_per_block - 1) of NMAT
// matrices [N, K] against up to RC staged activation rows, for all K chunks.
// `src(r)` yields activation row r of the chunk; `sink(n, r, acc)` receives the
// finished dot products (called by one lane per row).
template <int FMT, int NMAT, int RC, class Src, class Sink>
QMOE_D void gemv_chunk(const Mat (&mats)[NMAT], int N, int K, int row, int g, int G,
                       int rc, int kc, int dtype, uint32_t* xs, float* sx, Src src,
                       Sink sink) {
  float acc[NMAT][RC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[m][r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kc) {
    const int kcur = min(kc, K - k0);
    const int U = kcur >> 5;
    __syncthreads();  // previous users of xs are done
    stage_rows<byte_order(FMT)>(xs, sx, rc, U, k0, src, dtype);
    __syncthreads();
    if (row < N) {
      const int ub = k0 >> 5;
      for (int ul = g; ul < U; ul += G) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          uint32_t codes[16];
          float c0, c1;
          load_unit<FMT>(mats[m], row, ub + ul, K, codes, c0, c1);
          unit_mac<FMT, RC>(codes, c0, c1, xs, sx, ul, U, acc[m]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[m][r] = group_sum_rt(acc[m][r], G);
  if (row < N && g == 0) {
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      if (r < rc) {
        float a[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) a[m] = acc[m][r];
        sink(row, r, a);
      }
    }
  }
}

// Run gemv_chunk for `rows_total` activation rows in chunks of at most rcl,
// picking the register-blocking RC (1, 2, 4, 8, 16) per chunk.
template <int FMT, int NMAT, class SrcOf, class SinkOf>
QMOE_D void gemv_rows(const Mat (&mats)[NMAT], int N, int K, int row, int g, int G,
                      int rows_total, int rcl, int kc, int dtype, uint32_t* xs, float* sx,
                      SrcOf src_of, SinkOf sink_of) {
  for (int c0 = 0; c0 < rows_total; c0 += rcl) {
    const int rc = min(rcl, rows_total - c0);
    auto src = [&](int r) { return src_of(c0 + r); };
    auto sink = [&](int n, int r, const float* a) { sink_of(n, c0 + r, a); };
    if (rc == 1)
      gemv_chunk<FMT, NMAT, 1>(mats, N, K, row, g, G, rc, kc, dtype, xs, sx, src, sink);
    else if (rc == 2)
      gemv_chunk<FMT, NMAT, 2>(mats, N, K, row, g, G, rc, kc, dtype, xs, sx, src, sink);
    else if (rc <= 4)
      gemv_chunk<FMT, NMAT, 4>(mats, N, K, row, g, G, rc, kc, dtype, xs, sx, src, sink);
    else if (rc <= 8)
      gemv_chunk<FMT, NMAT, 8>(mats, N, K, row, g, G, rc, kc, dtype, xs, sx, src, sink);
    else
      gemv_chunk<FMT, NMAT, 16>(mats, N, K, row, g, G, rc, kc, dtype, xs, sx, src, sink);
  }
}

// ----------------------------------------------------------- qgemv ------
struct GemvParams {
  const void* W;
  int N, K;
  const void* x;
  int x_dtype, R;
  float* y;
  int G, rcl, kc;
};

template <int FMT>
__global__ __launch_bounds__(kBlock) void qgemv_kernel(GemvParams P) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int G = P.G, sub = 64 / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (blockIdx.x * kWaves + wave) * sub + lane / G;
  const int g = lane & (G - 1);
  uint32_t* xs = smem;
  float* sx = (float*)(smem + (size_t)P.rcl * P.kc / 2);
  const Mat mats[1] = {mat_of(P.W, FMT, P.N, P.K)};
  const int esz = P.x_dtype == QMOE_F32 ? 4 : 2;
  gemv_rows<FMT, 1>(
      mats, P.N, P.K, row, g, G, P.R, P.rcl, P.kc, P.x_dtype, xs, sx,
      [&](int r) { return (const void*)((const char*)P.x + (size_t)r * P.K * esz); },
      [&](int n, int r, const float* a) { P.y[(size_t)r * P.N + n] = a[0]; });
}

// ------------------------------------------------------- routed FFN -----
struct FfnParams {
  qmoe_tier tiers[QMOE_MAX_TIERS];
  int n_tiers, E, H, F, T, k;
  const void* x;
  int x_dtype;
  const int32_t* offsets;
  const int32_t* perm;
  float* h;  // [T*k, F] workspace (SwiGLU output, permuted rows)
  float* o;  // [T*k, H]
  int ntiles, G, rcl, kc;
};

// The expert whose first permuted position is `slot`, or -1.  Positions of
// expert e are offsets[e] .. offsets[e+1]-1; ids outside [0, E) never got a
// position, so they are never visited ([P2] bug items 1 and 3).
QMOE_D int expert_at(const int32_t* offsets, int E, int slot) {
  if (slot >= offsets[E]) return -1;
  int lo = 0, hi = E;  // invariant: offsets[lo] <= slot
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= slot) lo = mid; else hi = mid;
  }
  return offsets[lo] == slot ? lo : -1;
}

QMOE_D const qmoe_tier* tier_of(const FfnParams& P, int e) {
  for (int i = 0; i < P.n_tiers; ++i)
    if (e >= P.tiers[i].e_begin && e < P.tiers[i].e_end) return &P.tiers[i];
  return nullptr;
}

QMOE_D float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

template <int FMT>
QMOE_D void ffn_gate_up_body(const FfnParams& P, const qmoe_tier* t, int e, int pos0, int m,
                             int tile, uint32_t* xs, float* sx) {
  const int G = P.G, sub = 64 / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (tile * kWaves + wave) * sub + lane / G;
  const int g = lane & (G - 1);
  const size_t stride = layout_of(FMT, P.F, P.H).total;
  const size_t eo = (size_t)(e - t->e_begin) * stride;
  const Mat mats[2] = {mat_of((const uint8_t*)t->gate + eo, FMT, P.F, P.H),
                       mat_of((const uint8_t*)t->up + eo, FMT, P.F, P.H)};
  const int esz = P.x_dtype == QMOE_F32 ? 4 : 2;
  gemv_rows<FMT, 2>(
      mats, P.F, P.H, row, g, G, m, P.rcl, P.kc, P.x_dtype, xs, sx,
      [&](int r) {
        const int tok = P.perm[pos0 + r] / P.k;
        return (const void*)((const char*)P.x + (size_t)tok * P.H * esz);
      },
      [&](int n, int r, const float* a) {
        P.h[(size_t)(pos0 + r) * P.F + n] = silu_mul(a[0], a[1]);
      });
}

template <int FMT>
QMOE_D void ffn_down_body(const FfnParams& P, const qmoe_tier* t, int e, int pos0, int m,
                          int tile, uint32_t* xs, float* sx) {
  const int G = P.G, sub = 64 / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (tile * kWaves + wave) * sub + lane / G;
  const int g = lane & (G - 1);
  const size_t stride = layout_of(FMT, P.H, P.F).total;
  const Mat mats[1] = {mat_of((const uint8_t*)t->down + (size_t)(e - t->e_begin) * stride,
                              FMT, P.H, P.F)};
  gemv_rows<FMT, 1>(
      mats, P.H, P.F, row, g, G, m, P.rcl, P.kc, QMOE_F32, xs, sx,
      [&](int r) { return (const void*)(P.h + (size_t)(pos0 + r) * P.F); },
      [&](int n, int r, const float* a) { P.o[(size_t)(pos0 + r) * P.H + n] = a[0]; });
}

// PHASE 0: gate/up + SwiGLU -> h;  PHASE 1: down -> o.
template <int PHASE>
__global__ __launch_bounds__(kBlock) void ffn_decode_kernel(FfnParams P) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int slot = blockIdx.x / P.ntiles, tile = blockIdx.x - slot * P.ntiles;
  const int e = expert_at(P.offsets, P.E, slot);
  if (e < 0) return;
  const qmoe_tier* t = tier_of(P, e);
  if (!t) return;
  const int m = P.offsets[e + 1] - slot;
  uint32_t* xs = smem;
  float* sx = (float*)(smem + (size_t)P.rcl * P.kc / 2);
  const int fmt = PHASE == 0 ? t->fmt_gate_up : t->fmt_down;
#define QMOE_FFN_CASE(F)                                                   \
  case F:                                                                  \
    if (PHASE == 0) ffn_gate_up_body<F>(P, t, e, slot, m, tile, xs, sx);   \
    else ffn_down_body<F>(P, t, e, slot, m, tile, xs, sx);                 \
    break;
  switch (fmt) {
    QMOE_FFN_CASE(QMOE_Q8_0)
    QMOE_FFN_CASE(QMOE_Q4_0)
    QMOE_FFN_CASE(QMOE_MXFP4)
    QMOE_FFN_CASE(QMOE_Q4_K)
    QMOE_FFN_CASE(QMOE_Q6_K)
    default: break;
  }
#undef QMOE_FFN_CASE
}

// ------------------------------------------------------ host helpers ----
// Lanes per weight row: the largest power of two <= 64 dividing K/32.
static int lanes_per_row(int K) {
  const int units = K / 32;
  int G = 1;
  while (G < 64 && units % (2 * G) == 0) G *= 2;
  return G;
}

// Activation rows per chunk and values per K-chunk for a given row count.
static void chunking(int rows, int K, int G, int& rcl, int& kc) {
  rcl = 1;
  while (rcl < 16 && rcl < rows) rcl *= 2;
  kc = K;
  if ((size_t)rcl * K > (size_t)kXCap) {
    kc = kXCap / rcl;
    const int step = 32 * G;
    kc = kc >= step ? kc / step * step : kc / 32 * 32;
  }
}

static size_t smem_bytes(int rcl, int kc) {
  return (size_t)rcl * kc * 2 + (size_t)rcl * (kc / 32) * 4;
}

static bool bad_fmt(int fmt) { return fmt < QMOE_Q8_0 || fmt > QMOE_Q6_K; }

static int qgemv_launch(int FMT, const void* W, int N, int K, const void* x, int x_dtype,
                        int R, float* y, void* stream) {
  if (!W || !x || !y) return fail(QMOE_ERR_INVALID_ARG, "qgemv: null pointer");
  if (N < 0 || K <= 0 || R < 0 || K % block_of(FMT) || K > 65536)
    return fail(QMOE_ERR_INVALID_ARG, "qgemv: bad sizes N=%d K=%d R=%d", N, K, R);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "qgemv: unknown x_dtype %d", x_dtype);
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(y, 4))
    return fail(QMOE_ERR_INVALID_ARG, "qgemv: misaligned pointer");
  if (N == 0 || R == 0) return QMOE_OK;
  GemvParams P{W, N, K, x, x_dtype, R, y, 0, 0, 0};
  P.G = lanes_per_row(K);
  chunking(R, K, P.G, P.rcl, P.kc);
  const int rows_per_block = kWaves * (64 / P.G);
  const dim3 grid((N + rows_per_block - 1) / rows_per_block);
  const size_t lds = smem_bytes(P.rcl, P.kc);
  hipStream_t s = (hipStream_t)stream;
  switch (FMT) {
    case QMOE_Q8_0: return QMOE_LAUNCH("qgemv", qgemv_kernel<QMOE_Q8_0>, grid, kBlock, lds, s, P);
    case QMOE_Q4_0: return QMOE_LAUNCH("qgemv", qgemv_kernel<QMOE_Q4_0>, grid, kBlock, lds, s, P);
    case QMOE_MXFP4: return QMOE_LAUNCH("qgemv", qgemv_kernel<QMOE_MXFP4>, grid, kBlock, lds, s, P);
    case QMOE_Q4_K: return QMOE_LAUNCH("qgemv", qgemv_kernel<QMOE_Q4_K>, grid, kBlock, lds, s, P);
    default: return QMOE_LAUNCH("qgemv", qgemv_kernel<QMOE_Q6_K>, grid, kBlock, lds, s, P);
  }
}

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);

}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qgemv_q8_0(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q8_0, W, N, K, x, d, R, y, s);
}
int qgemv_q4_0(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q4_0, W, N, K, x, d, R, y, s);
}
int qgemv_mxfp4(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_MXFP4, W, N, K, x, d, R, y, s);
}
int qgemv_q4_k(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q4_K, W, N, K, x, d, R, y, s);
}
int qgemv_q6_k(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q6_K, W, N, K, x, d, R, y, s);
}

size_t moe_ffn_workspace_size(int T, int k, int F) {
  if (T < 0 || k < 0 || F < 0) return 0;
  return round_up256((size_t)T * k * F * sizeof(float)) + 256;
}

int moe_ffn_tiered(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, const void* x,
                   int x_dtype, int T, int k, const int32_t* offsets, const int32_t* perm,
                   float* o, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 0) return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: T=%d k=%d", T, k);
  if (T == 0 || k == 0) return QMOE_OK;
  int st = validate_tiers(tiers, n_tiers, E, H, F, false);
  if (st) return st;
  if (!x || !offsets || !perm || !o)
    return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: null pointer");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: unknown x_dtype %d", x_dtype);
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(o, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: misaligned x/o");
  const size_t need = moe_ffn_workspace_size(T, k, F);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_ffn_tiered: workspace %zu < %zu (or misaligned)",
                ws_bytes, need);
  const long long A = (long long)T * k;
  if (A > (1 << 24)) return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: T*k too large");
  hipStream_t s = (hipStream_t)stream;
  FfnParams P{};
  for (int i = 0; i < n_tiers; ++i) P.tiers[i] = tiers[i];
  P.n_tiers = n_tiers; P.E = E; P.H = H; P.F = F; P.T = T; P.k = k;
  P.x = x; P.x_dtype = x_dtype; P.offsets = offsets; P.perm = perm;
  P.h = (float*)ws; P.o = o;
  // phase 0: gate/up over K = H, rows = F
  P.G = lanes_per_row(H);
  chunking(T, H, P.G, P.rcl, P.kc);
  int rpb = kWaves * (64 / P.G);
  P.ntiles = (F + rpb - 1) / rpb;
  if (A * (long long)((H + 3) / 4) >= (1LL << 31) || A * (long long)P.ntiles >= (1LL << 31))
    return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: grid too large");
  st = QMOE_LAUNCH("ffn_gate_up", ffn_decode_kernel<0>, dim3((unsigned)(A * P.ntiles)), kBlock,
                   smem_bytes(P.rcl, P.kc), s, P);
  if (st) return st;
  // phase 1: down over K = F, rows = H
  P.G = lanes_per_row(F);
  chunking(T, F, P.G, P.rcl, P.kc);
  rpb = kWaves * (64 / P.G);
  P.ntiles = (H + rpb - 1) / rpb;
  return QMOE_LAUNCH("ffn_down", ffn_decode_kernel<1>, dim3((unsigned)(A * P.ntiles)), kBlock,
                     smem_bytes(P.rcl, P.kc), s, P);
}

}  // extern "C"
