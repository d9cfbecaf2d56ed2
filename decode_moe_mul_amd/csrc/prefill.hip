// qgemm_grouped_prefill: the routed-expert FFN for long chunks (a 2048-token
// prefill chunk, [P4] "DwarfStar on 8x L40S", section
// "120 t/s 的秘密微批次分组解码") as a grouped GEMM on the gfx950 matrix cores.
// Prefill turns the per-expert GEMV into a real contraction ([P1] "NInfer 80 SM
// port", section 九.3: group-wise 4/5-bit weights dequantized on chip and fed
// to a bf16 GEMM).
//
// Tiling.  The tokens of expert e (positions offsets[e] .. offsets[e+1]-1 of
// the permutation) are cut into 64-row tiles; a schedule kernel prefix-sums
// the tile counts.  One block (4 waves) computes one 64-row tile against
// 4 * NB * 16 output columns:
//  * activations (x rows gathered through perm, or h rows) are rounded to
//    bf16 and staged in LDS, 256 values of K at a time;
//  * each wave dequantizes its own weight columns straight into the MFMA
//    B-operand registers: lane (n, g) owns 32-value units g and g+4 of the
//    K-chunk of weight row n, so every weight byte is read by one lane only;
//  * v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The contraction order
//    inside a K-chunk is a fixed permutation of K applied identically to the
//    A and B operands.
//  Pass 1 (NMAT = 2): gate and up tiles, SiLU(g) * u -> h (bf16, workspace).
//  Pass 2 (NMAT = 1): down tiles over K = F -> o (fp32, permuted rows).
#include "common.hpp"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPW = 4;              // waves per block
constexpr int kPB = 64 * kPW;       // threads per block
constexpr int kBM = 64;             // rows (tokens) per tile
constexpr int kBK = 256;            // K values per chunk
constexpr int kAStride = kBK + 8;   // LDS row stride in bf16 (pad against conflicts)

struct PrefillParams {
  qmoe_tier tiers[QMOE_MAX_TIERS];
  int n_tiers, E, H, F, T, k;
  const void* x;
  int x_dtype;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tile_off;  // [E+1] prefix sum of 64-row tiles per expert
  uint16_t* h;              // [T*k, F] bf16
  float* o;                 // [T*k, H]
  int ntiles;               // column tiles of this pass
};

// byte I of x as a float (selected into v_cvt_f32_ubyteI)
template <int I>
QMOE_D float ubyte(uint32_t x) { return (float)((x >> (8 * I)) & 0xFFu); }

QMOE_D uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantize unit u (32 values) of weight row `row` of a [N, K] tensor into
// 16 words of bf16 pairs in natural element order (word w = elements 2w,
// 2w+1).  Units at or beyond K give zeros.
template <int FMT>
QMOE_D void dequant_unit_bf16(const uint8_t* base, int N, int K, int row, int u, uint32_t out[16]) {
  if (row >= N || 32 * u >= K) {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0u;
    return;
  }
  const Layout L = layout_of(FMT, N, K);
  const uint8_t* p0 = base + L.off[0];
  const uint8_t* p1 = base + L.off[1];
  const size_t nb32 = (size_t)(K >> 5);
  if constexpr (FMT == QMOE_Q8_0) {
    const uint4* q = (const uint4*)(p0 + (size_t)row * K + 32 * (size_t)u);
    const uint4 a = q[0], b = q[1];
    const float d = f16_bits_to_f32(((const uint16_t*)p1)[row * nb32 + u]);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t ww = w[c] ^ 0x80808080u;  // q + 128
      const float bias = -128.f * d;
      out[2 * c] = pack_bf16(fmaf(ubyte<0>(ww), d, bias),
                             fmaf(ubyte<1>(ww), d, bias));
      out[2 * c + 1] = pack_bf16(fmaf(ubyte<2>(ww), d, bias),
                                 fmaf(ubyte<3>(ww), d, bias));
    }
  } else if constexpr (FMT == QMOE_MXFP4) {
    const uint4 q = *(const uint4*)(p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const float scale = e8m0_to_f32(p1[row * nb32 + u]);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      out[4 * c + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 0));
      out[4 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 1));
      out[4 * c + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 2));
      out[4 * c + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 3));
    }
  } else if constexpr (FMT == QMOE_Q4_0 || FMT == QMOE_Q4_K) {
    const uint4 q = *(const uint4*)(p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    float a, b;  // value = a * q + b
    if constexpr (FMT == QMOE_Q4_0) {
      a = f16_bits_to_f32(((const uint16_t*)p1)[row * nb32 + u]);
      b = -8.f * a;
    } else {
      const uint4 meta = ((const uint4*)p1)[(size_t)row * (K >> 8) + (u >> 3)];
      const int j = u & 7;
      const uint64_t lo = (uint64_t)meta.y | ((uint64_t)meta.z << 32);
      const uint64_t hi = (uint64_t)meta.z | ((uint64_t)meta.w << 32);
      a = f16_bits_to_f32(meta.x & 0xFFFFu) * (float)((lo >> (6 * j)) & 63u);
      b = -f16_bits_to_f32(meta.x >> 16) * (float)((hi >> (16 + 6 * j)) & 63u);
    }
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t lo4 = w[c] & 0x0F0F0F0Fu;         // elements 8c, 8c+2, 8c+4, 8c+6
      const uint32_t hi4 = (w[c] >> 4) & 0x0F0F0F0Fu;  // elements 8c+1, 8c+3, ...
      out[4 * c + 0] = pack_bf16(fmaf(ubyte<0>(lo4), a, b),
                                 fmaf(ubyte<0>(hi4), a, b));
      out[4 * c + 1] = pack_bf16(fmaf(ubyte<1>(lo4), a, b),
                                 fmaf(ubyte<1>(hi4), a, b));
      out[4 * c + 2] = pack_bf16(fmaf(ubyte<2>(lo4), a, b),
                                 fmaf(ubyte<2>(hi4), a, b));
      out[4 * c + 3] = pack_bf16(fmaf(ubyte<3>(lo4), a, b),
                                 fmaf(ubyte<3>(hi4), a, b));
    }
  } else {  // Q6_K
    const uint4 ql = *(const uint4*)(p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const uint2 qh = *(const uint2*)(p1 + (size_t)row * (K >> 2) + 8 * (size_t)u);
    const size_t sb = (size_t)row * (K >> 8) + (u >> 3);
    const uint32_t sc2 = ((const uint16_t*)(base + L.off[2] + 16 * sb))[u & 7];
    const float d = f16_bits_to_f32(((const uint16_t*)(base + L.off[3]))[sb]);
    const float a0 = d * (float)(int8_t)(sc2 & 0xFFu), a1 = d * (float)(int8_t)(sc2 >> 8);
    const uint32_t w[4] = {ql.x, ql.y, ql.z, ql.w};
    const uint32_t hw[2] = {qh.x, qh.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // 8 elements 8c..8c+7: low nibbles in w[c], high bit pairs in 16 bits of qh
      const uint32_t h16 = (hw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
      const float a = c < 2 ? a0 : a1;
      const float b = -32.f * a;
      // byte i of q6 holds element 8c+2i (even) / 8c+2i+1 (odd) codes
      const uint32_t lo_e = (w[c] & 0x0F0F0F0Fu);
      const uint32_t lo_o = (w[c] >> 4) & 0x0F0F0F0Fu;
      // high bits: element 8c+m at bits 2m of h16
      uint32_t he = 0, ho = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        he |= ((h16 >> (4 * i)) & 3u) << (8 * i + 4);
        ho |= ((h16 >> (4 * i + 2)) & 3u) << (8 * i + 4);
      }
      const uint32_t ce = lo_e | he, co = lo_o | ho;
      out[4 * c + 0] = pack_bf16(fmaf(ubyte<0>(ce), a, b),
                                 fmaf(ubyte<0>(co), a, b));
      out[4 * c + 1] = pack_bf16(fmaf(ubyte<1>(ce), a, b),
                                 fmaf(ubyte<1>(co), a, b));
      out[4 * c + 2] = pack_bf16(fmaf(ubyte<2>(ce), a, b),
                                 fmaf(ubyte<2>(co), a, b));
      out[4 * c + 3] = pack_bf16(fmaf(ubyte<3>(ce), a, b),
                                 fmaf(ubyte<3>(co), a, b));
    }
  }
}

// The (expert, tile) of schedule slot i, or e = -1.
QMOE_D int tile_expert(const int32_t* tile_off, int E, int i, int& mt) {
  if (i >= tile_off[E]) return -1;
  int lo = 0, hi = E;  // largest e with tile_off[e] <= i
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= i) lo = mid; else hi = mid;
  }
  mt = i - tile_off[lo];
  return lo;
}

QMOE_D const qmoe_tier* prefill_tier(const PrefillParams& P, int e) {
  for (int i = 0; i < P.n_tiers; ++i)
    if (e >= P.tiers[i].e_begin && e < P.tiers[i].e_end) return &P.tiers[i];
  return nullptr;
}

// Stage rows 0..63 of the tile, values k0 .. k0+255, as bf16 into As.
// PASS 1: x rows gathered by token; PASS 2: h rows (bf16) by position.
template <int PASS>
QMOE_D void stage_tile(const PrefillParams& P, uint16_t* As, int pos0, int cnt, int K, int k0) {
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;  // 64 values per thread
  uint32_t w[32];
  const int kk = k0 + 64 * part;
  if (r < cnt && kk < K) {
    const int pos = pos0 + r;
    if (PASS == 1) {
      const int tok = P.perm[pos] / P.k;
      if (P.x_dtype == QMOE_F32) {
        const float4* src = (const float4*)((const float*)P.x + (size_t)tok * K + kk);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float4 f = src[i];
          w[2 * i] = pack_bf16(f.x, f.y);
          w[2 * i + 1] = pack_bf16(f.z, f.w);
        }
      } else {
        const uint4* src = (const uint4*)((const uint16_t*)P.x + (size_t)tok * K + kk);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 b = src[i];
          w[4 * i] = b.x; w[4 * i + 1] = b.y; w[4 * i + 2] = b.z; w[4 * i + 3] = b.w;
        }
      }
    } else {
      const uint4* src = (const uint4*)(P.h + (size_t)pos * K + kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 b = src[i];
        w[4 * i] = b.x; w[4 * i + 1] = b.y; w[4 * i + 2] = b.z; w[4 * i + 3] = b.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = 0u;
  }
  uint4* dst = (uint4*)(As + r * kAStride + 64 * part);
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

// One block: rows of tile mt of expert e x columns [n0, n0 + 4*NB*16).
template <int FMT, int PASS, int NB>
QMOE_D void prefill_tile(const PrefillParams& P, const qmoe_tier* t, int e, int mt, int nt,
                         uint16_t* As) {
  constexpr int NMAT = PASS == 1 ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int m_e = P.offsets[e + 1] - P.offsets[e];
  const int pos0 = P.offsets[e] + mt * kBM;
  const int cnt = min(kBM, m_e - mt * kBM);
  const int nmi = (cnt + 15) >> 4;
  const int N = PASS == 1 ? P.F : P.H;
  const int K = PASS == 1 ? P.H : P.F;
  const size_t stride = PASS == 1 ? layout_of(FMT, P.F, P.H).total : layout_of(FMT, P.H, P.F).total;
  const size_t eo = (size_t)(e - t->e_begin) * stride;
  const uint8_t* W0 = (const uint8_t*)(PASS == 1 ? t->gate : t->down) + eo;
  const uint8_t* W1 = (const uint8_t*)t->up + eo;
  const int n0 = nt * (kPW * NB * 16) + wave * (NB * 16);

  f32x4_t acc[NB][NMAT][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    stage_tile<PASS>(P, As, pos0, cnt, K, k0);
    __syncthreads();
    const int u0 = (k0 >> 5) + g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int row = n0 + b * 16 + li;
      uint32_t wb[NMAT][2][16];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        dequant_unit_bf16<FMT>(m == 0 ? W0 : W1, N, K, row, u0, wb[m][0]);
        dequant_unit_bf16<FMT>(m == 0 ? W0 : W1, N, K, row, u0 + 4, wb[m][1]);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int half = s >> 2, q = s & 3;  // unit g (+4 for half 1), values 8q..8q+7
        const int acol = 128 * half + 32 * g + 8 * q;
        bf16x8_t bop[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint4 v = make_uint4(wb[m][half][4 * q], wb[m][half][4 * q + 1],
                                     wb[m][half][4 * q + 2], wb[m][half][4 * q + 3]);
          bop[m] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < nmi) {
            const uint4 av = *(const uint4*)(As + (16 * i + li) * kAStride + acol);
            const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
              acc[b][m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[m], acc[b][m][i], 0, 0, 0);
          }
        }
      }
    }
  }
  // epilogue: lane holds rows 16i + 4g + j, column n0 + 16b + li
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int col = n0 + b * 16 + li;
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + 4 * g + j;
        if (r >= cnt) continue;
        const size_t pos = (size_t)(pos0 + r);
        if constexpr (PASS == 1) {
          const float gv = acc[b][0][i][j], uv = acc[b][1][i][j];
          const float hv = gv / (1.f + expf(-gv)) * uv;
          P.h[pos * P.F + col] = (uint16_t)(pack_bf16(hv, 0.f) & 0xFFFFu);
        } else {
          P.o[pos * P.H + col] = acc[b][0][i][j];
        }
      }
    }
  }
}

template <int PASS, int NB>
__global__ __launch_bounds__(kPB) void prefill_kernel(PrefillParams P) {
  __shared__ __align__(16) uint16_t As[kBM * kAStride];
  const int i = blockIdx.x / P.ntiles, nt = blockIdx.x - i * P.ntiles;
  int mt = 0;
  const int e = tile_expert(P.tile_off, P.E, i, mt);
  if (e < 0) return;
  const qmoe_tier* t = prefill_tier(P, e);
  if (!t) return;
  const int fmt = PASS == 1 ? t->fmt_gate_up : t->fmt_down;
  switch (fmt) {
    case QMOE_Q8_0: prefill_tile<QMOE_Q8_0, PASS, NB>(P, t, e, mt, nt, As); break;
    case QMOE_Q4_0: prefill_tile<QMOE_Q4_0, PASS, NB>(P, t, e, mt, nt, As); break;
    case QMOE_MXFP4: prefill_tile<QMOE_MXFP4, PASS, NB>(P, t, e, mt, nt, As); break;
    case QMOE_Q4_K: prefill_tile<QMOE_Q4_K, PASS, NB>(P, t, e, mt, nt, As); break;
    case QMOE_Q6_K: prefill_tile<QMOE_Q6_K, PASS, NB>(P, t, e, mt, nt, As); break;
    default: break;
  }
}

// tile_off[e] = sum over e' < e of ceil(m_e' / 64), one block.
__global__ __launch_bounds__(1024) void prefill_schedule_kernel(const int32_t* offsets, int E,
                                                                int32_t* tile_off) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (E + 1023) / 1024;
  const int e_lo = min(E, (int)threadIdx.x * per), e_hi = min(E, e_lo + per);
  int local = 0;
  for (int e = e_lo; e < e_hi; ++e) local += (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
  int v = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int run = v - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int e = e_lo; e < e_hi; ++e) {
    tile_off[e] = run;
    run += (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
  }
  if (threadIdx.x == 1023) {
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    tile_off[E] = total;
  }
}

constexpr int kNB1 = 2;  // pass 1: 4 waves x 2 x 16 = 128 columns of F per block
constexpr int kNB2 = 4;  // pass 2: 4 waves x 4 x 16 = 256 columns of H per block

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);

}  // namespace qmoe

using namespace qmoe;

extern "C" {

size_t qgemm_grouped_prefill_workspace_size(int T, int k, int E, int F) {
  if (T < 0 || k < 0 || E <= 0 || F < 0) return 0;
  return round_up256((size_t)T * k * F * sizeof(uint16_t)) +
         round_up256((size_t)(E + 1) * sizeof(int32_t)) + 256;
}

int qgemm_grouped_prefill(const qmoe_tier* tiers, int n_tiers, int E, int H, int F,
                          const void* x, int x_dtype, int T, int k, const int32_t* offsets,
                          const int32_t* perm, float* o, void* ws, size_t ws_bytes,
                          void* stream) {
  if (T < 0 || k < 0)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_grouped_prefill: T=%d k=%d", T, k);
  if (T == 0 || k == 0) return QMOE_OK;
  int st = validate_tiers(tiers, n_tiers, E, H, F, true);
  if (st) return st;
  if (E > 8192) return fail(QMOE_ERR_UNSUPPORTED, "qgemm_grouped_prefill: E=%d > 8192", E);
  if (H % 64 || F % 64)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_grouped_prefill: H and F must be multiples of 64");
  if (!x || !offsets || !perm || !o)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_grouped_prefill: null pointer");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "qgemm_grouped_prefill: unknown x_dtype %d", x_dtype);
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(o, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_grouped_prefill: misaligned x/o");
  const size_t need = qgemm_grouped_prefill_workspace_size(T, k, E, F);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "qgemm_grouped_prefill: workspace %zu < %zu", ws_bytes, need);
  const long long A = (long long)T * k;
  if (A > (1 << 24)) return fail(QMOE_ERR_UNSUPPORTED, "qgemm_grouped_prefill: T*k too large");
  hipStream_t s = (hipStream_t)stream;
  PrefillParams P{};
  for (int i = 0; i < n_tiers; ++i) P.tiers[i] = tiers[i];
  P.n_tiers = n_tiers; P.E = E; P.H = H; P.F = F; P.T = T; P.k = k;
  P.x = x; P.x_dtype = x_dtype; P.offsets = offsets; P.perm = perm; P.o = o;
  P.h = (uint16_t*)ws;
  int32_t* tile_off = (int32_t*)((char*)ws + round_up256((size_t)A * F * sizeof(uint16_t)));
  P.tile_off = tile_off;
  st = QMOE_LAUNCH("prefill_schedule", prefill_schedule_kernel, dim3(1), 1024, 0, s, offsets, E,
                   tile_off);
  if (st) return st;
  const long long max_tiles = (A + kBM - 1) / kBM + (A < E ? A : E);
  P.ntiles = (F + kPW * kNB1 * 16 - 1) / (kPW * kNB1 * 16);
  st = QMOE_LAUNCH("prefill_gate_up", (prefill_kernel<1, kNB1>), dim3((unsigned)(max_tiles * P.ntiles)),
                   kPB, 0, s, P);
  if (st) return st;
  P.ntiles = (H + kPW * kNB2 * 16 - 1) / (kPW * kNB2 * 16);
  return QMOE_LAUNCH("prefill_down", (prefill_kernel<2, kNB2>), dim3((unsigned)(max_tiles * P.ntiles)),
                     kPB, 0, s, P);
}

}  // extern "C"
