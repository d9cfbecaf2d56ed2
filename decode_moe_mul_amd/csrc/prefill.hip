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
#include "dequant.hpp"

namespace qmoe {

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
  uint16_t* h;              // [T*k, F] bf16 (prefill)
  float* h32;               // [T*k, F] fp32 (decode)
  float* o;                 // [T*k, H]
  int ntiles;               // column tiles of this pass
  int m_min;                // decode: only experts with more rows than this
};

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

// The tier holding expert e, assembled field by field with constant indices
// only (a runtime index or struct copy out of the by-value kernel argument
// would spill the whole argument block to scratch).
QMOE_D bool prefill_tier(const PrefillParams& P, int e, qmoe_tier& out) {
  bool found = false;
  int32_t eb = 0, ee = 0, fgu = 0, fd = 0;
  const void *g = nullptr, *u = nullptr, *d = nullptr;
#pragma unroll
  for (int i = 0; i < QMOE_MAX_TIERS; ++i) {
    const bool hit = !found && i < P.n_tiers && e >= P.tiers[i].e_begin && e < P.tiers[i].e_end;
    if (hit) {
      eb = P.tiers[i].e_begin; ee = P.tiers[i].e_end;
      fgu = P.tiers[i].fmt_gate_up; fd = P.tiers[i].fmt_down;
      g = P.tiers[i].gate; u = P.tiers[i].up; d = P.tiers[i].down;
      found = true;
    }
  }
  out.e_begin = eb; out.e_end = ee; out.fmt_gate_up = fgu; out.fmt_down = fd;
  out.gate = g; out.up = u; out.down = d;
  return found;
}

// Stage rows 0 .. 16*MI-1 of a tile, values k0 .. k0+255, into As as bf16
// (prefill) or fp16 (DEC, decode rows); rows >= cnt and values >= K are zero.
// PASS 1: x rows gathered by token; PASS 2: h rows by position (bf16 for
// prefill, fp32 in the decode workspace).
template <int PASS, int MI, bool DEC>
QMOE_D void stage_tile(const PrefillParams& P, uint16_t* As, int pos0, int cnt, int K, int k0) {
  constexpr int ROWS = 16 * MI, CH = kBK / 8;  // 8-value chunks per row
  for (int idx = threadIdx.x; idx < ROWS * CH; idx += kPB) {
    const int r = idx / CH, c = idx - r * CH;
    const int kk = k0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < cnt && kk < K) {
      const int pos = pos0 + r;
      if (PASS == 1) {
        const int tok = P.perm[pos] / P.k;
        if (P.x_dtype == QMOE_F32) {
          const float4* src = (const float4*)((const float*)P.x + (size_t)tok * K + kk);
          const float4 a = src[0], b = src[1];
          v = make_uint4(pack2<DEC>(a.x, a.y), pack2<DEC>(a.z, a.w), pack2<DEC>(b.x, b.y),
                         pack2<DEC>(b.z, b.w));
        } else {
          v = *(const uint4*)((const uint16_t*)P.x + (size_t)tok * K + kk);
          if (DEC) {  // bf16 -> fp16
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              o[j] = pack_f16(bf16_bits_to_f32(w[j] & 0xFFFFu), bf16_bits_to_f32(w[j] >> 16));
            v = make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      } else if (DEC) {
        const float4* src = (const float4*)(P.h32 + (size_t)pos * K + kk);
        const float4 a = src[0], b = src[1];
        v = make_uint4(pack_f16(a.x, a.y), pack_f16(a.z, a.w), pack_f16(b.x, b.y),
                       pack_f16(b.z, b.w));
      } else {
        v = *(const uint4*)(P.h + (size_t)pos * K + kk);
      }
    }
    *(uint4*)(As + r * kAStride + 8 * c) = v;
  }
}

// One block: rows pos0 .. pos0+cnt-1 (cnt <= 16*MI) of expert e's permuted
// positions x columns [n0, n0 + 4*NB*16) of column tile nt.
template <int FMT, int PASS, int NB, int MI, bool DEC>
QMOE_D void mfma_tile(const PrefillParams& P, const qmoe_tier* t, int e, int pos0, int cnt,
                      int nt, uint16_t* As) {
  constexpr int NMAT = PASS == 1 ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int nmi = (cnt + 15) >> 4;
  const int N = PASS == 1 ? P.F : P.H;
  const int K = PASS == 1 ? P.H : P.F;
  const size_t stride = PASS == 1 ? layout_of(FMT, P.F, P.H).total : layout_of(FMT, P.H, P.F).total;
  const size_t eo = (size_t)(e - t->e_begin) * stride;
  const uint8_t* W0 = (const uint8_t*)(PASS == 1 ? t->gate : t->down) + eo;
  const uint8_t* W1 = (const uint8_t*)t->up + eo;
  const int n0 = nt * (kPW * NB * 16) + wave * (NB * 16);

  f32x4_t acc[NB][NMAT][MI];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[b][m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    stage_tile<PASS, MI, DEC>(P, As, pos0, cnt, K, k0);
    __syncthreads();
    const int u0 = (k0 >> 5) + g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int row = n0 + b * 16 + li;
      uint32_t wb[NMAT][2][16];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        dequant_unit<FMT, DEC>(m == 0 ? W0 : W1, N, K, row, u0, wb[m][0]);
        dequant_unit<FMT, DEC>(m == 0 ? W0 : W1, N, K, row, u0 + 4, wb[m][1]);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int half = s >> 2, q = s & 3;  // unit g (+4 for half 1), values 8q..8q+7
        const int acol = 128 * half + 32 * g + 8 * q;
        uint4 bop[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          bop[m] = make_uint4(wb[m][half][4 * q], wb[m][half][4 * q + 1],
                              wb[m][half][4 * q + 2], wb[m][half][4 * q + 3]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (i < nmi) {
            const uint4 av = *(const uint4*)(As + (16 * i + li) * kAStride + acol);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              if constexpr (DEC)
                acc[b][m][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(f16x8_t, av), __builtin_bit_cast(f16x8_t, bop[m]),
                    acc[b][m][i], 0, 0, 0);
              else
                acc[b][m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bop[m]),
                    acc[b][m][i], 0, 0, 0);
            }
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
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + 4 * g + j;
        if (r >= cnt) continue;
        const size_t pos = (size_t)(pos0 + r);
        if constexpr (PASS == 1) {
          const float gv = acc[b][0][i][j], uv = acc[b][1][i][j];
          const float hv = gv / (1.f + expf(-gv)) * uv;
          if (DEC) P.h32[pos * P.F + col] = hv;
          else P.h[pos * P.F + col] = (uint16_t)(pack_bf16(hv, 0.f) & 0xFFFFu);
        } else {
          P.o[pos * P.H + col] = acc[b][0][i][j];
        }
      }
    }
  }
}

template <int PASS, int MI, bool DEC, int NB>
QMOE_D void mfma_dispatch(const PrefillParams& P, const qmoe_tier* t, int e, int pos0, int cnt,
                          int nt, uint16_t* As) {
  const int fmt = PASS == 1 ? t->fmt_gate_up : t->fmt_down;
  switch (fmt) {
    case QMOE_Q8_0: mfma_tile<QMOE_Q8_0, PASS, NB, MI, DEC>(P, t, e, pos0, cnt, nt, As); break;
    case QMOE_Q4_0: mfma_tile<QMOE_Q4_0, PASS, NB, MI, DEC>(P, t, e, pos0, cnt, nt, As); break;
    case QMOE_MXFP4: mfma_tile<QMOE_MXFP4, PASS, NB, MI, DEC>(P, t, e, pos0, cnt, nt, As); break;
    case QMOE_Q4_K: mfma_tile<QMOE_Q4_K, PASS, NB, MI, DEC>(P, t, e, pos0, cnt, nt, As); break;
    case QMOE_Q6_K: mfma_tile<QMOE_Q6_K, PASS, NB, MI, DEC>(P, t, e, pos0, cnt, nt, As); break;
    default: break;
  }
}

template <int PASS, int NB>
__global__ __launch_bounds__(kPB) void prefill_kernel(PrefillParams P) {
  __shared__ __align__(16) uint16_t As[kBM * kAStride];
  const int i = blockIdx.x / P.ntiles, nt = blockIdx.x - i * P.ntiles;
  int mt = 0;
  const int e = tile_expert(P.tile_off, P.E, i, mt);
  if (e < 0) return;
  qmoe_tier tier;
  if (!prefill_tier(P, e, tier)) return;
  const qmoe_tier* t = &tier;
  const int m_e = P.offsets[e + 1] - P.offsets[e];
  const int pos0 = P.offsets[e] + mt * kBM;
  const int cnt = min(kBM, m_e - mt * kBM);
  mfma_dispatch<PASS, kBM / 16, false, NB>(P, t, e, pos0, cnt, nt, As);
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
