// qgemm_grouped_prefill: the routed-expert FFN for long chunks (a 2048-token
// prefill chunk, [P4] "DwarfStar on 8x L40S", section
// "120 t/s 的秘密微批次分组解码") as a grouped GEMM on the gfx950 matrix cores.
// Prefill turns the per-expert GEMV into a real contraction ([P1] "NInfer 80 SM
// port", section 九.3: group-wise 4/5-bit weights dequantized on chip and fed
// to a 16-bit GEMM).
//
// Launches:
//  1. prefill_prep_kernel: block 0 cuts every expert's rows (positions
//     offsets[e] .. offsets[e+1]-1 of the permutation) into tiles of up to
//     128 rows and lists them (tiles of more than 32 rows, the rest); the
//     other blocks round x to fp16 once.
//  2. prefill_kernel<PASS 1> over each list: gate and up tiles,
//     SiLU(g) * u -> h (fp16).
//  3. prefill_kernel<PASS 2> over each list: down tiles over K = F -> o
//     (fp32, permuted rows).
//
// One block (4 waves) computes one row tile of one expert against
// 4 * NB * 16 output columns, K in steps of 128 values (4 units of 32):
//  * lane (n, g) of a wave owns unit g of the step in weight row n of each of
//    its NB column blocks: it loads the unit's codes and scales two steps
//    ahead and dequantizes them to fp16 in registers with packed fp16
//    arithmetic (exact codes, one rounding by the scale), so every weight byte
//    is read and decoded by one lane only;
//  * the unit's 32 values feed 4 v_mfma_f32_16x16x32_f16 (8 values each), so
//    the contraction order inside a step is a fixed permutation of K; the
//    activation rows are staged in LDS (double-buffered) already permuted the
//    same way, so A and B agree;
//  * every staged 16-row group of activations is multiplied against the
//    decoded weights held in registers, fp32 accumulation.  Staged rows are
//    256 bytes; the 16-byte chunk c of row r sits at chunk c ^ (r & 15), so the
//    16 rows a matrix-core operand reads lie on distinct banks.
// Activations and h are fp16 (11-bit significands) inside the products.
#include <algorithm>

#include "mx.hpp"

#pragma clang fp contract(off)

namespace qmoe {

typedef _Float16 pf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPW = 4;             // waves per block
constexpr int kPB = 64 * kPW;      // threads per block
constexpr int kMI = 8;             // 16-row groups per tile
constexpr int kBM = 16 * kMI;      // rows (assignments) per tile
constexpr int kBK = 128;           // K values per step
constexpr int kAS = kBK;           // LDS row stride of staged activations (fp16)
constexpr int kNB1 = 1;            // pass 1: 4 waves x 1 x 16 = 64 columns of F
constexpr int kNB2 = 2;            // pass 2: 4 waves x 2 x 16 = 128 columns of H

struct PrefillParams {
  qmoe_tier tiers[QMOE_MAX_TIERS];
  int n_tiers, E, H, F, T, k;
  const int32_t* offsets;
  const int32_t* perm;
  const int2* tiles;     // big list [tiles_cap_big], then small list: (expert, tile)
  const int* counts;     // lengths of the two lists
  int tiles_cap_big;
  const uint16_t* x16;   // [T + 1, xs] fp16 (row T zero, columns >= H zero)
  uint16_t* h;           // [T*k + 1, hs] fp16 (row T*k zero, columns >= F zero)
  int xs, hs;            // row strides: H and F rounded up to whole K steps
  float* o;              // [T*k, H]
  int ntiles;            // column tiles of this pass
  // block-scaled path (qgemm_grouped_prefill_mx): tiers whose gate/up and
  // down are both MXFP4 read MXFP8 activations: x8 [T + 1, xs] and h8
  // [T*k + 1, hs] E4M3 bytes (last rows and padding zero) with E8M0 scales
  // x8s [T + 1, xs / 32], h8s [T*k + 1, hs / 32]
  const uint8_t* x8;
  const uint8_t* x8s;
  uint8_t* h8;
  uint8_t* h8s;
};

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

// ------------------------------------------------ one unit of weights ----
// Planes of one [N, K] weight matrix.
struct Planes {
  const uint8_t* p0;
  const uint8_t* p1;
  const uint8_t* p2;
  const uint8_t* p3;
};

QMOE_D Planes planes_of(const void* base, int fmt, int N, int K) {
  const Layout L = layout_of(fmt, N, K);
  const uint8_t* b = (const uint8_t*)base;
  return {b + L.off[0], b + L.off[1], b + L.off[2], b + L.off[3]};
}

// Raw bytes of unit u (32 values) of weight row `row`.
template <int FMT>
struct RawUnit {
  uint4 q, q2;    // codes (q2: second half of a Q8_0 unit)
  uint4 meta;     // Q4_K super-block meta
  uint2 qh;       // Q6_K high bits
  uint32_t s0, s1;

  QMOE_D void load(const Planes& M, int row, int u, int K) {
    const uint32_t r = (uint32_t)row, uu = (uint32_t)u, nb32 = (uint32_t)(K >> 5);
    if constexpr (FMT == QMOE_Q8_0) {
      const uint32_t qo = r * (uint32_t)K + (uu << 5);
      q = *(const uint4*)(M.p0 + qo);
      q2 = *(const uint4*)(M.p0 + qo + 16u);
      s0 = *(const uint16_t*)(M.p1 + ((r * nb32 + uu) << 1));
    } else {
      q = *(const uint4*)(M.p0 + r * (uint32_t)(K >> 1) + (uu << 4));
      if constexpr (FMT == QMOE_Q4_0) {
        s0 = *(const uint16_t*)(M.p1 + ((r * nb32 + uu) << 1));
      } else if constexpr (FMT == QMOE_MXFP4) {
        s0 = M.p1[r * nb32 + uu];
      } else if constexpr (FMT == QMOE_Q4_K) {
        meta = *(const uint4*)(M.p1 + ((r * (uint32_t)(K >> 8) + (uu >> 3)) << 4));
      } else {
        qh = *(const uint2*)(M.p1 + r * (uint32_t)(K >> 2) + (uu << 3));
        const uint32_t sb = r * (uint32_t)(K >> 8) + (uu >> 3);
        // the aligned word holding the unit's two sub-block scales (bytes
        // 2j, 2j + 1 of the super-block's 16, j = u & 7)
        s0 = *(const uint32_t*)(M.p2 + (sb << 4) + ((uu & 6u) << 1));
        s1 = *(const uint16_t*)(M.p3 + (sb << 1));
      }
    }
  }

  // The unit as 16 words of fp16 pairs in the format's pair order (see
  // stage_perm): the exact code times the scale, rounded once to fp16.
  QMOE_D void dequant(int u, uint32_t w[16]) const {
    if constexpr (FMT == QMOE_Q8_0) {
      bytes_to_h2(q, q2, w);  // exact q
      const uint32_t d2 = (s0 & 0xFFFFu) * 0x10001u;
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = pk_mul_h2(w[i], d2);
    } else if constexpr (FMT == QMOE_Q4_0) {
      nibbles_to_h2(q, H2_NEG_1032, w);  // exact q - 8
      const uint32_t d2 = (s0 & 0xFFFFu) * 0x10001u;
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = pk_mul_h2(w[i], d2);
    } else if constexpr (FMT == QMOE_MXFP4) {
      const float sc = e8m0_to_f32(s0);
      const uint32_t c[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[i], sc, 0));
        w[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[i], sc, 1));
        w[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[i], sc, 2));
        w[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[i], sc, 3));
      }
    } else if constexpr (FMT == QMOE_Q4_K) {
      nibbles_to_h2(q, H2_NEG_1024, w);  // exact q
      // 6-bit fields of the 96-bit word (y, z, w): sc_j at bit 6j, m_j at
      // bit 48 + 6j, j = u & 7
      const uint32_t b = 6u * (uint32_t)(u & 7), bm = b + 16u;
      const bool lo_b = b < 32u, lo_m = bm < 32u;
      const uint32_t sc = __builtin_amdgcn_alignbit(lo_b ? meta.z : meta.w, lo_b ? meta.y : meta.z,
                                                    b & 31u) & 63u;
      const uint32_t mn = __builtin_amdgcn_alignbit(lo_m ? meta.w : 0u, lo_m ? meta.z : meta.w,
                                                    bm & 31u) & 63u;
      const float a = f16_bits_to_f32(meta.x & 0xFFFFu) * (float)sc;
      const float c = -(f16_bits_to_f32(meta.x >> 16) * (float)mn);
      const h2_t a2 = __builtin_bit_cast(h2_t, pack_h2(a, a));
      const h2_t c2 = __builtin_bit_cast(h2_t, pack_h2(c, c));
#pragma unroll
      for (int i = 0; i < 16; ++i)
        w[i] = __builtin_bit_cast(uint32_t,
                                  __builtin_elementwise_fma(__builtin_bit_cast(h2_t, w[i]), a2, c2));
    } else {
      q6_to_h2(q, qh, w);  // exact q - 32; words 0..7 are sub-block 2j, 8..15 2j + 1
      const float d = f16_bits_to_f32(s1);
      const uint32_t sh = (uint32_t)(u & 1) * 16u;
      const float a0 = d * (float)(int)__builtin_amdgcn_sbfe(s0, sh, 8u);
      const float a1 = d * (float)(int)__builtin_amdgcn_sbfe(s0, sh + 8u, 8u);
      const uint32_t h0 = pack_h2(a0, a0), h1 = pack_h2(a1, a1);
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = pk_mul_h2(w[i], i < 8 ? h0 : h1);
    }
  }
};

// ------------------------------------------------ staged activations -----
// Eight consecutive fp16 activations (words v0..v3 = values (0,1) .. (6,7))
// reordered to the format's pair order within 8 values:
//   4- and 6-bit codes: (0,4) (1,5) (2,6) (3,7)
//   Q8_0 bytes:         (0,2) (1,3) (4,6) (5,7)
//   MXFP4:              natural
template <int FMT>
QMOE_D uint4 stage_perm(uint4 v) {
  if constexpr (FMT == QMOE_MXFP4) {
    return v;
  } else if constexpr (FMT == QMOE_Q8_0) {
    return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u),
                      __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                      __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
  } else {
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                      __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
  }
}

QMOE_D pf32x4_t mfma_f16(uint4 a, const uint32_t* b, pf32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(pf16x8_t, a),
      __builtin_bit_cast(pf16x8_t, make_uint4(b[0], b[1], b[2], b[3])), c, 0, 0, 0);
}

// One tile: rows pos0 .. pos0 + cnt - 1 (cnt <= 16 MI) of the permuted
// positions x columns [nt * 64 NB, (nt + 1) * 64 NB) of the pass's output.
// W0: gate (pass 1) or down (pass 2) of the expert; W1: up.  FULL: all MI
// row groups hold rows (no per-group guards, so the compiler can interleave
// the decode of one unit with the matrix-core ops of another); otherwise
// groups past the tile's rows are skipped.
template <int FMT, int PASS, int NB, int MI, bool FULL>
QMOE_D void tile_gemm(const PrefillParams& P, const void* W0, const void* W1, int pos0, int cnt,
                      int nt, uint16_t* As) {
  constexpr int NMAT = PASS == 1 ? 2 : 1;
  constexpr int BM = 16 * MI;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int nmi = FULL ? MI : (cnt + 15) >> 4;  // block-uniform
  const int N = PASS == 1 ? P.F : P.H, K = PASS == 1 ? P.H : P.F;
  const int U = K >> 5, nsteps = (U + 3) >> 2;
  const int n0 = nt * (kPW * NB * 16) + wave * (NB * 16);
  Planes mats[NMAT];
  mats[0] = planes_of(W0, FMT, N, K);
  if constexpr (NMAT == 2) mats[1] = planes_of(W1, FMT, N, K);
  int wrow[NB];  // weight rows past N re-read row N - 1 (never stored)
#pragma unroll
  for (int b = 0; b < NB; ++b) wrow[b] = min(n0 + 16 * b + li, N - 1);

  // staging: thread tid stages chunk (tid & 15) (8 values) of row
  // 16 j + (tid >> 4) of every row group j.  Activation rows are stored with
  // a stride of whole steps (zero-padded past K), and rows past the tile
  // read an all-zero row, so every staging load is unconditional.
  const int sr = tid >> 4, sc = tid & 15;
  const int ks = PASS == 1 ? P.xs : P.hs;  // row stride (fp16 values)
  const uint16_t* src[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int r = 16 * j + sr;
    if constexpr (PASS == 1) {
      const int tok = r < cnt ? P.perm[pos0 + r] / P.k : P.T;  // row T is zero
      src[j] = P.x16 + (size_t)tok * ks + 8 * sc;
    } else {
      src[j] = P.h + (size_t)(r < cnt ? pos0 + r : P.T * P.k) * ks + 8 * sc;
    }
  }
  auto load_a = [&](int step, uint4 (&ra)[MI]) {
#pragma unroll
    for (int j = 0; j < MI; ++j)
      if (FULL || j < nmi) ra[j] = *(const uint4*)(src[j] + step * kBK);
  };
  auto write_a = [&](int buf, const uint4 (&ra)[MI]) {
    uint16_t* base = As + buf * (BM * kAS);
#pragma unroll
    for (int j = 0; j < MI; ++j)
      if (FULL || j < nmi)
        *(uint4*)(base + (16 * j + sr) * kAS + 8 * (sc ^ sr)) = stage_perm<FMT>(ra[j]);
  };
  auto load_b = [&](int step, RawUnit<FMT> (&rb)[NB][NMAT]) {
    const int u = min(step * 4 + g, U - 1);  // units past K meet zero activations
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) rb[b][m].load(mats[m], wrow[b], u, K);
  };

  pf32x4_t acc[NB][NMAT][MI];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[b][m][i] = pf32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, int step, const RawUnit<FMT> (&rb)[NB][NMAT]) {
    const int u = min(step * 4 + g, U - 1);
    uint32_t wd[NB][NMAT][16];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) rb[b][m].dequant(u, wd[b][m]);
    const uint16_t* base = As + buf * (BM * kAS) + li * kAS;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cs = 8 * ((4 * g + s) ^ li);  // row 16 i + li: swizzle by li
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (FULL || i < nmi) {
          const uint4 av = *(const uint4*)(base + 16 * i * kAS + cs);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[b][m][i] = mfma_f16(av, &wd[b][m][4 * s], acc[b][m][i]);
        }
      }
    }
  };

  // Pipeline: the weights and activations of steps s + 1 and s + 2 are in
  // flight while step s is computed (register sets alternate with the step's
  // parity); LDS buffer s & 1 holds the activations of step s.  After step s
  // the activations of s + 1 go to LDS and the loads of s + 3 (activations)
  // and s + 2 (weights) are issued into the sets just freed.  Prefetches past
  // the last step re-read the last step (cache hits, never used), so the loop
  // body has no branches and the loads stay in flight across it.
  const int last = nsteps - 1;
  RawUnit<FMT> rb0[NB][NMAT], rb1[NB][NMAT];
  uint4 ra0[MI], ra1[MI];
  load_b(0, rb0);
  load_a(0, ra0);
  load_b(min(1, last), rb1);
  load_a(min(1, last), ra1);
  // the block's previous item may still be reading LDS buffer 0 (its last
  // step, when the step count is odd)
  __syncthreads();
  write_a(0, ra0);
  load_a(min(2, last), ra0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    compute(0, s, rb0);
    write_a(1, ra1);
    load_a(min(s + 3, last), ra1);
    load_b(min(s + 2, last), rb0);
    __syncthreads();
    compute(1, s + 1, rb1);
    write_a(0, ra0);
    load_a(min(s + 4, last), ra0);
    load_b(min(s + 3, last), rb1);
    __syncthreads();
  }
  if (s < nsteps) compute(0, s, rb0);  // odd step count: buffer 0, set 0

  // epilogue: lane holds rows 16i + 4g + j of column n0 + 16b + li
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int col = n0 + b * 16 + li;
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (!FULL && i >= nmi) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + 4 * g + j;
        if (r >= cnt) continue;
        const size_t pos = (size_t)(pos0 + r);
        if constexpr (PASS == 1) {
          const float gv = acc[b][0][i][j], uv = acc[b][1][i][j];
          const float hv = gv / (1.f + expf(-gv)) * uv;
          P.h[pos * P.hs + col] = (uint16_t)f32_to_f16_bits(hv);
        } else {
          P.o[pos * N + col] = acc[b][0][i][j];
        }
      }
    }
  }
}

// One tile of an MXFP4/MXFP4 tier on the block-scaled matrix cores: rows
// pos0 .. pos0 + cnt - 1 x the pass's column tile nt.  Weights are used as
// stored (lane (n, g) loads unit g of the step in row n, 16 bytes, and its
// E8M0 byte); activations are the MXFP8 rows x8 (pass 1, gathered by token)
// or h8 (pass 2, by position), loaded straight from global memory; rows past
// the tile read the zero row.  Row groups are taken 4 at a time (64 rows), so
// a 128-row tile streams its weights twice (the second time from the caches).
// Pass 1 writes h = SiLU(g) * u through the LDS tile hl [16 MI][64] and
// quantizes each row's two 32-column blocks to MXFP8 into h8 / h8s.
template <int PASS, int NB, int MI>
QMOE_D void tile_mx(const PrefillParams& P, const void* W0, const void* W1, int pos0, int cnt,
                    int nt, float* hl) {
  static_assert(PASS != 1 || NB == 1, "the gate/up epilogue assumes 16 columns per wave");
  constexpr int NMAT = PASS == 1 ? 2 : 1;
  constexpr int SMI = MI < 4 ? MI : 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int N = PASS == 1 ? P.F : P.H, K = PASS == 1 ? P.H : P.F;
  const int U = K >> 5, nsteps = (U + 3) >> 2;
  const int n0 = nt * (kPW * NB * 16) + wave * (NB * 16);
  Planes mats[NMAT];
  mats[0] = planes_of(W0, QMOE_MXFP4, N, K);
  if constexpr (NMAT == 2) mats[1] = planes_of(W1, QMOE_MXFP4, N, K);
  uint32_t wrow[NB];  // weight rows past N re-read row N - 1 (never stored)
#pragma unroll
  for (int b = 0; b < NB; ++b) wrow[b] = (uint32_t)min(n0 + 16 * b + li, N - 1);
  const uint32_t astride = (uint32_t)(PASS == 1 ? P.xs : P.hs), sstride = astride >> 5;
  const uint8_t* abase = PASS == 1 ? P.x8 : P.h8;
  const uint8_t* sbase = PASS == 1 ? P.x8s : P.h8s;
  const int zero_row = PASS == 1 ? P.T : P.T * P.k;
  const int nmi = (cnt + 15) >> 4;  // block-uniform
  const int last = nsteps - 1;
  __syncthreads();  // the block's previous item may still be reading the LDS tile
  struct A8 { uint4 lo, hi; uint32_t s; };
  struct B4 { uint4 q; uint32_t s; };
  for (int gi0 = 0; gi0 < nmi; gi0 += SMI) {
    uint32_t arow[SMI];
#pragma unroll
    for (int i = 0; i < SMI; ++i) {
      const int r = 16 * (gi0 + i) + li;
      arow[i] = (uint32_t)(r < cnt ? (PASS == 1 ? P.perm[pos0 + r] / P.k : pos0 + r) : zero_row);
    }
    auto load = [&](int st, A8 (&a)[SMI], B4 (&w)[NB][NMAT]) {
      const uint32_t k0 = (uint32_t)st * 128u, ab = (uint32_t)st * 4u + (uint32_t)g;
      const uint32_t u = (uint32_t)min(st * 4 + g, U - 1);  // units past K meet zero rows
#pragma unroll
      for (int i = 0; i < SMI; ++i) {
        const uint8_t* row = abase + arow[i] * astride + k0;
        a[i].lo = *(const uint4*)(row + 16u * g);
        a[i].hi = *(const uint4*)(row + 64u + 16u * g);
        a[i].s = sbase[arow[i] * sstride + ab];
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          w[b][m].q = *(const uint4*)(mats[m].p0 + wrow[b] * (uint32_t)(K >> 1) + 16u * u);
          w[b][m].s = mats[m].p1[wrow[b] * (uint32_t)U + u];
        }
    };
    mx_v4f acc[NMAT][NB][SMI];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < SMI; ++i) acc[m][b][i] = mx_v4f{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const A8 (&a)[SMI], const B4 (&w)[NB][NMAT]) {
#pragma unroll
      for (int i = 0; i < SMI; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
            acc[m][b][i] = mx_mma(a[i].lo, a[i].hi, a[i].s, w[b][m].q, w[b][m].s, acc[m][b][i]);
    };
    A8 a0[SMI], a1[SMI];
    B4 w0[NB][NMAT], w1[NB][NMAT];
    load(0, a0, w0);
    int st = 0;
    for (; st + 1 < nsteps; st += 2) {
      load(st + 1, a1, w1);
      mma(a0, w0);
      load(min(st + 2, last), a0, w0);
      mma(a1, w1);
    }
    if (st < nsteps) mma(a0, w0);
    // lane holds rows 16 (gi0 + i) + 4 g + j of column n0 + 16 b + li
#pragma unroll
    for (int i = 0; i < SMI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * (gi0 + i) + 4 * g + j;
        if (r >= cnt) continue;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int col = n0 + 16 * b + li;
          if constexpr (PASS == 1) {
            const float gv = acc[0][b][i][j], uv = acc[1][b][i][j];
            hl[r * 64 + wave * 16 + li] = gv / (1.f + expf(-gv)) * uv;
          } else {
            if (col < N) P.o[(size_t)(pos0 + r) * N + col] = acc[0][b][i][j];
          }
        }
      }
  }
  if constexpr (PASS == 1) {
    // quantize the tile's h rows: thread t takes row t >> 1, 32-column half t & 1
    __syncthreads();
    const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
    if (r < cnt) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = hl[r * 64 + 32 * half + j];
      uint32_t out[8];
      const uint32_t e = mx_quantize32(v, out);
      const size_t pos = (size_t)(pos0 + r);
      uint4* dst = (uint4*)(P.h8 + pos * P.hs + nt * 64 + 32 * half);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      P.h8s[pos * (P.hs >> 5) + nt * 2 + half] = (uint8_t)e;
    }
    __syncthreads();  // the LDS tile is reused by the next item
  }
}

// Tiles of more than kSmall rows (up to kBM) take 16 kMI-row register
// blocks; tiles of at most kSmall rows (experts with a few rows, whose time is
// the weight stream) take kMIsmall-row blocks.
constexpr int kSmall = 32;
constexpr int kMIsmall = kSmall / 16;

template <int FMT, int PASS, int NB, int MI>
QMOE_D void tile_dispatch_full(const PrefillParams& P, const void* W0, const void* W1, int pos0,
                               int cnt, int nt, uint16_t* As) {
  if (MI == kMIsmall || cnt == 16 * MI)
    tile_gemm<FMT, PASS, NB, MI, true>(P, W0, W1, pos0, cnt, nt, As);
  else
    tile_gemm<FMT, PASS, NB, MI, false>(P, W0, W1, pos0, cnt, nt, As);
}

// Work item (tile of list `list`, column tile nt) with MI-row register blocks.
template <int PASS, int NB, int MI, bool MXP>
QMOE_D void prefill_item(const PrefillParams& P, int list, int tile, int nt, uint16_t* As) {
  const int2 te = P.tiles[(list ? P.tiles_cap_big : 0) + tile];
  const int e = te.x;
  qmoe_tier t;
  if (!prefill_tier(P, e, t)) return;
  const int pos0 = P.offsets[e] + te.y * kBM;
  const int cnt = min(kBM, P.offsets[e + 1] - pos0);
  const int fmt = PASS == 1 ? t.fmt_gate_up : t.fmt_down;
  const int N = PASS == 1 ? P.F : P.H, K = PASS == 1 ? P.H : P.F;
  const size_t eo = (size_t)(e - t.e_begin) * layout_of(fmt, N, K).total;
  const uint8_t* W0 = (const uint8_t*)(PASS == 1 ? t.gate : t.down) + eo;
  const uint8_t* W1 = (const uint8_t*)t.up + eo;
  switch (fmt) {
    case QMOE_Q8_0: tile_dispatch_full<QMOE_Q8_0, PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, As); break;
    case QMOE_Q4_0: tile_dispatch_full<QMOE_Q4_0, PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, As); break;
    case QMOE_MXFP4:
      if constexpr (MXP) {
        if (t.fmt_gate_up == QMOE_MXFP4 && t.fmt_down == QMOE_MXFP4) {
          tile_mx<PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, (float*)As);
          break;
        }
      }
      tile_dispatch_full<QMOE_MXFP4, PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, As);
      break;
    case QMOE_Q4_K: tile_dispatch_full<QMOE_Q4_K, PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, As); break;
    case QMOE_Q6_K: tile_dispatch_full<QMOE_Q6_K, PASS, NB, MI>(P, W0, W1, pos0, cnt, nt, As); break;
    default: break;
  }
}

// One launch per pass: block b takes work items b, b + gridDim.x, ... of the
// (tile, column tile) items of the big-tile list, then of the small-tile
// list, so that the many-row tiles (bound by the matrix cores) and the
// few-row tiles (bound by the weight stream) run side by side (the gate/up
// launch has a block per item, the down launch the resident blocks).  Item w of
// a list runs on XCD w & 7 (the grid and each list's item count are multiples
// of 8); the column tiles of one row tile share an XCD and follow each other
// there, so its staged activation rows are read from that XCD's L2.
// MXP: MXFP4/MXFP4 tiers take the block-scaled path (instantiated apart, so
// the plain kernels keep their registers).
template <int PASS, int NB, bool MXP>
__global__ __launch_bounds__(kPB, 2) void prefill_kernel(PrefillParams P) {
  __shared__ __align__(16) uint16_t As[2 * 16 * kMI * kAS];
  const int ntl = P.ntiles;
  const int count_big = P.counts[0], count_small = P.counts[1];
  const int items_big = (count_big + 7) / 8 * 8 * ntl;
  const int items = items_big + (count_small + 7) / 8 * 8 * ntl;
  for (int w0 = blockIdx.x; w0 < items; w0 += gridDim.x) {
    const bool big = w0 < items_big;  // block-uniform
    const int w = big ? w0 : w0 - items_big;
    const int slot = w >> 3;
    const int tile = (slot / ntl) * 8 + (w & 7), nt = slot - (slot / ntl) * ntl;
    if (tile >= (big ? count_big : count_small)) continue;  // block-uniform
    if (big) prefill_item<PASS, NB, kMI, MXP>(P, 0, tile, nt, As);
    else prefill_item<PASS, NB, kMIsmall, MXP>(P, 1, tile, nt, As);
  }
}

// Block 0: the two tile lists.  Expert e's rows are cut into kBM-row tiles
// t = 0, 1, ...; tile (e, t) goes to the big list when it holds more than
// kSmall rows, else to the small list, each list in expert order.
// counts[0], counts[1]: the lists' lengths.  Other blocks: x (fp32 or bf16)
// [T, H] -> x16 [T + 1, xs] fp16 with zero padding and a zero last row, and
// zeros in h [A + 1, hs] past column F and in its last row.
__global__ __launch_bounds__(kPB) void prefill_prep_kernel(const int32_t* offsets, int E,
                                                           int cap_big, int2* tiles, int* counts,
                                                           const void* x, int x_dtype, int T,
                                                           int H, int xs, uint16_t* x16, int A,
                                                           int F, int hs, uint16_t* h16) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    __shared__ int wsum[2][kPW];
    const int lane = tid & 63, wave = tid >> 6;
    const int per = (E + kPB - 1) / kPB;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    auto split = [&](int m, int& nb, int& ns) {  // big / small tiles of m rows
      const int full = m / kBM, rest = m - full * kBM;
      nb = full + (rest > kSmall);
      ns = rest > 0 && rest <= kSmall;
    };
    int lb = 0, ls = 0;
    for (int e = lo; e < hi; ++e) {
      int nb, ns;
      split(offsets[e + 1] - offsets[e], nb, ns);
      lb += nb;
      ls += ns;
    }
    int vb = lb, vs = ls;
    for (int off = 1; off < 64; off <<= 1) {
      const int ob = __shfl_up(vb, off, 64), os = __shfl_up(vs, off, 64);
      if (lane >= off) { vb += ob; vs += os; }
    }
    if (lane == 63) { wsum[0][wave] = vb; wsum[1][wave] = vs; }
    __syncthreads();
    int rb = vb - lb, rs = vs - ls;
    for (int w = 0; w < wave; ++w) { rb += wsum[0][w]; rs += wsum[1][w]; }
    if (tid == kPB - 1) {
      counts[0] = rb + lb;
      counts[1] = rs + ls;
    }
    for (int e = lo; e < hi; ++e) {
      const int m = offsets[e + 1] - offsets[e];
      for (int t = 0; t * kBM < m; ++t) {
        if (min(kBM, m - t * kBM) > kSmall) tiles[rb++] = make_int2(e, t);
        else tiles[cap_big + rs++] = make_int2(e, t);
      }
    }
    return;
  }
  // 8-value chunks: x16 rows 0..T, then the padding of h
  const long long xc = (long long)(T + 1) * (xs / 8);
  const int pc = (hs - F) / 8;
  const long long hc = (long long)A * pc + hs / 8;
  const long long stride = (long long)(gridDim.x - 1) * kPB;
  for (long long i = (long long)(blockIdx.x - 1) * kPB + tid; i < xc + hc; i += stride) {
    uint4 out = make_uint4(0u, 0u, 0u, 0u);
    if (i < xc) {
      const long long row = i / (xs / 8);
      const int col = 8 * (int)(i - row * (xs / 8));
      if (row < T && col < H) {
        const long long at = row * H + col;
        if (x_dtype == QMOE_F32) {
          const float4 a = *(const float4*)((const float*)x + at);
          const float4 b = *(const float4*)((const float*)x + at + 4);
          out = make_uint4(pack_h2(a.x, a.y), pack_h2(a.z, a.w), pack_h2(b.x, b.y),
                           pack_h2(b.z, b.w));
        } else {
          const uint4 v = *(const uint4*)((const uint16_t*)x + at);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = pack_h2(bf16_bits_to_f32(w[j] & 0xFFFFu), bf16_bits_to_f32(w[j] >> 16));
          out = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
      *(uint4*)(x16 + row * xs + col) = out;
    } else {
      const long long j = i - xc;
      const long long pad = (long long)A * pc;
      const long long at = j < pad ? (j / pc) * hs + F + 8 * (j % pc) : (long long)A * hs + 8 * (j - pad);
      *(uint4*)(h16 + at) = out;
    }
  }
}

// Block-scaled path: x (fp32 or bf16) [T, H] -> MXFP8 x8 [T + 1, xs] and
// x8s [T + 1, xs / 32] (32-value blocks past H and the last row: zero codes,
// scale byte 0), and zero codes / scales in h8's last row and its blocks
// past F.  One thread per 32-value block.
__global__ __launch_bounds__(kPB) void prefill_mx_prep_kernel(const void* x, int x_dtype, int T,
                                                              int H, int xs, uint8_t* x8,
                                                              uint8_t* x8s, int A, int F, int hs,
                                                              uint8_t* h8, uint8_t* h8s) {
  const long long xb = (long long)(T + 1) * (xs / 32);
  const int pb = (hs - F) / 32;                     // pad blocks per h8 row
  const long long hb = (long long)A * pb + hs / 32;  // pads, then the last row
  const long long i = (long long)blockIdx.x * kPB + threadIdx.x;
  if (i >= xb + hb) return;
  uint32_t out[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t e = 0;
  uint8_t* codes;
  uint8_t* scale;
  if (i < xb) {
    const long long row = i / (xs / 32);
    const int blk = (int)(i - row * (xs / 32));
    if (row < T && 32 * blk < H) {
      float v[32];
      const long long at = row * H + 32 * blk;
#pragma unroll
      for (int j = 0; j < 32; ++j)
        v[j] = x_dtype == QMOE_F32 ? ((const float*)x)[at + j]
                                   : bf16_bits_to_f32(((const uint16_t*)x)[at + j]);
      e = mx_quantize32(v, out);
    }
    codes = x8 + row * xs + 32 * blk;
    scale = x8s + row * (xs / 32) + blk;
  } else {
    const long long j = i - xb;
    const long long pad = (long long)A * pb;
    const long long row = j < pad ? j / pb : A;
    const int blk = j < pad ? F / 32 + (int)(j % pb) : (int)(j - pad);
    codes = h8 + row * hs + 32 * blk;
    scale = h8s + row * (hs / 32) + blk;
  }
  uint4* dst = (uint4*)codes;
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  *scale = (uint8_t)e;
}

// Activation row strides: whole K steps.
QMOE_HD int step_round(int K) { return (K + kBK - 1) / kBK * kBK; }

// List capacities for A assignments over E experts: a big tile holds more
// than kSmall rows; only an expert's last tile can be small.
QMOE_HD long long prefill_cap_big(long long A) { return A / (kSmall + 1) + 1; }
QMOE_HD long long prefill_cap_small(long long A, int E) { return (A < E ? A : E) + 1; }

// Resident blocks of a persistent prefill kernel: what the occupancy
// calculator allows per compute unit, times the compute units, rounded
// down to whole groups of 8 (one per XCD).
template <class Kernel>
static int persistent_grid(Kernel kernel) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kPB, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const int g = per_cu * cus;
  return g >= 8 ? g / 8 * 8 : 8;
}

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);

// Workspace: fp16 h and x, the tile lists, then the MXFP8 rows and scales of
// x and h (used by the block-scaled path only).
static size_t mx_bytes(long long rows, int stride) {
  return round_up256((size_t)rows * stride) + round_up256((size_t)rows * (stride / 32));
}

static size_t prefill_workspace_bytes(int T, int k, int E, int H, int F) {
  if (T < 0 || k < 0 || E <= 0 || H < 0 || F < 0) return 0;
  const long long A = (long long)T * k;
  return round_up256((size_t)(A + 1) * step_round(F) * sizeof(uint16_t)) +
         round_up256((size_t)(T + 1) * step_round(H) * sizeof(uint16_t)) +
         round_up256((size_t)(prefill_cap_big(A) + prefill_cap_small(A, E)) * sizeof(int2)) +
         256 + 256 + mx_bytes(T + 1, step_round(H)) + mx_bytes(A + 1, step_round(F));
}

// one launch per pass (both tile lists)
template <bool MXP>
static int prefill_launch(PrefillParams P, hipStream_t s) {
  static int grid_down = 0;
  if (!grid_down) grid_down = persistent_grid(prefill_kernel<2, kNB2, MXP>);
  // Pass 1 takes one block per possible item (the list capacities bound the
  // items; blocks past the lists' real items exit at once), so the hardware's
  // block dispatch balances items of unequal cost: gate/up 420 -> 398 us on
  // the 2048-row chunk.  Pass 2 keeps the resident grid (one block per item
  // measured 233 -> 238 us there).
  const long long A = (long long)P.T * P.k;
  const long long list_slots =
      (prefill_cap_big(A) + 7) / 8 * 8 + (prefill_cap_small(A, P.E) + 7) / 8 * 8;
  P.ntiles = (P.F + kPW * kNB1 * 16 - 1) / (kPW * kNB1 * 16);
  const long long items1 = list_slots * P.ntiles;
  if (items1 >= (1LL << 31)) return fail(QMOE_ERR_UNSUPPORTED, "prefill: too many work items");
  int st = QMOE_LAUNCH("prefill_gate_up", (prefill_kernel<1, kNB1, MXP>), dim3((unsigned)items1),
                       kPB, 0, s, P);
  if (st) return st;
  P.ntiles = (P.H + kPW * kNB2 * 16 - 1) / (kPW * kNB2 * 16);
  return QMOE_LAUNCH("prefill_down", (prefill_kernel<2, kNB2, MXP>), dim3(grid_down), kPB, 0, s, P);
}

static int prefill_run(const char* who, bool mx, const qmoe_tier* tiers, int n_tiers, int E,
                       int H, int F, const void* x, int x_dtype, int T, int k,
                       const int32_t* offsets, const int32_t* perm, float* o, void* ws,
                       size_t ws_bytes, void* stream) {
  if (T < 0 || k < 0)
    return fail(QMOE_ERR_INVALID_ARG, "%s: T=%d k=%d", who, T, k);
  if (T == 0 || k == 0) return QMOE_OK;
  int st = validate_tiers(tiers, n_tiers, E, H, F, true);
  if (st) return st;
  if (E > 8192) return fail(QMOE_ERR_UNSUPPORTED, "%s: E=%d > 8192", who, E);
  if (H % 64 || F % 64)
    return fail(QMOE_ERR_INVALID_ARG, "%s: H and F must be multiples of 64", who);
  if ((long long)H * F >= (1LL << 32))  // plane offsets are 32-bit
    return fail(QMOE_ERR_UNSUPPORTED, "%s: H*F too large", who);
  if (!x || !offsets || !perm || !o)
    return fail(QMOE_ERR_INVALID_ARG, "%s: null pointer", who);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: unknown x_dtype %d", who, x_dtype);
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(o, 16))
    return fail(QMOE_ERR_INVALID_ARG, "%s: misaligned x/o", who);
  const size_t need = prefill_workspace_bytes(T, k, E, H, F);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, need);
  const long long A = (long long)T * k;
  if (A > (1 << 24)) return fail(QMOE_ERR_UNSUPPORTED, "%s: T*k too large", who);
  hipStream_t s = (hipStream_t)stream;
  PrefillParams P{};
  for (int i = 0; i < n_tiers; ++i) P.tiers[i] = tiers[i];
  P.n_tiers = n_tiers; P.E = E; P.H = H; P.F = F; P.T = T; P.k = k;
  P.offsets = offsets; P.perm = perm; P.o = o;
  P.xs = step_round(H);
  P.hs = step_round(F);
  char* w = (char*)ws;
  P.h = (uint16_t*)w;
  w += round_up256((size_t)(A + 1) * P.hs * sizeof(uint16_t));
  uint16_t* x16 = (uint16_t*)w;
  P.x16 = x16;
  w += round_up256((size_t)(T + 1) * P.xs * sizeof(uint16_t));
  int* counts = (int*)w;
  P.counts = counts;
  w += 256;
  int2* tiles = (int2*)w;
  P.tiles = tiles;
  P.tiles_cap_big = (int)prefill_cap_big(A);
  w += round_up256((size_t)(prefill_cap_big(A) + prefill_cap_small(A, E)) * sizeof(int2));
  uint8_t* x8 = (uint8_t*)w;
  P.x8 = x8;
  w += round_up256((size_t)(T + 1) * P.xs);
  uint8_t* x8s = (uint8_t*)w;
  P.x8s = x8s;
  w += round_up256((size_t)(T + 1) * (P.xs / 32));
  P.h8 = (uint8_t*)w;
  w += round_up256((size_t)(A + 1) * P.hs);
  P.h8s = (uint8_t*)w;
  const long long chunks = (long long)(T + 1) * (P.xs / 8) + A * ((P.hs - F) / 8) + P.hs / 8;
  const long long conv_blocks = std::min<long long>(1024, (chunks + kPB - 1) / kPB);
  st = QMOE_LAUNCH("prefill_prep", prefill_prep_kernel, dim3((unsigned)(1 + conv_blocks)), kPB, 0,
                   s, offsets, E, P.tiles_cap_big, tiles, counts, x, x_dtype, T, H, P.xs, x16,
                   (int)A, F, P.hs, P.h);
  if (st) return st;
  if (mx) {
    const long long blocks = (long long)(T + 1) * (P.xs / 32) + A * ((P.hs - F) / 32) + P.hs / 32;
    st = QMOE_LAUNCH("prefill_mx_prep", prefill_mx_prep_kernel,
                     dim3((unsigned)((blocks + kPB - 1) / kPB)), kPB, 0, s, x, x_dtype, T, H,
                     P.xs, x8, x8s, (int)A, F, P.hs, P.h8, P.h8s);
    if (st) return st;
  }
  return mx ? prefill_launch<true>(P, s) : prefill_launch<false>(P, s);
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

size_t qgemm_grouped_prefill_workspace_size(int T, int k, int E, int H, int F) {
  return prefill_workspace_bytes(T, k, E, H, F);
}

int qgemm_grouped_prefill(const qmoe_tier* tiers, int n_tiers, int E, int H, int F,
                          const void* x, int x_dtype, int T, int k, const int32_t* offsets,
                          const int32_t* perm, float* o, void* ws, size_t ws_bytes,
                          void* stream) {
  return prefill_run("qgemm_grouped_prefill", false, tiers, n_tiers, E, H, F, x, x_dtype, T, k,
                     offsets, perm, o, ws, ws_bytes, stream);
}

int qgemm_grouped_prefill_mx(const qmoe_tier* tiers, int n_tiers, int E, int H, int F,
                             const void* x, int x_dtype, int T, int k, const int32_t* offsets,
                             const int32_t* perm, float* o, void* ws, size_t ws_bytes,
                             void* stream) {
  return prefill_run("qgemm_grouped_prefill_mx", true, tiers, n_tiers, E, H, F, x, x_dtype, T,
                     k, offsets, perm, o, ws, ws_bytes, stream);
}

}  // extern "C"
