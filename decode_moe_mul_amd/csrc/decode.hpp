// Internal header: the decode-side building blocks shared by the routed FFN
// kernels and the one-launch decode layer -- weight units and their decode,
// activation staging, the fp16 dot-product and matrix-core row passes, the
// block schedule over routed experts -- and the host-side choices of lanes
// per row, register blocking and row tiles.
//
// Include it after any header whose arithmetic must keep the default
// contraction: from here on nothing is contracted.
#pragma once
#include <algorithm>

#include "common.hpp"
#include "dequant.hpp"

// Every fused multiply-add below is written out (fmaf); nothing else is
// contracted, so a row's arithmetic does not depend on which register slot
// (row position within a chunk) it occupies.
#pragma clang fp contract(off)

namespace qmoe {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kLdsCap = 65536 - 256;

struct Mat {
  const uint8_t* base;
  const uint8_t* p0;
  const uint8_t* p1;
  const uint8_t* p2;
  const uint8_t* p3;
};

QMOE_D Mat mat_of(const void* base, int fmt, int N, int K) {
  const Layout L = layout_of(fmt, N, K);
  const uint8_t* b = (const uint8_t*)base;
  return {b, b + L.off[0], b + L.off[1], b + L.off[2], b + L.off[3]};
}

// ---------------------------------------------------- one 32-value unit --
// Raw bytes of unit u of one weight row (loaded early), and its decode into
// 16 fp16-pair code words plus fp32 coefficients:
//   Q8_0/Q4_0/MXFP4: value = c0 * code
//   Q4_K:            value = c0 * code - c1   (c1 multiplies the sum of x)
//   Q6_K:            value = c0 * code (values 0..15), c1 * code (16..31)
template <int FMT>
struct Unit {
  uint4 q, q2;   // codes (q2: second half of a Q8_0 unit)
  uint4 meta;    // Q4_K superblock meta
  uint2 qh;      // Q6_K high bits
  uint32_t s0, s1;

  // Offsets are 32-bit (a plane of one matrix is < 4 GiB) and products use
  // the 24-bit multiplier (row < 65536, row strides <= 32 KiB), so a load
  // costs a couple of vector instructions on top of the matrix's scalar base.
  QMOE_D void load(const Mat& M, int row, int u, int K) {
    const uint32_t r = (uint32_t)row, uu = (uint32_t)u, nb32 = (uint32_t)(K >> 5);
    if constexpr (FMT == QMOE_Q8_0) {
      const uint32_t qo = mad24(r, (uint32_t)K, uu << 5);
      q = load_stream(M.p0 + qo);
      q2 = load_stream(M.p0 + qo + 16u);
      s0 = *(const uint16_t*)(M.p1 + (mad24(r, nb32, uu) << 1));
    } else {
      const uint32_t qo = mad24(r, (uint32_t)(K >> 1), uu << 4);
      q = load_stream(M.p0 + qo);
      if constexpr (FMT == QMOE_Q4_0) {
        s0 = *(const uint16_t*)(M.p1 + (mad24(r, nb32, uu) << 1));
      } else if constexpr (FMT == QMOE_MXFP4) {
        s0 = M.p1[mad24(r, nb32, uu)];
      } else if constexpr (FMT == QMOE_Q4_K) {
        meta = *(const uint4*)(M.p1 + (mad24(r, (uint32_t)(K >> 8), uu >> 3) << 4));
      } else {
        qh = *(const uint2*)(M.p1 + mad24(r, (uint32_t)(K >> 2), uu << 3));
        const uint32_t sb = mad24(r, (uint32_t)(K >> 8), uu >> 3);
        // the aligned word holding the unit's two sub-block scales (bytes
        // 2j, 2j+1 of the super-block's 16, j = u & 7; picked at decode)
        s0 = *(const uint32_t*)(M.p2 + (sb << 4) + ((uu & 6u) << 1));
        s1 = *(const uint16_t*)(M.p3 + (sb << 1));
      }
    }
  }

  // unit coefficients (see above)
  QMOE_D void coefs(int u, float& c0, float& c1) const {
    if constexpr (FMT == QMOE_Q8_0 || FMT == QMOE_Q4_0) {
      c0 = f16_bits_to_f32(s0);
      c1 = 0.f;
    } else if constexpr (FMT == QMOE_MXFP4) {
      c0 = e8m0_to_f32(s0);
      c1 = 0.f;
    } else if constexpr (FMT == QMOE_Q4_K) {
      // 6-bit fields of the 96-bit word (y, z, w): sc_j at bit 6j, m_j at
      // bit 48 + 6j; 32-bit funnel shifts only, so the loaded words are used
      // in place (no 64-bit register pairs to assemble)
      // (operands are selected first so that no branch is generated)
      const uint32_t b = 6u * (uint32_t)(u & 7), bm = b + 16u;
      const bool lo_b = b < 32u, lo_m = bm < 32u;
      const uint32_t sc = __builtin_amdgcn_alignbit(lo_b ? meta.z : meta.w, lo_b ? meta.y : meta.z,
                                                    b & 31u) & 63u;
      const uint32_t mn = __builtin_amdgcn_alignbit(lo_m ? meta.w : 0u, lo_m ? meta.z : meta.w,
                                                    bm & 31u) & 63u;
      c0 = f16_bits_to_f32(meta.x & 0xFFFFu) * (float)sc;
      c1 = f16_bits_to_f32(meta.x >> 16) * (float)mn;
    } else {
      const float d = f16_bits_to_f32(s1);
      const uint32_t sh = (uint32_t)(u & 1) * 16u;
      // (the builtin's result type is unsigned: reinterpret before converting)
      c0 = d * (float)(int)__builtin_amdgcn_sbfe(s0, sh, 8u);
      c1 = d * (float)(int)__builtin_amdgcn_sbfe(s0, sh + 8u, 8u);
    }
  }

  // biased codes in the dot-product pair order (pair_elem_biased)
  QMOE_D void decode(int u, uint32_t codes[16], float& c0, float& c1) const {
    if constexpr (FMT == QMOE_Q8_0) bytes_biased(q, q2, codes);
    else if constexpr (FMT == QMOE_MXFP4) e2m1_natural(q, codes);
    else if constexpr (FMT == QMOE_Q6_K) q6_biased(q, qh, codes);
    else nibbles_biased(q, codes);
    coefs(u, c0, c1);
  }

  // The 8-value slice [8g, 8g + 8) of unit u for the matrix-core path:
  // q.x (Q8_0: q.x, q.y) holds its codes; scales as for the whole unit.
  QMOE_D void load_slice(const Mat& M, int row, int u, int g, int K) {
    const uint32_t r = (uint32_t)row, uu = (uint32_t)u, gg = (uint32_t)g, nb32 = (uint32_t)(K >> 5);
    if constexpr (FMT == QMOE_Q8_0) {
      const uint2 v = *(const uint2*)(M.p0 + mad24(r, (uint32_t)K, (uu << 5) + (gg << 3)));
      q.x = v.x;
      q.y = v.y;
      s0 = *(const uint16_t*)(M.p1 + (mad24(r, nb32, uu) << 1));
    } else {
      q.x = *(const uint32_t*)(M.p0 + mad24(r, (uint32_t)(K >> 1), (uu << 4) + (gg << 2)));
      if constexpr (FMT == QMOE_Q4_0) {
        s0 = *(const uint16_t*)(M.p1 + (mad24(r, nb32, uu) << 1));
      } else if constexpr (FMT == QMOE_MXFP4) {
        s0 = M.p1[mad24(r, nb32, uu)];
      } else if constexpr (FMT == QMOE_Q4_K) {
        meta = *(const uint4*)(M.p1 + (mad24(r, (uint32_t)(K >> 8), uu >> 3) << 4));
      } else {
        // high bits of values 8g..8g+7: bytes 2g, 2g + 1 of the unit's 8,
        // read as the aligned word holding them (half picked at decode)
        qh.x = *(const uint32_t*)(M.p1 + mad24(r, (uint32_t)(K >> 2), (uu << 3) + ((gg >> 1) << 2)));
        const uint32_t sb = mad24(r, (uint32_t)(K >> 8), uu >> 3);
        s0 = *(const uint32_t*)(M.p2 + (sb << 4) + ((uu & 6u) << 1));
        s1 = *(const uint16_t*)(M.p3 + (sb << 1));
      }
    }
  }

  // the slice as 4 fp16 pair words in slice order (slice_elem): exact codes,
  // or biased ones (1024 + code, 1024 + 16 code on odd pairs) for Q4_0/Q4_K
  QMOE_D void decode_slice(int u, int g, uint32_t out[4], float& c0, float& c1) const {
    if constexpr (FMT == QMOE_Q8_0) {
      const uint32_t w[2] = {q.x ^ 0x80808080u, q.y ^ 0x80808080u};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        out[2 * i] = pk_add_h2(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04020400u), H2_NEG_1152);
        out[2 * i + 1] = pk_add_h2(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04030401u), H2_NEG_1152);
      }
    } else if constexpr (FMT == QMOE_MXFP4) {
      out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q.x, 1.f, 0));
      out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q.x, 1.f, 1));
      out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q.x, 1.f, 2));
      out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q.x, 1.f, 3));
    } else if constexpr (FMT == QMOE_Q6_K) {
      const uint32_t h16 = (g & 1) ? qh.x >> 16 : qh.x & 0xFFFFu;
      const uint32_t hh = (h16 & 0xFFu) | ((h16 & 0xFF00u) << 8);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = (q.x >> (4 * p)) & 0x000F000Fu;
        const uint32_t hi = ((hh >> (2 * p)) & 0x00030003u) << 4;
        out[p] = pk_add_h2(lo | hi | H2_MAGIC, H2_NEG_1056);
      }
    } else {
      // plain and/or here, not the and_or helper: these words feed the
      // matrix cores, and the compiler only inserts the wait states a
      // vector write needs before a matrix-core read for code it generated
      const uint32_t t = q.x >> 8;
      out[0] = (q.x & 0x000F000Fu) | H2_MAGIC;
      out[1] = (q.x & 0x00F000F0u) | H2_MAGIC;
      out[2] = (t & 0x000F000Fu) | H2_MAGIC;
      out[3] = (t & 0x00F000F0u) | H2_MAGIC;
    }
    coefs(u, c0, c1);
  }
};

// acc + <unit, one staged activation row>, from the biased codes; bv holds
// the unit's staged sums for that row (see stage_rows).
template <int FMT>
QMOE_D float unit_dot(const uint32_t codes[16], float c0, float c1, const uint32_t xv[16],
                      float2 bv, float acc) {
  float s0 = 0.f, s1 = 0.f;
  if constexpr (FMT == QMOE_Q6_K) {
#pragma unroll
    for (int p = 0; p < 8; ++p) s0 = fdot2(codes[p], xv[p], s0);
#pragma unroll
    for (int p = 8; p < 16; ++p) s1 = fdot2(codes[p], xv[p], s1);
    return fmaf(c1, s1 - bv.y, fmaf(c0, s0 - bv.x, acc));
  } else {
#pragma unroll
    for (int p = 0; p < 16; p += 2) {
      s0 = fdot2(codes[p], xv[p], s0);
      s1 = fdot2(codes[p + 1], xv[p + 1], s1);
    }
    acc = fmaf(c0, (s0 + s1) - bv.x, acc);
    if constexpr (FMT == QMOE_Q4_K) acc = fmaf(-c1, bv.y, acc);
    return acc;
  }
}

// ---------------------------------------------- staged activation rows --
// Row r of a chunk occupies `tok_stride(U)` bytes of LDS: unit u (16 words)
// at byte 64u + 16(u/4).  The 16-byte pad after every 4 units puts the 16-byte
// reads of 8 consecutive lanes (consecutive units) on distinct banks.
QMOE_HD int tok_stride(int U) { return 64 * U + 16 * ((U + 3) >> 2); }
QMOE_HD int unit_off(int u) { return 64 * u + 16 * (u >> 2); }

// Activation rows written earlier in the same launch by other blocks are read
// with coherent loads (COH, or XDT = kF32Coherent): fp32, past the L2.
constexpr int kF32Coherent = 0x100;

// 32 activation values (fp32 or raw bf16) starting at element 32u of row.
template <bool COH = false>
QMOE_D void load32(const void* row, int dtype, int u, float v[32]) {
  if constexpr (COH) {
    const float* p = (const float*)row + 32 * u;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = load_coherent(p + i);
  } else if (dtype == QMOE_F32) {
    const float4* p = (const float4*)((const float*)row + 32 * u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = (const uint4*)((const uint16_t*)row + 32 * u);
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
}

// Stage rc activation rows for format FMT: per unit, 16 fp16 pair words in
// the biased-code pair order (odd pairs of the 4/6-bit formats divided by
// 16) and two fp32 sums that remove the code bias from the unit's dot
// product.  With S = sum of the staged values and X = sum of the values the
// codes effectively meet (staged value, times 16 on the divided pairs):
//   Q4_0: {1024 S + 8 X, 0}          Q4_K: {1024 S, X}  (X meets the min)
//   Q6_K: {1024 S + 32 X} over elements 0..15 and over 16..31
//   Q8_0: {1152 S, 0}                MXFP4: {0, 0}
template <int FMT>
QMOE_D void stage_unit(uint8_t* xs, float2* sb, int r, int u, int U, const float (&v)[32]) {
  uint32_t w[16];
  float S[2] = {0.f, 0.f}, X[2] = {0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const bool up4 = pair_up4<FMT>(p);
    const float sc = up4 ? 0.0625f : 1.f;
    const float a = f16_bits_to_f32(f32_to_f16_bits(v[pair_elem_biased<FMT>(p, 0)])) * sc;
    const float b = f16_bits_to_f32(f32_to_f16_bits(v[pair_elem_biased<FMT>(p, 1)])) * sc;
    w[p] = pack_h2(a, b);
    const float fa = f16_bits_to_f32(w[p] & 0xFFFFu), fb = f16_bits_to_f32(w[p] >> 16);
    S[p >> 3] += fa + fb;
    X[p >> 3] += up4 ? 16.f * (fa + fb) : fa + fb;
  }
  float2 out = make_float2(0.f, 0.f);
  if constexpr (FMT == QMOE_Q4_0) out.x = 1024.f * (S[0] + S[1]) + 8.f * (X[0] + X[1]);
  if constexpr (FMT == QMOE_Q4_K) out = make_float2(1024.f * (S[0] + S[1]), X[0] + X[1]);
  if constexpr (FMT == QMOE_Q6_K)
    out = make_float2(1024.f * S[0] + 32.f * X[0], 1024.f * S[1] + 32.f * X[1]);
  if constexpr (FMT == QMOE_Q8_0) out.x = 1152.f * (S[0] + S[1]);
  sb[r * U + u] = out;
  uint4* dst = (uint4*)(xs + (size_t)r * tok_stride(U) + unit_off(u));
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  dst[2] = make_uint4(w[8], w[9], w[10], w[11]);
  dst[3] = make_uint4(w[12], w[13], w[14], w[15]);
}

template <int FMT, bool COH = false, class Src>
QMOE_D void stage_rows(uint8_t* xs, float2* sb, int rc, int U, Src src, int dtype) {
  for (int idx = threadIdx.x; idx < rc * U; idx += kBlock) {
    const int r = idx / U, u = idx - r * U;
    float v[32];
    load32<COH>(src(r), dtype, u, v);
    stage_unit<FMT>(xs, sb, r, u, U, v);
  }
}

// ------------------------------------------------ DPP group reduction ---
template <int CTRL, int ROW_MASK>
QMOE_D float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); the group's
// total ends up in its last lane (lane G-1 of the group).
QMOE_D float group_reduce(float v, int G) {
  if (G >= 2) v += dpp_move<0x111, 0xF>(v);   // row_shr:1
  if (G >= 4) v += dpp_move<0x112, 0xF>(v);   // row_shr:2
  if (G >= 8) v += dpp_move<0x114, 0xF>(v);   // row_shr:4
  if (G >= 16) v += dpp_move<0x118, 0xF>(v);  // row_shr:8
  if (G >= 32) v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (G >= 64) v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// ---------------------------------------------- few rows: fp16 dots -----
// Units in flight per lane on the dot-product path: gate and up together
// hold two units per position.  FEW (the routed FFN, whose blocks are few
// and short): with one staged row the ring is deeper, so that a block
// requests most of its weights at once.  Streaming launches (a dense GEMV)
// keep the shallower ring and their occupancy.
template <int NMAT, int RC, bool FEW>
QMOE_HD constexpr int valu_depth() {
  return NMAT == 2 ? (FEW && RC <= 1 ? 4 : 3) : (FEW && RC <= 1 ? 5 : 4);
}

// The weight stream of one wave over rows [rb, re) of NMAT matrices: lane
// slot `slot` of each G-lane group takes row first + i * step + slot of row
// group i and units g, g + G, ... of it.  Positions are flat (row group,
// unit) pairs in consumption order; every load is unconditional (positions
// past the wave's last re-read the tile's last row), so no load sits behind
// a branch and each slot's data is consumed in the registers it was loaded
// into.
template <int FMT, int NMAT, int D>
struct ValuRing {
  Unit<FMT> buf[D][NMAT];
  int first, step, re, slot, g, G, UPL, n_rg, nflat;
  int irg, it;  // next position to load

  // (the wave-uniform fields are moved to scalar registers)
  QMOE_D ValuRing(int K, int rb, int re_, int G_) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    G = __builtin_amdgcn_readfirstlane(G_);
    const int sub = 64 / G;
    g = lane & (G - 1);
    slot = lane / G;
    UPL = __builtin_amdgcn_readfirstlane((K >> 5) / G);
    re = __builtin_amdgcn_readfirstlane(re_);
    first = __builtin_amdgcn_readfirstlane(rb) + wave * sub;
    step = kWaves * sub;
    n_rg = first < re ? (re - first + step - 1) / step : 0;
    nflat = n_rg * UPL;
    irg = 0;
    it = 0;
  }
  QMOE_D void issue(const Mat (&mats)[NMAT], int K, int i) {
    const int row = min(first + irg * step + slot, re - 1);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) buf[i][m].load(mats[m], row, g + it * G, K);
    if (++it == UPL) { it = 0; ++irg; }
  }
  // The first D positions, in the order the pass consumes them (the
  // scheduling barrier keeps the compiler from interleaving them).
  QMOE_D void prime(const Mat (&mats)[NMAT], int K) {
    irg = 0;
    it = 0;
    if (nflat == 0) return;  // wave-uniform
#pragma unroll
    for (int i = 0; i < D; ++i) {
      issue(mats, K, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Rows [rb, re) of NMAT matrices [*, K] against the rc (<= RC) staged rows,
// streaming through a primed ring.  sink(row, r, const float* v[NMAT]) is
// called once per (row, r).  NO_TAIL: the last round issues no loads (a
// few-row block then ends without loads in flight; elsewhere the second copy
// of the round costs more instruction cache than the loads cost time).
template <int FMT, int NMAT, int RC, int D, bool NO_TAIL, class Sink>
QMOE_D void valu_pass(const Mat (&mats)[NMAT], int K, ValuRing<FMT, NMAT, D>& ring, int rc,
                      const uint8_t* xs, const float2* sb, Sink sink) {
  const int G = ring.G, g = ring.g, UPL = ring.UPL;
  const int U = K >> 5, ts = tok_stride(U);
  if (ring.nflat == 0) return;  // wave-uniform

  auto compute = [&](Unit<FMT> (&w)[NMAT], int u, float (&acc)[NMAT][RC]) {
    // decode every matrix's unit once, then take the staged rows one at a
    // time (one row's activations live in registers at a time)
    uint32_t codes[NMAT][16];
    float c0[NMAT], c1[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) w[m].decode(u, codes[m], c0[m], c1[m]);
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      if (r < rc) {
        const uint4* xp = (const uint4*)(xs + (size_t)r * ts + unit_off(u));
        const uint4 v0 = xp[0], v1 = xp[1], v2 = xp[2], v3 = xp[3];
        const uint32_t xv[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                                 v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
        const float2 bv = FMT == QMOE_MXFP4 ? make_float2(0.f, 0.f) : sb[r * U + u];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m][r] = unit_dot<FMT>(codes[m], c0[m], c1[m], xv, bv, acc[m][r]);
      }
    }
  };

  float acc[NMAT][RC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[m][r] = 0.f;
  int crg = 0, ct = 0;  // (row group, unit) being computed
  // nflat rounded up to a multiple of D: the extra positions are computed on
  // re-read data and never stored (their row group is past the last).
  auto round = [&](bool refill) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      compute(ring.buf[i], g + ct * G, acc);
      if (refill) ring.issue(mats, K, i);
      if (++ct == UPL) {  // wave-uniform
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RC; ++r) acc[m][r] = group_reduce(acc[m][r], G);
        const int row = ring.first + crg * ring.step + ring.slot;
        if (crg < ring.n_rg && row < ring.re && g == G - 1) {
#pragma unroll
          for (int r = 0; r < RC; ++r) {
            if (r < rc) {
              float v[NMAT];
#pragma unroll
              for (int m = 0; m < NMAT; ++m) v[m] = acc[m][r];
              sink(row, r, v);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RC; ++r) acc[m][r] = 0.f;
        ct = 0;
        ++crg;
      }
    }
  };
  if constexpr (NO_TAIL) {
    int f0 = 0;
    for (; f0 + D < ring.nflat; f0 += D) round(true);
    round(false);
  } else {
    for (int f0 = 0; f0 < ring.nflat; f0 += D) round(true);
  }
}

// Stage up to `chunk` (<= RC) rows at a time and stream the tile against
// them.  FEW, with at most two rows per chunk and one staged unit per thread:
// each chunk's first weight units are requested right after its activations,
// so that both are in flight together (staging four rows needs the registers
// the ring would hold).
template <int FMT, int NMAT, int RC, bool COH = false, bool FEW = false, class SrcOf,
          class SinkOf>
QMOE_D void valu_rows(const Mat (&mats)[NMAT], int K, int rb, int re, int G, int rows_total,
                      int dtype, uint8_t* lds, SrcOf src_of, SinkOf sink_of, int chunk = RC) {
  constexpr int D = valu_depth<NMAT, RC, FEW>();
  constexpr bool kPrimeFirst = FEW && RC <= 2;
  const int U = K >> 5;
  uint8_t* xs = lds;
  float2* sb = (float2*)(lds + (size_t)chunk * tok_stride(U));
  for (int c0 = 0; c0 < rows_total; c0 += chunk) {
    const int rc = min(chunk, rows_total - c0);
    // the register blocking of the pass follows this chunk's row count, so
    // an expert with one row does not pay for the dots of RC rows
    auto sink = [&](int n, int r, const float* a) { sink_of(n, c0 + r, a); };
    auto pass = [&](ValuRing<FMT, NMAT, D>& ring) {
      if constexpr (RC >= 4) {
        if (rc > 2) {
          valu_pass<FMT, NMAT, 4, D, kPrimeFirst>(mats, K, ring, rc, xs, sb, sink);
          return;
        }
      }
      if constexpr (RC >= 2) {
        if (rc == 2) {
          valu_pass<FMT, NMAT, 2, D, kPrimeFirst>(mats, K, ring, rc, xs, sb, sink);
          return;
        }
      }
      valu_pass<FMT, NMAT, 1, D, kPrimeFirst>(mats, K, ring, rc, xs, sb, sink);
    };
    // early (block-uniform): one unit of one row per thread.  Loads complete
    // in issue order, so the activation loads go first: converting them then
    // waits only for them, with the weight loads still in flight.  Every
    // thread loads (the spare ones re-read the last unit) and only the first
    // rc * U store.
    const bool early = kPrimeFirst && rc * U <= kBlock;
    ValuRing<FMT, NMAT, D> ring(K, rb, re, G);
    const int idx = min((int)threadIdx.x, rc * U - 1);
    const int r = idx / U, u = idx - r * U;
    float v[32];
    if (early) {
      load32<COH>(src_of(c0 + r), dtype, u, v);
      __builtin_amdgcn_sched_barrier(0);
      ring.prime(mats, K);
    }
    __syncthreads();  // earlier readers of the LDS are done
    if (early) {
      if ((int)threadIdx.x < rc * U) stage_unit<FMT>(xs, sb, r, u, U, v);
    } else {
      stage_rows<FMT, COH>(xs, sb, rc, U, [&](int rr) { return src_of(c0 + rr); }, dtype);
    }
    __syncthreads();
    if (!early) ring.prime(mats, K);
    pass(ring);
  }
}

// ------------------------------------------- many rows: matrix cores ----
// Weight rows [cb, ce) of NMAT matrices [N, K] (the output columns) against
// rows_total activation rows, in 16 x 16 output tiles on the matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation).  One matrix-core op covers
// exactly one 32-value unit: lane (n = lane % 16, g = lane / 16) holds values
// [8g, 8g + 8) of unit u of weight row c + n as exact fp16 codes and the same
// values of activation row n rounded to fp16, so every product is exact and
// the unit's scale is applied to the op's fp32 result (weights are never
// rounded).  The 4-bit formats use biased codes (as on the dot-product path);
// two more ops against constant operands give the unit's activation sums that
// remove the bias and carry the Q4_K minimum.  Q6_K units have two 16-value
// sub-scales, so they take two ops with half the lanes zeroed.  The 4 waves
// split K (wave w takes units w, w + 4, ...) and add their partial tiles in
// LDS in wave order; each slot's next unit is loaded as soon as the slot is
// decoded, and the next unit's activations one unit ahead.
// 16-column blocks per pass (gate and up together hold twice the registers)
QMOE_HD constexpr int mfma_cols_per_pass(int nmat) { return nmat == 2 ? 2 : 4; }

// Position within the 8-value slice of member i of pair p, and whether the
// pair's codes sit four bits up (activations then divided by 16).
template <int FMT>
QMOE_HD int slice_elem(int p, int i) {
  if constexpr (FMT == QMOE_Q8_0) return 4 * (p >> 1) + (p & 1) + 2 * i;
  else if constexpr (FMT == QMOE_MXFP4) return 2 * p + i;
  else return p + 4 * i;
}
template <int FMT>
QMOE_HD bool slice_up4(int p) {
  return (FMT == QMOE_Q4_0 || FMT == QMOE_Q4_K) && (p & 1);
}
template <int FMT>
constexpr bool slice_biased() {
  return FMT == QMOE_Q4_0 || FMT == QMOE_Q4_K;
}

// 8 raw activation values [8g, 8g + 8) of unit u (fp32: 32 B; bf16: 16 B)
struct XRaw8 {
  uint4 a, b;
};

template <int XDT>
QMOE_D void xslice_load(const void* row, int u, int g, XRaw8& x) {
  if constexpr (XDT == QMOE_F32) {
    const uint4* p = (const uint4*)((const float*)row + 32 * u + 8 * g);
    x.a = p[0];
    x.b = p[1];
  } else if constexpr (XDT == kF32Coherent) {
    const float* p = (const float*)row + 32 * u + 8 * g;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_bit_cast(uint32_t, load_coherent(p + i));
    x.a = make_uint4(w[0], w[1], w[2], w[3]);
    x.b = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    x.a = *(const uint4*)((const uint16_t*)row + 32 * u + 8 * g);
  }
}

// fp16 pair words of the slice in the format's slice order (zeros if !valid)
template <int FMT, int XDT>
QMOE_D void xslice_pairs(const XRaw8& x, bool valid, uint32_t out[4]) {
  float v[8];
  if constexpr (XDT == QMOE_F32 || XDT == kF32Coherent) {
    const uint32_t w[8] = {x.a.x, x.a.y, x.a.z, x.a.w, x.b.x, x.b.y, x.b.z, x.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
  } else {
    const uint32_t w[4] = {x.a.x, x.a.y, x.a.z, x.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h = pack_f16(v[slice_elem<FMT>(p, 0)], v[slice_elem<FMT>(p, 1)]);
    if (slice_up4<FMT>(p)) h = pk_mul_h2(h, 0x2C002C00u);  // x 1/16, exact
    out[p] = valid ? h : 0u;
  }
}

QMOE_D f32x4_t mfma16(const uint32_t a[4], const uint32_t b[4], f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(f16x8_t, make_uint4(a[0], a[1], a[2], a[3])),
      __builtin_bit_cast(f16x8_t, make_uint4(b[0], b[1], b[2], b[3])), c, 0, 0, 0);
}

QMOE_HD size_t mfma_red_bytes(int nmat) {
  return (size_t)kWaves * mfma_cols_per_pass(nmat) * nmat * 4 * 64 * sizeof(float);
}

template <int FMT, int NMAT, int XDT, class SrcOf, class SinkOf>
QMOE_D void mfma_cols(const Mat (&mats)[NMAT], int K, int cb, int ce, int rows_total,
                      uint8_t* lds, SrcOf src_of, SinkOf sink_of) {
  constexpr int NC = mfma_cols_per_pass(NMAT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int U = K >> 5;
  const int nu = U > wave ? (U - wave + kWaves - 1) / kWaves : 0;  // this wave's units
  float* red = (float*)lds;  // [kWaves][NC][NMAT][4][64]
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // earlier readers of the LDS are done
  for (int r0 = 0; r0 < rows_total; r0 += 16) {
    const bool rvalid = r0 + n < rows_total;
    const void* xrow = src_of(rvalid ? r0 + n : r0);
    for (int cg = cb; cg < ce; cg += 16 * NC) {
      f32x4_t acc[NC][NMAT];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[c][m] = zero;
      if (nu > 0) {
        // loads are unconditional: rows past ce re-read row ce - 1 and units
        // past the wave's last re-read it (their results are not used)
        auto unit_of = [&](int ui) { return wave + kWaves * min(ui, nu - 1); };
        int wrow[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) wrow[c] = min(cg + 16 * c + n, ce - 1);
        // two slot sets, each holding one unit's slices, consumed in turn
        // and refilled with the unit two ahead: two units of loads are in
        // flight while one is computed
        Unit<FMT> wa[NC][NMAT], wb[NC][NMAT];
        XRaw8 xa_raw, xb_raw;
        auto fill = [&](Unit<FMT> (&w)[NC][NMAT], XRaw8& xr, int ui) {
          const int u = unit_of(ui);
          xslice_load<XDT>(xrow, u, g, xr);
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) w[c][m].load_slice(mats[m], wrow[c], u, g, K);
        };
        // keep = 0 for the unit past the wave's last (its slices are a re-read)
        auto step = [&](Unit<FMT> (&w)[NC][NMAT], XRaw8& xr, int ui, float keep) {
          const int u = unit_of(ui);
          uint32_t xa[4];
          xslice_pairs<FMT, XDT>(xr, rvalid, xa);
          f32x4_t s_st = zero, s_x = zero;  // sums of staged / effective activations
          if constexpr (slice_biased<FMT>()) {
            const uint32_t ones[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
            const uint32_t eff[4] = {0x3C003C00u, 0x4C004C00u, 0x3C003C00u, 0x4C004C00u};
            s_st = mfma16(xa, ones, zero);
            s_x = mfma16(xa, eff, zero);
          }
          uint32_t bw[NC][NMAT][4];
          float c0[NC][NMAT], c1[NC][NMAT];
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              w[c][m].decode_slice(u, g, bw[c][m], c0[c][m], c1[c][m]);
              c0[c][m] *= keep;
              c1[c][m] *= keep;
              // the decoded operands are materialised here (an empty volatile
              // asm the compiler cannot move or see through), so no part of
              // the decode sinks below the refill and the loaded words need
              // not outlive it
              asm volatile("" : "+v"(c0[c][m]), "+v"(c1[c][m]), "+v"(bw[c][m][0]),
                           "+v"(bw[c][m][1]), "+v"(bw[c][m][2]), "+v"(bw[c][m][3]));
            }
          // the barriers keep each set's refill in program order, so the wait
          // for a set leaves the other set's loads in flight
          __builtin_amdgcn_sched_barrier(0);
          fill(w, xr, ui + 2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              if constexpr (FMT == QMOE_Q6_K) {
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                  lo[p] = g < 2 ? bw[c][m][p] : 0u;
                  hi[p] = g < 2 ? 0u : bw[c][m][p];
                }
                const f32x4_t dl = mfma16(xa, lo, zero), dh = mfma16(xa, hi, zero);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  acc[c][m][j] = fmaf(c1[c][m], dh[j], fmaf(c0[c][m], dl[j], acc[c][m][j]));
              } else {
                const f32x4_t d = mfma16(xa, bw[c][m], zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  if constexpr (FMT == QMOE_Q4_K) {
                    acc[c][m][j] = fmaf(-c1[c][m], s_x[j],
                                        fmaf(c0[c][m], d[j] - 1024.f * s_st[j], acc[c][m][j]));
                  } else if constexpr (FMT == QMOE_Q4_0) {
                    acc[c][m][j] =
                        fmaf(c0[c][m], d[j] - (1024.f * s_st[j] + 8.f * s_x[j]), acc[c][m][j]);
                  } else {
                    acc[c][m][j] = fmaf(c0[c][m], d[j], acc[c][m][j]);
                  }
                }
              }
            }
          }
        };
        fill(wa, xa_raw, 0);
        __builtin_amdgcn_sched_barrier(0);
        fill(wb, xb_raw, 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int ui = 0; ui < nu; ui += 2) {
          step(wa, xa_raw, ui, 1.f);
          step(wb, xb_raw, ui + 1, ui + 1 < nu ? 1.f : 0.f);
        }
      }
      // lane holds activation rows r0 + 4g + j of weight row cg + 16c + n;
      // wave j adds the four waves' partials for row 4g + j in wave order
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            red[(((wave * NC + c) * NMAT + m) * 4 + j) * 64 + lane] = acc[c][m][j];
      __syncthreads();
      {
        const int j = wave, r = r0 + 4 * g + j;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int col = cg + 16 * c + n;
          if (col < ce && r < rows_total) {
            float v[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              float sum = red[(((0 * NC + c) * NMAT + m) * 4 + j) * 64 + lane];
#pragma unroll
              for (int w = 1; w < kWaves; ++w)
                sum += red[(((w * NC + c) * NMAT + m) * 4 + j) * 64 + lane];
              v[m] = sum;
            }
            sink_of(col, r, v);
          }
        }
      }
      __syncthreads();
    }
  }
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
  int ntiles, G, tile_rows;
  int m_max;       // experts with more rows use the matrix cores
  int ntiles_big;  // blocks (column tiles) per such expert
  int chunk;       // rows staged per dot-product pass (0: the kernel's RC)
};

// The tier holding expert e, assembled field by field with constant indices
// only: any runtime index or struct copy out of the by-value kernel argument
// would make the compiler spill the whole argument block to scratch.
QMOE_D bool tier_of(const qmoe_tier (&tiers)[QMOE_MAX_TIERS], int n_tiers, int e,
                    qmoe_tier& out) {
  bool found = false;
  int32_t eb = 0, ee = 0, fgu = 0, fd = 0;
  const void *g = nullptr, *u = nullptr, *d = nullptr;
#pragma unroll
  for (int i = 0; i < QMOE_MAX_TIERS; ++i) {
    const bool hit = !found && i < n_tiers && e >= tiers[i].e_begin && e < tiers[i].e_end;
    if (hit) {
      eb = tiers[i].e_begin; ee = tiers[i].e_end;
      fgu = tiers[i].fmt_gate_up; fd = tiers[i].fmt_down;
      g = tiers[i].gate; u = tiers[i].up; d = tiers[i].down;
      found = true;
    }
  }
  out.e_begin = eb; out.e_end = ee; out.fmt_gate_up = fgu; out.fmt_down = fd;
  out.gate = g; out.up = u; out.down = d;
  return found;
}

QMOE_D float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// Block schedule.  Experts with more than m_max rows ("big") come first with
// ntiles_big blocks each, then the experts with 1..m_max rows with ntiles
// blocks each, both groups in id order.  Returns the expert of block b (-1
// past the end) and sets its tile index, group, first position pos0 and row
// count m.  Thread t reads the row counts of experts [t per, (t + 1) per)
// from the offsets (E + 1 entries, global memory); the counts' prefix over
// the wave comes from ballots (one per bit of a thread's count), over the
// waves from red (2 * kWaves + 3 ints of LDS).  Block-wide; every thread gets
// the result.  Experts never routed to have no rows and are never scheduled,
// nor are ids outside [0, E) ([P2] bug items 1 and 3).
constexpr int kSchedRedInts = 2 * kWaves + 3;

QMOE_D int scheduled_expert(const int32_t* offsets, int E, int m_max, int b, int ntiles,
                            int ntiles_big, int* red, int& tile, bool& big, int& pos0,
                            int& m_out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int per = (E + kBlock - 1) / kBlock;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int nb = 0, ns = 0;
  // Up to kKeep experts per thread (E <= 1024): the thread's offsets stay in
  // registers for the lookup below, which then needs no second memory round
  // trip.  All kKeep + 1 loads are unconditional (clamped to offsets[E]).
  constexpr int kKeep = 4;
  const bool keep = per <= kKeep;  // block-uniform
  int ov[kKeep + 1];
  if (keep) {
#pragma unroll
    for (int j = 0; j <= kKeep; ++j) ov[j] = offsets[min(lo + j, E)];
#pragma unroll
    for (int j = 0; j < kKeep; ++j) {
      const int m = ov[j + 1] - ov[j];
      if (lo + j < hi) {
        nb += m > m_max;
        ns += m > 0 && m <= m_max;
      }
    }
  } else {
    int prev = lo < hi ? offsets[lo] : 0;
    for (int e0 = lo; e0 < hi; e0 += 4) {
      int nx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) nx[j] = e0 + j < hi ? offsets[e0 + j + 1] : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (e0 + j < hi) {
          const int m = nx[j] - prev;
          nb += m > m_max;
          ns += m > 0 && m <= m_max;
          prev = nx[j];
        }
      }
    }
  }
  // exclusive prefixes within the wave and wave totals, bit by bit
  int xb = 0, xs = 0, wb = 0, ws = 0;
  for (int bit = 0; (1 << bit) <= per; ++bit) {
    const uint64_t bb = __ballot((nb >> bit) & 1), bs = __ballot((ns >> bit) & 1);
    xb += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u)) << bit;
    xs += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0u)) << bit;
    wb += __popcll(bb) << bit;
    ws += __popcll(bs) << bit;
  }
  if ((tid & 63) == 0) { red[wave] = wb; red[kWaves + wave] = ws; }
  if (tid == 0) red[2 * kWaves] = -1;
  __syncthreads();
  int tb = 0, ts = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) { xb += red[w]; xs += red[kWaves + w]; }
    tb += red[w];
    ts += red[kWaves + w];
  }
  const long long big_blocks = (long long)tb * ntiles_big;
  big = b < big_blocks;
  const int rel = big ? b : (int)(b - big_blocks);
  const int per_expert = big ? ntiles_big : ntiles;
  const int want = rel / per_expert;
  tile = rel - want * per_expert;
  const int first = big ? xb : xs, count = big ? nb : ns;
  if ((big || want < ts) && want >= first && want < first + count) {
    int c = first;
    if (keep) {
#pragma unroll
      for (int j = 0; j < kKeep; ++j) {
        const int p0 = ov[j], m = ov[j + 1] - p0;
        if (lo + j < hi && (big ? m > m_max : (m > 0 && m <= m_max))) {
          if (c == want) {
            red[2 * kWaves] = lo + j;
            red[2 * kWaves + 1] = p0;
            red[2 * kWaves + 2] = m;
          }
          ++c;
        }
      }
    } else {
      for (int e = lo; e < hi; ++e) {
        const int p0 = offsets[e], m = offsets[e + 1] - p0;
        if (big ? m > m_max : (m > 0 && m <= m_max)) {
          if (c == want) {
            red[2 * kWaves] = e;
            red[2 * kWaves + 1] = p0;
            red[2 * kWaves + 2] = m;
            break;
          }
          ++c;
        }
      }
    }
  }
  __syncthreads();
  pos0 = red[2 * kWaves + 1];
  m_out = red[2 * kWaves + 2];
  return red[2 * kWaves];
}

// Weight rows [rb, re) of the phase's matrix that work item (e, tile) covers
// (empty when rb >= re): few-row experts take row tiles of tile_rows, many-row
// experts slices of whole matrix-core passes, N split over at most
// ntiles_big blocks.
template <int PHASE>
QMOE_D void item_rows(const FfnParams& P, int tile, bool big, int& rb, int& re) {
  const int N = PHASE == 0 ? P.F : P.H;
  const int pass = 16 * mfma_cols_per_pass(PHASE == 0 ? 2 : 1);
  const int cpt = ((N + P.ntiles_big - 1) / P.ntiles_big + pass - 1) / pass * pass;
  rb = big ? tile * cpt : tile * P.tile_rows;
  re = min(N, rb + (big ? cpt : P.tile_rows));
}

// One work item of the routed FFN: row tile `tile` of expert e, whose rows
// are positions pos0 .. pos0 + m - 1 of the permutation (perm_of(pos) gives
// the flat assignment t * k + i).  PHASE 0: gate/up + SwiGLU -> h;
// PHASE 1: down -> o.  COH: h is read past the L2 (written by other blocks
// of the same launch); COH_OUT: h and o are written through for readers in
// the same launch.
template <int PHASE, int RC, bool MFMA, bool COH, bool COH_OUT, class PermOf>
QMOE_D void ffn_item(const FfnParams& P, int e, int tile, bool big, int pos0, int m,
                     uint8_t* smem, PermOf perm_of) {
  const int H = P.H, F = P.F, kk = P.k, dtype = P.x_dtype, G = P.G;
  const int chunk = P.chunk > 0 && P.chunk < RC ? P.chunk : RC;
  const char* xb = (const char*)P.x;
  float* hbuf = P.h;
  float* obuf = P.o;
  qmoe_tier t;
  if (!tier_of(P.tiers, P.n_tiers, e, t)) return;
  const int fmt = PHASE == 0 ? t.fmt_gate_up : t.fmt_down;
  const int N = PHASE == 0 ? F : H, K = PHASE == 0 ? H : F;
  int rb, re;
  item_rows<PHASE>(P, tile, big, rb, re);
  if (rb >= re) return;
  const size_t xrow_bytes = (size_t)H * (dtype == QMOE_F32 ? 4 : 2);
  auto x_row = [=](int rr) {
    return (const void*)(xb + (size_t)(perm_of(pos0 + rr) / kk) * xrow_bytes);
  };
  auto h_out = [=](int n, int rr, const float* a) {
    float* dst = hbuf + (size_t)(pos0 + rr) * F + n;
    if constexpr (COH_OUT) store_coherent(dst, silu_mul(a[0], a[1]));
    else *dst = silu_mul(a[0], a[1]);
  };
  auto h_row = [=](int rr) { return (const void*)(hbuf + (size_t)(pos0 + rr) * F); };
  auto o_out = [=](int n, int rr, const float* a) {
    float* dst = obuf + (size_t)(pos0 + rr) * H + n;
    if constexpr (COH_OUT) store_coherent(dst, a[0]);
    else *dst = a[0];
  };
#define QMOE_FFN_CASE(FM)                                                                  \
  case FM: {                                                                               \
    const size_t eo = (size_t)(e - t.e_begin) * layout_of(FM, N, K).total;                  \
    if (PHASE == 0) {                                                                      \
      const Mat mats[2] = {mat_of((const uint8_t*)t.gate + eo, FM, N, K),                  \
                           mat_of((const uint8_t*)t.up + eo, FM, N, K)};                   \
      if (MFMA && big && dtype == QMOE_F32)                                                \
        mfma_cols<FM, 2, QMOE_F32>(mats, K, rb, re, m, smem, x_row, h_out);                \
      else if (MFMA && big)                                                                \
        mfma_cols<FM, 2, QMOE_BF16>(mats, K, rb, re, m, smem, x_row, h_out);               \
      else valu_rows<FM, 2, RC, false, true>(mats, K, rb, re, G, m, dtype, smem, x_row,     \
                                             h_out, chunk);                                \
    } else {                                                                               \
      const Mat mats[1] = {mat_of((const uint8_t*)t.down + eo, FM, N, K)};                 \
      if (MFMA && big)                                                                     \
        mfma_cols<FM, 1, COH ? kF32Coherent : QMOE_F32>(mats, K, rb, re, m, smem, h_row,   \
                                                        o_out);                            \
      else valu_rows<FM, 1, RC, COH, true>(mats, K, rb, re, G, m, QMOE_F32, smem, h_row,   \
                                           o_out, chunk);                                  \
    }                                                                                      \
  } break;
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

// ---------------------------------------- host-side launch choices ----
// Lanes per weight row: the largest power of two <= 64 dividing the unit
// count K/32 that still leaves every lane >= 4 units.
inline int lanes_per_row(int K) {
  const int units = K / 32;
  int G = 1;
  while (G < 64 && units % (2 * G) == 0 && units / (2 * G) >= 4) G *= 2;
  return G;
}

inline size_t stage_bytes(int RC, int K) {
  const int U = K / 32;
  return (size_t)RC * tok_stride(U) + (size_t)RC * U * sizeof(float2);
}

// LDS budget for staged activation rows in the routed FFN.  Registers bound
// the resident blocks of these kernels (2-3 per CU), so a block may stage up
// to 96 KB of the 160 KB a gfx950 compute unit holds (four rows of a
// 7168-wide hidden dimension take 68 KB).
constexpr size_t kFfnStageBudget = 96 << 10;

// Kernels that may take more than 64 KB of LDS declare it (host side).
template <class Kernel>
inline void allow_lds(Kernel kernel, size_t lds) {
  if (lds > (64u << 10))
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
}

// Rows per register pass: 1, 2 or 4 (enough for `rows`), halved until the
// staged rows fit `budget` bytes of LDS.  0 if even one row does not fit.
inline int pick_rc(int rows, int K, size_t budget = kLdsCap) {
  int rc = rows <= 1 ? 1 : rows <= 2 ? 2 : 4;
  while (rc > 1 && stage_bytes(rc, K) > budget) rc >>= 1;
  return stage_bytes(rc, K) <= (budget > (size_t)kLdsCap ? budget : (size_t)kLdsCap) ? rc : 0;
}

// Rows per block for N rows when `work_items` independent matrices run in
// the same launch: about per_cu blocks per compute unit overall, so that every
// CU keeps enough weight loads in flight to cover HBM latency.  A multiple of
// a wave pass and of the 16-row matrix-core blocks.
inline int pick_tile_rows(int N, int G, int work_items, int per_cu = 8) {
  int group = kWaves * (64 / G);
  if (group < 16) group = 16;
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const long long want = (long long)per_cu * cus;
  long long tiles = (want + work_items - 1) / work_items;
  const long long max_tiles = (N + group - 1) / group;
  if (tiles > max_tiles) tiles = max_tiles;
  if (tiles < 1) tiles = 1;
  const int rows = (int)((N + tiles - 1) / tiles);
  return (rows + group - 1) / group * group;
}

}  // namespace qmoe
