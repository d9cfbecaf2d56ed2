// Internal header: dequantization of a 32-value unit of a weight row into
// bf16 or fp16 pairs for the matrix-core tiles (prefill and many-row decode).
#pragma once
#include "common.hpp"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// byte I of x as a float (selected into v_cvt_f32_ubyteI)
template <int I>
QMOE_D float ubyte(uint32_t x) { return (float)((x >> (8 * I)) & 0xFFu); }

QMOE_D uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
QMOE_D uint32_t pack_f16(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Operand element type of the matrix-core tiles: bf16 (prefill) or fp16
// (decode rows, whose activations are already fp16 in the dot-product path).
template <bool F16>
QMOE_D uint32_t pack2(float lo, float hi) { return F16 ? pack_f16(lo, hi) : pack_bf16(lo, hi); }

// Dequantize unit u (32 values) of weight row `row` of a [N, K] tensor into
// 16 words of bf16 (or fp16) pairs in natural element order (word w =
// elements 2w, 2w+1): the exact value computed in fp32, rounded once.  Units
// at or beyond K give zeros.
template <int FMT, bool F16>
QMOE_D void dequant_unit(const uint8_t* base, int N, int K, int row, int u, uint32_t out[16]) {
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
      out[2 * c] = pack2<F16>(fmaf(ubyte<0>(ww), d, bias),
                             fmaf(ubyte<1>(ww), d, bias));
      out[2 * c + 1] = pack2<F16>(fmaf(ubyte<2>(ww), d, bias),
                                 fmaf(ubyte<3>(ww), d, bias));
    }
  } else if constexpr (FMT == QMOE_MXFP4) {
    const uint4 q = *(const uint4*)(p0 + (size_t)row * (K >> 1) + 16 * (size_t)u);
    const float scale = e8m0_to_f32(p1[row * nb32 + u]);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (F16) {
        out[4 * c + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], scale, 0));
        out[4 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], scale, 1));
        out[4 * c + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], scale, 2));
        out[4 * c + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], scale, 3));
      } else {
        out[4 * c + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 0));
        out[4 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 1));
        out[4 * c + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 2));
        out[4 * c + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 3));
      }
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
      out[4 * c + 0] = pack2<F16>(fmaf(ubyte<0>(lo4), a, b),
                                 fmaf(ubyte<0>(hi4), a, b));
      out[4 * c + 1] = pack2<F16>(fmaf(ubyte<1>(lo4), a, b),
                                 fmaf(ubyte<1>(hi4), a, b));
      out[4 * c + 2] = pack2<F16>(fmaf(ubyte<2>(lo4), a, b),
                                 fmaf(ubyte<2>(hi4), a, b));
      out[4 * c + 3] = pack2<F16>(fmaf(ubyte<3>(lo4), a, b),
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
      out[4 * c + 0] = pack2<F16>(fmaf(ubyte<0>(ce), a, b),
                                 fmaf(ubyte<0>(co), a, b));
      out[4 * c + 1] = pack2<F16>(fmaf(ubyte<1>(ce), a, b),
                                 fmaf(ubyte<1>(co), a, b));
      out[4 * c + 2] = pack2<F16>(fmaf(ubyte<2>(ce), a, b),
                                 fmaf(ubyte<2>(co), a, b));
      out[4 * c + 3] = pack2<F16>(fmaf(ubyte<3>(ce), a, b),
                                 fmaf(ubyte<3>(co), a, b));
    }
  }
}

}  // namespace qmoe
