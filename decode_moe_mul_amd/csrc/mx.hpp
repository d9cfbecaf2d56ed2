// Internal header: MXFP8 (E4M3 elements, E8M0 scale per 32 values)
// quantization and the block-scaled matrix-core op, shared by the MX GEMM and
// the MX path of the prefill.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on the device
// with a one-wave probe against a CPU model): lane l = 16 g + i supplies
//  * B (FP4, 4 registers): column i, K values 32 g .. 32 g + 31 in nibble
//    order (low nibble first): unit g of the step in weight row i;
//  * A (FP8, 8 registers): row i, K values 16 g .. 16 g + 15 (bytes 0..15)
//    and 64 + 16 g .. 64 + 16 g + 15 (bytes 16..31);
//  * scale bytes (byte 0 of a register): the scale of K block g (values
//    32 g .. 32 g + 31) of its row (A) or column (B), whichever lanes hold
//    that block's data;
//  * result: rows 4 g .. 4 g + 3 of column i.
#pragma once
#include "common.hpp"

namespace qmoe {

typedef int mx_v8i __attribute__((ext_vector_type(8)));
typedef float mx_v4f __attribute__((ext_vector_type(4)));

// |x| / 2^E (in [0, 512)) to the nearest E4M3 magnitude code, ties to even,
// saturating at 448 (code 0x7E).  Exact: the subnormal range is an integer
// multiple of 2^-9, the normal range keeps 3 of the 23 mantissa bits.
QMOE_D uint32_t e4m3_code_of(float m) {
  if (!(m < 448.f)) return 0x7Eu;
  if (m < 0.015625f) return (uint32_t)__builtin_rintf(m * 512.f);  // 2^-6: subnormals
  const uint32_t b = __builtin_bit_cast(uint32_t, m);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);  // round 23 -> 3 mantissa bits
  const uint32_t code = ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// One 32-value block: E = floor(log2 max|v|) - 8 as the E8M0 byte (clamped to
// [0, 254], 0 for an all-zero block) and the 32 E4M3 codes, 4 per word.
QMOE_D uint32_t mx_quantize32(const float (&v)[32], uint32_t (&out)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
    e = min(max(127 + (ex - 1) - 8, 0), 254);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xv = v[4 * i + j];
      uint32_t c = e4m3_code_of(ldexpf(fabsf(xv), 127 - e));
      if (xv < 0.f) c |= 0x80u;
      word |= c << (8 * j);
    }
    out[i] = word;
  }
  return (uint32_t)e;
}

// acc += A (FP8 E4M3, scale sa) x B (FP4 E2M1 codes q, scale sb), K = 128
QMOE_D mx_v4f mx_mma(uint4 alo, uint4 ahi, uint32_t sa, uint4 q, uint32_t sb, mx_v4f acc) {
  const mx_v8i av = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                     (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  const mx_v8i bv = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0 /* A: FP8 E4M3 */,
                                                          4 /* B: FP4 E2M1 */, 0, (int)sa, 0,
                                                          (int)sb);
}

}  // namespace qmoe
