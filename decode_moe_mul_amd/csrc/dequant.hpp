// Internal header: operand types of the matrix-core tiles of the decode
// kernels (fp16 operands, fp32 accumulators).
#pragma once
#include "common.hpp"

namespace qmoe {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Two fp32 values rounded to fp16 (nearest even) and packed (lo, hi).
QMOE_D uint32_t pack_f16(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace qmoe
