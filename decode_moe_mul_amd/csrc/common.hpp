// Internal header of libqmoe: plane layout, number conversions, per-format
// decoding of 32-value units, launch/error/profiling helpers.
//
// The value formulas are those of the block formats named on the "RTX 3090
// Llama 70B three-tier cache" page (section 一) and the "Three RTX 3090
// Qwen3.8-Flash-Next guide" page (section 优化策略二); the plane layout is this
// library's own and is described in include/qmoe.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qmoe.h"

#define QMOE_HD __host__ __device__ __forceinline__
#define QMOE_D __device__ __forceinline__

namespace qmoe {

// ------------------------------------------------------------- layout ----
struct Layout {
  size_t off[4];
  size_t total;
  int nplanes;
};

QMOE_HD size_t round_up256(size_t n) { return (n + 255) & ~size_t(255); }

QMOE_HD int block_of(int fmt) {
  return (fmt == QMOE_Q4_K || fmt == QMOE_Q6_K) ? 256
         : (fmt >= QMOE_Q8_0 && fmt <= QMOE_MXFP4) ? 32
         : fmt == QMOE_T5                           ? 128
                                                  : 0;
}

// The formats of the routed-expert tiers (the ternary T5 is a dense-GEMV format).
QMOE_HD bool tier_format(int fmt) { return fmt >= QMOE_Q8_0 && fmt <= QMOE_Q6_K; }

// T5: 28-byte groups of 128 weights (26 base-3 code bytes, then fp16 d).
constexpr int kT5GroupBytes = 28;

// Plane sizes per format, in storage order, for a [N, K] tensor.
QMOE_HD Layout layout_of(int fmt, int N, int K) {
  Layout L{};
  const size_t n = (size_t)N, k = (size_t)K;
  size_t sz[4] = {0, 0, 0, 0};
  int np = 2;
  switch (fmt) {
    case QMOE_Q8_0: sz[0] = n * k; sz[1] = n * (k / 32) * 2; break;
    case QMOE_Q4_0: sz[0] = n * k / 2; sz[1] = n * (k / 32) * 2; break;
    case QMOE_MXFP4: sz[0] = n * k / 2; sz[1] = n * (k / 32); break;
    case QMOE_Q4_K: sz[0] = n * k / 2; sz[1] = n * (k / 256) * 16; break;
    case QMOE_Q6_K:
      sz[0] = n * k / 2; sz[1] = n * k / 4; sz[2] = n * (k / 256) * 16;
      sz[3] = n * (k / 256) * 2; np = 4; break;
    case QMOE_T5: sz[0] = n * (k / 128) * kT5GroupBytes; np = 1; break;
    default: np = 0;
  }
  size_t pos = 0;
  for (int i = 0; i < np; ++i) {
    L.off[i] = pos;
    pos = round_up256(pos + sz[i]);
  }
  L.total = pos;
  L.nplanes = np;
  return L;
}

// ------------------------------------------------------- conversions ----
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

QMOE_D float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
QMOE_D uint32_t f32_to_f16_bits(float v) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}
QMOE_D uint32_t pack_h2(float lo, float hi) {
  return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}
QMOE_D float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
QMOE_D uint32_t pk_add_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) + __builtin_bit_cast(h2_t, b));
}
QMOE_D uint32_t pk_mul_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b));
}
// sum over the pair: a.lo*b.lo + a.hi*b.hi + c, fp32 accumulate
QMOE_D float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}
// 2^(e-127) for an E8M0 byte; 255 is NaN; e = 0 is the fp32 subnormal 2^-127
// a * b + c with the 24-bit multiplier (a, b < 2^24; the result must fit in 32
// bits): one full-rate v_mad_u32_u24 instead of a 32- or 64-bit multiply.
QMOE_D uint32_t mad24(uint32_t a, uint32_t b, uint32_t c) { return __umul24(a, b) + c; }

// Weight bytes are read once per call: the nontemporal hint streams them
// past the caches instead of displacing lines that are reused.
QMOE_D uint4 load_stream(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load((const v4u*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

QMOE_D float e8m0_to_f32(uint32_t e) {
  uint32_t bits = e == 255u ? 0x7FC00000u : (e == 0u ? 0x00400000u : (e << 23));
  return __builtin_bit_cast(float, bits);
}

// Load an activation element (fp32 or raw bf16) as fp32.
QMOE_D float load_act(const void* x, int dtype, size_t i) {
  return dtype == QMOE_F32 ? ((const float*)x)[i]
                           : bf16_bits_to_f32(((const uint16_t*)x)[i]);
}

// --------------------------------------------------- unit decoding ------
// A "unit" is 32 consecutive values of one weight row.  Its codes are turned
// into 16 words of two fp16 each, holding exact small integers (or exact E2M1
// values), so that a unit's dot product with fp16 activations is 16
// v_dot2_f32_f16 followed by one multiply with the unit's scale.
//
// Pair order.  4-bit codes: word c of the 16 code bytes holds elements
// 8c..8c+7 as nibbles; pair 4c+j = elements (8c+j, 8c+j+4).  8-bit codes:
// word c holds elements 4c..4c+3; pair 2c+j = elements (4c+j, 4c+j+2).  The
// activations are staged in the same pair order ("nibble" / "byte" order).

constexpr uint32_t H2_MAGIC = 0x64006400u;  // fp16 1024 in both halves
constexpr uint32_t H2_NEG_1024 = 0xE400E400u;
constexpr uint32_t H2_NEG_1032 = 0xE408E408u;  // -(1024 + 8)
constexpr uint32_t H2_NEG_1056 = 0xE420E420u;  // -(1024 + 32)
constexpr uint32_t H2_NEG_1152 = 0xE480E480u;  // -(1024 + 128)
constexpr uint32_t H2_2P14 = 0x74007400u;      // 2^14

// nibble codes + fp16 bias  ->  exact (code - bias) in fp16 pairs
QMOE_D void nibbles_to_h2(const uint4 q, uint32_t neg_bias, uint32_t out[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[4 * c + j] = pk_add_h2(((w[c] >> (4 * j)) & 0x000F000Fu) | H2_MAGIC, neg_bias);
}

// E2M1 codes -> exact E2M1 values in fp16 pairs.  (m << 9) read as fp16 is
// E2M1(m) * 2^-14 for the 3-bit magnitude m (m = 1 lands on an fp16
// subnormal), so one multiply by 2^14 gives the value exactly.
QMOE_D void e2m1_to_h2(const uint4 q, uint32_t out[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[c] >> (4 * j);
      const uint32_t bits = ((v & 0x00070007u) << 9) | ((v & 0x00080008u) << 12);
      out[4 * c + j] = pk_mul_h2(bits, H2_2P14);
    }
}

// Q6_K: low nibbles + 2 high bits per element -> exact (q - 32)
QMOE_D void q6_to_h2(const uint4 ql, const uint2 qh, uint32_t out[16]) {
  const uint32_t w[4] = {ql.x, ql.y, ql.z, ql.w};
  const uint32_t hw[4] = {qh.x & 0xFFFFu, qh.x >> 16, qh.y & 0xFFFFu, qh.y >> 16};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // element i of the 8 has its high bits at 2i; spread so that elements j
    // and j+4 sit at bits 2j and 16+2j
    const uint32_t hh = (hw[c] & 0xFFu) | ((hw[c] & 0xFF00u) << 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (w[c] >> (4 * j)) & 0x000F000Fu;
      const uint32_t hi = ((hh >> (2 * j)) & 0x00030003u) << 4;
      out[4 * c + j] = pk_add_h2(lo | hi | H2_MAGIC, H2_NEG_1056);
    }
  }
}

// Q8_0: signed bytes -> exact q in fp16 pairs (byte order)
QMOE_D void bytes_to_h2(const uint4 a, const uint4 b, uint32_t out[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t u = w[c] ^ 0x80808080u;  // q + 128 as unsigned bytes
    out[2 * c] = pk_add_h2((u & 0x00FF00FFu) | H2_MAGIC, H2_NEG_1152);
    out[2 * c + 1] = pk_add_h2(((u >> 8) & 0x00FF00FFu) | H2_MAGIC, H2_NEG_1152);
  }
}

// ---- biased codes (dot-product path) ----------------------------------
// The same magic-number decode without the bias subtraction: the fp16 code
// words hold bias + code exactly, and the unit's dot product with the staged
// activations carries bias * (their sum), which the staging computes once per
// unit and the dot subtracts.  In the 4- and 6-bit formats the codes of odd
// pair index j are taken four bits up (fp16 1024 + 16 * code), which needs no
// shift; the activations of those pairs are staged divided by 16.

// Q4_0 / Q4_K nibbles: pair 4c+j = (1024 + e, 1024 + e') for even j and
// (1024 + 16e, 1024 + 16e') for odd j, e = element 8c+j, e' = element 8c+j+4.
// (x & mask) | bits in one instruction.  The compiler splits this pattern
// into an and plus an or when the operands are constants, so the operation
// is written out; mask comes in a scalar register, bits in a vector one.
// Only for values consumed by vector ALU instructions: the compiler does not
// see this write when it spaces vector writes from matrix-core reads.
QMOE_D uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
  return r;
}

QMOE_D void nibbles_biased(const uint4 q, uint32_t out[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t t = w[c] >> 8;
    out[4 * c + 0] = and_or(w[c], 0x000F000Fu, H2_MAGIC);
    out[4 * c + 1] = and_or(w[c], 0x00F000F0u, H2_MAGIC);
    out[4 * c + 2] = and_or(t, 0x000F000Fu, H2_MAGIC);
    out[4 * c + 3] = and_or(t, 0x00F000F0u, H2_MAGIC);
  }
}

// Q6_K: the unsigned 6-bit code (low nibble + 2 high bits) in the same
// positions: 1024 + q (even j) or 1024 + 16 q (odd j), q in [0, 63].
QMOE_D void q6_biased(const uint4 ql, const uint2 qh, uint32_t out[16]) {
  const uint32_t w[4] = {ql.x, ql.y, ql.z, ql.w};
  const uint32_t hw[4] = {qh.x & 0xFFFFu, qh.x >> 16, qh.y & 0xFFFFu, qh.y >> 16};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // high bits of elements 8c+j and 8c+j+4 at bits 2j and 16+2j
    const uint32_t hh = (hw[c] & 0xFFu) | ((hw[c] & 0xFF00u) << 8);
    const uint32_t t = w[c] >> 8;
    out[4 * c + 0] = and_or(hh << 4, 0x00300030u, and_or(w[c], 0x000F000Fu, H2_MAGIC));
    out[4 * c + 1] = and_or(hh << 6, 0x03000300u, and_or(w[c], 0x00F000F0u, H2_MAGIC));
    out[4 * c + 2] = and_or(hh, 0x00300030u, and_or(t, 0x000F000Fu, H2_MAGIC));
    out[4 * c + 3] = and_or(hh << 2, 0x03000300u, and_or(t, 0x00F000F0u, H2_MAGIC));
  }
}

// Q8_0 (byte order): 1152 + q for the signed byte q.
QMOE_D void bytes_biased(const uint4 a, const uint4 b, uint32_t out[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  // byte permute from {0x64646464 : u}: (byte 0, 0x64, byte 2, 0x64) and
  // (byte 1, 0x64, byte 3, 0x64), i.e. fp16 1024 + byte in both halves
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t u = w[c] ^ 0x80808080u;
    out[2 * c] = __builtin_amdgcn_perm(0x64646464u, u, 0x04020400u);
    out[2 * c + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030401u);
  }
}

// MXFP4 in natural pair order (elements 2p, 2p+1): the exact E2M1 values,
// one hardware conversion per byte (scale 1).
QMOE_D void e2m1_natural(const uint4 q, uint32_t out[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    out[4 * c + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], 1.f, 0));
    out[4 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], 1.f, 1));
    out[4 * c + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], 1.f, 2));
    out[4 * c + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], 1.f, 3));
  }
}

// Position, within a unit's 32 values, of element i of pair p (i = 0, 1).
QMOE_HD int pair_elem_nibble(int p, int i) { return 8 * (p >> 2) + (p & 3) + 4 * i; }
QMOE_HD int pair_elem_byte(int p, int i) { return 4 * (p >> 1) + (p & 1) + 2 * i; }
constexpr bool byte_order(int fmt) { return fmt == QMOE_Q8_0; }

// Pair order of the biased codes: element of member i of pair p, and whether
// the pair's codes sit four bits up (activations staged divided by 16).
template <int FMT>
QMOE_HD int pair_elem_biased(int p, int i) {
  if constexpr (FMT == QMOE_Q8_0) return pair_elem_byte(p, i);
  else if constexpr (FMT == QMOE_MXFP4) return 2 * p + i;
  else return pair_elem_nibble(p, i);
}
template <int FMT>
QMOE_HD bool pair_up4(int p) {
  return (FMT == QMOE_Q4_0 || FMT == QMOE_Q4_K || FMT == QMOE_Q6_K) && (p & 1);
}

// ------------------------------------ hand-over between blocks ------
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
QMOE_D void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
QMOE_D int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This thread's outstanding vector-memory operations have completed (its
// written-through stores are visible device-wide) before it goes on.
QMOE_D void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------- wave reductions ------
// Wave-wide max / min of unsigned values through DPP row shifts and row
// broadcasts (lanes whose source is out of range keep the identity); the
// result is read from lane 63 and is wave-uniform.
template <int CTRL, int ROW_MASK>
QMOE_D uint32_t dpp_u32(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xF, false);
}
QMOE_D uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF>(0u, v));  // row_shr:1
  v = max(v, dpp_u32<0x112, 0xF>(0u, v));  // row_shr:2
  v = max(v, dpp_u32<0x114, 0xF>(0u, v));  // row_shr:4
  v = max(v, dpp_u32<0x118, 0xF>(0u, v));  // row_shr:8
  v = max(v, dpp_u32<0x142, 0xA>(0u, v));  // row_bcast:15
  v = max(v, dpp_u32<0x143, 0xC>(0u, v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
QMOE_D uint32_t wave_min_u32(uint32_t v) {
  const uint32_t id = 0xFFFFFFFFu;
  v = min(v, dpp_u32<0x111, 0xF>(id, v));
  v = min(v, dpp_u32<0x112, 0xF>(id, v));
  v = min(v, dpp_u32<0x114, 0xF>(id, v));
  v = min(v, dpp_u32<0x118, 0xF>(id, v));
  v = min(v, dpp_u32<0x142, 0xA>(id, v));
  v = min(v, dpp_u32<0x143, 0xC>(id, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}


// Sum across aligned groups of G lanes (G a power of two <= 64).
template <int G>
QMOE_D float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace qmoe

// ----------------------------------------------- host-side helpers ------
// (implemented in api.hip)
namespace qmoe {
int fail(int status, const char* fmt, ...);   // records qmoe_last_error text
int check_launch(const char* kernel);         // hipGetLastError -> status
bool profiling_on();
void profile_begin(const char* kernel, hipStream_t s);
void profile_end(const char* kernel, hipStream_t s);
int cu_count();
}  // namespace qmoe

// Launch with optional event timing and error check; returns a qmoe status.
#define QMOE_LAUNCH(name, kernel, grid, block, lds, stream, ...)            \
  ([&]() -> int {                                                            \
    if (qmoe::profiling_on()) qmoe::profile_begin(name, stream);             \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);       \
    int st_ = qmoe::check_launch(name);                                      \
    if (qmoe::profiling_on()) qmoe::profile_end(name, stream);               \
    return st_;                                                              \
  }())

#define QMOE_ALIGNED(p, a) ((((uintptr_t)(p)) & ((a)-1)) == 0)
