// Block-format quantizers and the reference dequantizers, on the device.
//
// qquantize_<fmt> packs fp32 weights into the plane layout (the offline
// per-tier packing of [P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section
// 优化策略二, done on the GPU so large expert banks pack in milliseconds).
// The rules are stated in include/qmoe.h; every decision (scale rounding,
// code rounding and clamping) is made in float64 with contraction disabled,
// so the bytes are a pure function of the fp32 inputs.
//
// qdequant_<fmt> writes each value as its exact format value rounded to
// nearest-even fp32: one correctly rounded operation per value.
#include "common.hpp"

#pragma clang fp contract(off)

namespace qmoe {

// float64 -> fp16 bits, round to nearest even, subnormals kept, overflow to
// infinity.
QMOE_D uint32_t f64_to_f16_rne(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull) return sign | (mag > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u);
  const int e = (int)(mag >> 52) - 1023;
  if (e > 15) return sign | 0x7C00u;
  if (e < -25) return sign;
  const uint64_t m = (mag & ((1ull << 52) - 1)) | (1ull << 52);
  const int shift = e >= -14 ? 42 : 28 - e;  // keep 11 bits (normal) or down to 2^-24
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    uint32_t ex = (uint32_t)(e + 15);
    if (q == 2048) { q = 1024; ++ex; }
    if (ex >= 31) return sign | 0x7C00u;
    return sign | (ex << 10) | (uint32_t)(q - 1024);
  }
  return sign | (uint32_t)q;  // subnormal (q == 1024 is the smallest normal)
}

QMOE_D double f16_bits_to_f64(uint32_t h) { return (double)f16_bits_to_f32(h); }

QMOE_D double round_half_away(double v) {
  const double t = trunc(v);
  const double f = fabs(v - t);
  return f >= 0.5 ? t + (v > 0 ? 1.0 : (v < 0 ? -1.0 : 0.0)) : t;
}
QMOE_D double safe_div(double num, double den) { return den != 0.0 ? num / den : 0.0; }
QMOE_D double clampd(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

// E2M1 magnitude code of m >= 0: nearest, ties to the even code, saturating.
QMOE_D uint32_t e2m1_code(double m) {
  if (m <= 0.25) return 0;
  if (m < 0.75) return 1;
  if (m <= 1.25) return 2;
  if (m < 1.75) return 3;
  if (m <= 2.5) return 4;
  if (m < 3.5) return 5;
  if (m <= 5.0) return 6;
  return 7;
}

// T5: one thread per 128-group.  d = fp16(mean |w|) (the float64 sum of the
// group's |w| divided by 128), t = clamp(round(w / d), -1, 1) against the
// stored d; code byte b = sum over r < 5 of (t + 1) * 3^r for weights 5b + r
// (t = 0 past weight 127); bytes 26, 27 = d.
__global__ __launch_bounds__(256) void quantize_t5_kernel(const float* w, int N, int K,
                                                          uint8_t* out) {
  const int nb = K / 128;
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (size_t)N * nb) return;
  const size_t n = blk / nb, b = blk - n * nb;
  const float* src = w + n * K + b * 128;
  double sum = 0.0;
  for (int i = 0; i < 128; ++i) sum += fabs((double)src[i]);
  const uint32_t d16 = f64_to_f16_rne(sum / 128.0);
  const double d = f16_bits_to_f64(d16);
  uint8_t* g = out + blk * kT5GroupBytes;
  for (int j = 0; j < 26; ++j) {
    uint32_t code = 0, pw = 1;
    for (int r = 0; r < 5; ++r) {
      const int i = 5 * j + r;
      const int t = i < 128 ? (int)clampd(round_half_away(safe_div((double)src[i], d)), -1, 1) : 0;
      code += (uint32_t)(t + 1) * pw;
      pw *= 3;
    }
    g[j] = (uint8_t)code;
  }
  g[26] = (uint8_t)d16;
  g[27] = (uint8_t)(d16 >> 8);
}

// T5 reference decoder: one thread per 32 values (d * t is exact in fp32).
__global__ __launch_bounds__(256) void dequant_t5_kernel(const uint8_t* W, int N, int K,
                                                         float* out) {
  const int U = K / 32;
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (size_t)N * U) return;
  const size_t n = id / U, u = id - n * U;
  const uint8_t* g = W + (n * (K / 128) + u / 4) * kT5GroupBytes;
  const float d = f16_bits_to_f32(g[26] | (g[27] << 8));
  float v[32];
  for (int i = 0; i < 32; ++i) {
    const int e = 32 * (int)(u & 3) + i;  // weight index within the group
    int c = g[e / 5];
    for (int r = 0; r < e % 5; ++r) c /= 3;
    v[i] = d * (float)(c % 3 - 1);
  }
  float4* dst = (float4*)(out + n * K + 32 * u);
  for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// One thread per block of B values.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* w, int N, int K, uint8_t* out) {
  constexpr int B = FMT == QMOE_Q4_K || FMT == QMOE_Q6_K ? 256 : 32;
  const int nb = K / B;
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (size_t)N * nb) return;
  const size_t n = blk / nb, b = blk - n * nb;
  const float* src = w + n * K + b * B;
  const Layout L = layout_of(FMT, N, K);
  uint8_t* p0 = out + L.off[0];
  uint8_t* p1 = out + L.off[1];
  if constexpr (FMT == QMOE_Q8_0 || FMT == QMOE_Q4_0) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)src[i]));
    const uint32_t d16 = f64_to_f16_rne(amax / (FMT == QMOE_Q8_0 ? 127.0 : 7.0));
    const double d = f16_bits_to_f64(d16);
    ((uint16_t*)p1)[blk] = (uint16_t)d16;
    if constexpr (FMT == QMOE_Q8_0) {
      int8_t* q = (int8_t*)p0 + n * K + b * 32;
      for (int i = 0; i < 32; ++i)
        q[i] = (int8_t)clampd(round_half_away(safe_div((double)src[i], d)), -127.0, 127.0);
    } else {
      uint8_t* q = p0 + n * (K / 2) + b * 16;
      for (int i = 0; i < 16; ++i) {
        const int lo = (int)clampd(round_half_away(safe_div((double)src[2 * i], d)) + 8, 0, 15);
        const int hi = (int)clampd(round_half_away(safe_div((double)src[2 * i + 1], d)) + 8, 0, 15);
        q[i] = (uint8_t)(lo | (hi << 4));
      }
    }
  } else if constexpr (FMT == QMOE_MXFP4) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)src[i]));
    int e = 0;
    if (amax > 0) {
      int ex;
      frexp(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
      e = 127 + (ex - 1) - 2;
      e = e < 0 ? 0 : (e > 254 ? 254 : e);
    }
    const double scale = ldexp(1.0, e - 127);
    p1[blk] = (uint8_t)e;
    uint8_t* q = p0 + n * (K / 2) + b * 16;
    for (int i = 0; i < 16; ++i) {
      uint32_t c[2];
      for (int h = 0; h < 2; ++h) {
        const double v = (double)src[2 * i + h];
        c[h] = e2m1_code(fabs(v) / scale) | (v < 0 ? 8u : 0u);
      }
      q[i] = (uint8_t)(c[0] | (c[1] << 4));
    }
  } else if constexpr (FMT == QMOE_Q4_K) {
    double s[8], mp[8], smax = 0.0, mmax = 0.0;
    for (int j = 0; j < 8; ++j) {
      double lo = (double)src[32 * j], hi = lo;
      for (int i = 1; i < 32; ++i) {
        const double v = (double)src[32 * j + i];
        lo = fmin(lo, v);
        hi = fmax(hi, v);
      }
      lo = fmin(0.0, lo);
      s[j] = (hi - lo) / 15.0;
      mp[j] = 0.0 - lo;  // +0 for an all-zero sub-block
      smax = fmax(smax, s[j]);
      mmax = fmax(mmax, mp[j]);
    }
    const uint32_t d16 = f64_to_f16_rne(smax / 63.0), m16 = f64_to_f16_rne(mmax / 63.0);
    const double d = f16_bits_to_f64(d16), dmin = f16_bits_to_f64(m16);
    uint64_t field_lo = 0, field_hi = 0;  // 96-bit field as bits 0..63 and 64..95
    uint8_t* q = p0 + n * (K / 2) + b * 128;
    for (int j = 0; j < 8; ++j) {
      const uint32_t sc = (uint32_t)clampd(round_half_away(safe_div(s[j], d)), 0, 63);
      const uint32_t mm = (uint32_t)clampd(round_half_away(safe_div(mp[j], dmin)), 0, 63);
      field_lo |= (uint64_t)sc << (6 * j);
      const int pos = 48 + 6 * j;  // m_j at bits pos .. pos+5 of the field
      if (pos + 6 <= 64) field_lo |= (uint64_t)mm << pos;
      else if (pos >= 64) field_hi |= (uint64_t)mm << (pos - 64);
      else { field_lo |= (uint64_t)mm << pos; field_hi |= (uint64_t)mm >> (64 - pos); }
      const double den = d * (double)sc, off = dmin * (double)mm;
      for (int i = 0; i < 16; ++i) {
        const double v0 = (double)src[32 * j + 2 * i] + off;
        const double v1 = (double)src[32 * j + 2 * i + 1] + off;
        const int c0 = (int)clampd(round_half_away(safe_div(v0, den)), 0, 15);
        const int c1 = (int)clampd(round_half_away(safe_div(v1, den)), 0, 15);
        q[16 * j + i] = (uint8_t)(c0 | (c1 << 4));
      }
    }
    uint8_t* meta = p1 + blk * 16;
    meta[0] = (uint8_t)d16; meta[1] = (uint8_t)(d16 >> 8);
    meta[2] = (uint8_t)m16; meta[3] = (uint8_t)(m16 >> 8);
    for (int i = 0; i < 8; ++i) meta[4 + i] = (uint8_t)(field_lo >> (8 * i));
    for (int i = 0; i < 4; ++i) meta[12 + i] = (uint8_t)(field_hi >> (8 * i));
  } else {  // Q6_K
    uint8_t* p2 = out + L.off[2];
    uint8_t* p3 = out + L.off[3];
    double s[16], smax = 0.0;
    for (int j = 0; j < 16; ++j) {
      double a = 0.0;
      for (int i = 0; i < 16; ++i) a = fmax(a, fabs((double)src[16 * j + i]));
      s[j] = a / 31.0;
      smax = fmax(smax, s[j]);
    }
    const uint32_t d16 = f64_to_f16_rne(smax / 127.0);
    const double d = f16_bits_to_f64(d16);
    ((uint16_t*)p3)[blk] = (uint16_t)d16;
    uint8_t* ql = p0 + n * (K / 2) + b * 128;
    uint8_t* qh = p1 + n * (K / 4) + b * 64;
    for (int j = 0; j < 16; ++j) {
      const int sc = (int)clampd(round_half_away(safe_div(s[j], d)), -128, 127);
      p2[blk * 16 + j] = (uint8_t)(int8_t)sc;
      const double den = d * (double)sc;
      int c[16];
      for (int i = 0; i < 16; ++i)
        c[i] = (int)clampd(round_half_away(safe_div((double)src[16 * j + i], den)) + 32, 0, 63);
      for (int i = 0; i < 8; ++i) ql[8 * j + i] = (uint8_t)((c[2 * i] & 15) | ((c[2 * i + 1] & 15) << 4));
      for (int i = 0; i < 4; ++i)
        qh[4 * j + i] = (uint8_t)((c[4 * i] >> 4) | ((c[4 * i + 1] >> 4) << 2) |
                                  ((c[4 * i + 2] >> 4) << 4) | ((c[4 * i + 3] >> 4) << 6));
    }
  }
}

// One thread per 32-value unit.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* W, int N, int K, float* out) {
  const int U = K / 32;
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (size_t)N * U) return;
  const size_t n = id / U, u = id - n * U;
  const Layout L = layout_of(FMT, N, K);
  const uint8_t* p0 = W + L.off[0];
  const uint8_t* p1 = W + L.off[1];
  float v[32];
  if constexpr (FMT == QMOE_Q8_0) {
    const float d = f16_bits_to_f32(((const uint16_t*)p1)[id]);
    const int8_t* q = (const int8_t*)p0 + n * K + 32 * u;
    for (int i = 0; i < 32; ++i) v[i] = d * (float)q[i];
  } else if constexpr (FMT == QMOE_Q4_0 || FMT == QMOE_MXFP4 || FMT == QMOE_Q4_K) {
    const uint8_t* q = p0 + n * (K / 2) + 16 * u;
    int c[32];
    for (int i = 0; i < 16; ++i) { c[2 * i] = q[i] & 15; c[2 * i + 1] = q[i] >> 4; }
    if constexpr (FMT == QMOE_Q4_0) {
      const float d = f16_bits_to_f32(((const uint16_t*)p1)[id]);
      for (int i = 0; i < 32; ++i) v[i] = d * (float)(c[i] - 8);
    } else if constexpr (FMT == QMOE_MXFP4) {
      const float scale = e8m0_to_f32(p1[id]);
      const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
      for (int i = 0; i < 32; ++i) {
        const float m = mag[c[i] & 7] * scale;
        v[i] = (c[i] & 8) ? -m : m;
      }
    } else {
      const uint8_t* meta = p1 + (n * (K / 256) + u / 8) * 16;
      const int j = (int)(u & 7);
      uint64_t lo = 0, hi = 0;
      for (int i = 0; i < 8; ++i) lo |= (uint64_t)meta[4 + i] << (8 * i);
      for (int i = 0; i < 8; ++i) hi |= (uint64_t)meta[8 + i] << (8 * i);
      const float sc = (float)((lo >> (6 * j)) & 63), mn = (float)((hi >> (16 + 6 * j)) & 63);
      const float a = f16_bits_to_f32(meta[0] | (meta[1] << 8)) * sc;       // exact
      const float m = f16_bits_to_f32(meta[2] | (meta[3] << 8)) * mn;       // exact
      for (int i = 0; i < 32; ++i) v[i] = fmaf(a, (float)c[i], -m);         // one rounding
    }
  } else {  // Q6_K
    const uint8_t* ql = p0 + n * (K / 2) + 16 * u;
    const uint8_t* qh = p1 + n * (K / 4) + 8 * u;
    const size_t sb = n * (K / 256) + u / 8;
    const int8_t* sc = (const int8_t*)(W + L.off[2]) + sb * 16 + 2 * (u & 7);
    const float d = f16_bits_to_f32(((const uint16_t*)(W + L.off[3]))[sb]);
    for (int i = 0; i < 32; ++i) {
      const int lo = (ql[i >> 1] >> (4 * (i & 1))) & 15;
      const int h2 = (qh[i >> 2] >> (2 * (i & 3))) & 3;
      const float a = d * (float)sc[i >> 4];                                // exact
      v[i] = a * (float)((lo | (h2 << 4)) - 32);                            // one rounding
    }
  }
  float4* dst = (float4*)(out + n * K + 32 * u);
  for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

static int check_tensor(const char* what, int fmt, const void* a, const void* b, int N, int K) {
  if (!a || !b) return fail(QMOE_ERR_INVALID_ARG, "%s: null pointer", what);
  if (N < 0 || K <= 0 || K % block_of(fmt) || K > 65536)
    return fail(QMOE_ERR_INVALID_ARG, "%s: bad sizes N=%d K=%d", what, N, K);
  return QMOE_OK;
}

template <int FMT>
static int quantize_launch(const float* w, int N, int K, void* out, void* stream) {
  int st = check_tensor("qquantize", FMT, w, out, N, K);
  if (st) return st;
  if (!QMOE_ALIGNED(out, 256)) return fail(QMOE_ERR_INVALID_ARG, "qquantize: misaligned out");
  if (N == 0) return QMOE_OK;
  const size_t nblk = (size_t)N * (K / block_of(FMT));
  if constexpr (FMT == QMOE_T5)
    return QMOE_LAUNCH("quantize", quantize_t5_kernel, dim3((unsigned)((nblk + 255) / 256)), 256,
                       0, (hipStream_t)stream, w, N, K, (uint8_t*)out);
  else
    return QMOE_LAUNCH("quantize", quantize_kernel<FMT>, dim3((unsigned)((nblk + 255) / 256)),
                       256, 0, (hipStream_t)stream, w, N, K, (uint8_t*)out);
}

template <int FMT>
static int dequant_launch(const void* W, int N, int K, float* out, void* stream) {
  int st = check_tensor("qdequant", FMT, W, out, N, K);
  if (st) return st;
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(out, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qdequant: misaligned pointer");
  if (N == 0) return QMOE_OK;
  const size_t nu = (size_t)N * (K / 32);
  if constexpr (FMT == QMOE_T5)
    return QMOE_LAUNCH("dequant", dequant_t5_kernel, dim3((unsigned)((nu + 255) / 256)), 256, 0,
                       (hipStream_t)stream, (const uint8_t*)W, N, K, out);
  else
    return QMOE_LAUNCH("dequant", dequant_kernel<FMT>, dim3((unsigned)((nu + 255) / 256)), 256,
                       0, (hipStream_t)stream, (const uint8_t*)W, N, K, out);
}

}  // namespace qmoe

using namespace qmoe;

#define QMOE_DEFINE_FORMAT(F, ID)                                                 \
  extern "C" int qquantize_##F(const float* w, int N, int K, void* out, void* s) { \
    return quantize_launch<ID>(w, N, K, out, s);                                  \
  }                                                                               \
  extern "C" int qdequant_##F(const void* W, int N, int K, float* out, void* s) {  \
    return dequant_launch<ID>(W, N, K, out, s);                                   \
  }
QMOE_DEFINE_FORMAT(q8_0, QMOE_Q8_0)
QMOE_DEFINE_FORMAT(q4_0, QMOE_Q4_0)
QMOE_DEFINE_FORMAT(mxfp4, QMOE_MXFP4)
QMOE_DEFINE_FORMAT(q4_k, QMOE_Q4_K)
QMOE_DEFINE_FORMAT(q6_k, QMOE_Q6_K)
QMOE_DEFINE_FORMAT(t5, QMOE_T5)
