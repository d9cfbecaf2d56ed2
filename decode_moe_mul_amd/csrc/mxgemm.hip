// MXFP4 weights x MXFP8 activations on the gfx950 block-scaled matrix cores.
//
// The "RTX 4080 SUPER native Windows 27B: NInfer 80 SM port" page (its list of
// hardware limits) names 4-bit weight and activation matrix ops as a tensor
// core feature its GPU lacks, so its 4-bit tier dequantizes on chip.  CDNA4
// multiplies block-scaled FP8/FP6/FP4 operands directly, one E8M0 scale per
// 32 values along K (OCP Microscaling Formats v1.0), with the two operands in
// different element types.  Here the MXFP4 weights are used as stored (codes
// and scales straight from HBM, no dequantization) and the activations are
// quantized once to MXFP8 with E4M3 elements:
//  * qquantize_act_mxfp8: per 32 values along K, E = floor(log2 max|x|) - 8,
//    stored as E + 127 clamped to [0, 254] (0 for an all-zero block); each
//    element is |x| / 2^E rounded to the nearest E4M3 value, ties to even,
//    saturating at 448, with the sign of x;
//  * qgemm_mxfp4_mxfp8: y[r, n] = sum_k w[n, k] x_q[r, k], one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 16 x 16 output tile and 128 values
//    of K (fp32 accumulation).
//
// The operand layout of that instruction is described in mx.hpp.
#include "mx.hpp"

#pragma clang fp contract(off)

namespace qmoe {

constexpr int kMxWaves = 4;
constexpr int kMxBlock = 64 * kMxWaves;
constexpr int kMxMI = 4;  // 16-row groups per wave: 64 rows
constexpr int kMxNB = 4;  // 16-column blocks per wave: 64 columns
// the 4 waves as 2 x 2: a block computes 128 rows x 128 columns
constexpr int kMxBM = 2 * 16 * kMxMI, kMxBN = 2 * 16 * kMxNB;

// ------------------------------------------------ activation quantizer ----
__global__ __launch_bounds__(256) void quantize_act_mxfp8_kernel(const void* x, int x_dtype,
                                                                 int R, int K, uint8_t* codes,
                                                                 uint8_t* scales) {
  const int nbk = K >> 5;
  const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (long long)R * nbk) return;
  const long long at = blk * 32;
  float v[32];
  if (x_dtype == QMOE_F32) {
    const float4* p = (const float4*)((const float*)x + at);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = (const uint4*)((const uint16_t*)x + at);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = p[i];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
        v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
  }
  uint32_t out[8];
  scales[blk] = (uint8_t)mx_quantize32(v, out);
  uint4* dst = (uint4*)(codes + at);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// ----------------------------------------------------------- the GEMM ----
struct MxParams {
  const uint8_t* wq;  // codes plane [N][K/2]
  const uint8_t* ws;  // E8M0 plane [N][K/32]
  const uint8_t* xq;  // [R][K] E4M3
  const uint8_t* xs;  // [R][K/32] E8M0
  float* y;           // [R][N]
  int N, K, R;
};

struct MxA {  // one lane's A operand of one 16-row group and step
  uint4 lo, hi;
  uint32_t s;
};
struct MxB {  // one lane's B operand of one 16-column block and step
  uint4 q;
  uint32_t s;
};

// Block (bx, by): rows by * 128 .., columns bx * 128 ..; wave w takes the
// 64 x 64 quarter (w >> 1, w & 1): 4 row groups x 4 column blocks, 16 matrix
// ops per step against 4 + 4 operand loads.  Loads of step s + 1 are in
// flight while step s is multiplied.  Rows and columns past the ends re-read
// the last one (never stored), so every load is unconditional.
__global__ __launch_bounds__(kMxBlock) void mxfp4_gemm_kernel(MxParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int K = P.K, nbk = K >> 5, nsteps = K >> 7;
  const int r0 = blockIdx.y * kMxBM + (wave >> 1) * (16 * kMxMI);
  const int c0 = blockIdx.x * kMxBN + (wave & 1) * (16 * kMxNB);
  uint32_t arow[kMxMI], bcol[kMxNB];
#pragma unroll
  for (int i = 0; i < kMxMI; ++i) arow[i] = (uint32_t)min(r0 + 16 * i + li, P.R - 1);
#pragma unroll
  for (int b = 0; b < kMxNB; ++b) bcol[b] = (uint32_t)min(c0 + 16 * b + li, P.N - 1);
  auto load = [&](int s, MxA (&a)[kMxMI], MxB (&w)[kMxNB]) {
    const uint32_t k0 = (uint32_t)s * 128u, blk = (uint32_t)s * 4u + (uint32_t)g;
#pragma unroll
    for (int i = 0; i < kMxMI; ++i) {
      const uint8_t* row = P.xq + arow[i] * (uint32_t)K + k0;
      a[i].lo = *(const uint4*)(row + 16u * g);
      a[i].hi = *(const uint4*)(row + 64u + 16u * g);
      a[i].s = P.xs[arow[i] * (uint32_t)nbk + blk];
    }
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) {
      w[b].q = *(const uint4*)(P.wq + bcol[b] * (uint32_t)(K >> 1) + 16u * blk);
      w[b].s = P.ws[bcol[b] * (uint32_t)nbk + blk];
    }
  };
  mx_v4f acc[kMxMI][kMxNB];
#pragma unroll
  for (int i = 0; i < kMxMI; ++i)
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) acc[i][b] = mx_v4f{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const MxA (&a)[kMxMI], const MxB (&w)[kMxNB]) {
#pragma unroll
    for (int i = 0; i < kMxMI; ++i)
#pragma unroll
      for (int b = 0; b < kMxNB; ++b)
        acc[i][b] = mx_mma(a[i].lo, a[i].hi, a[i].s, w[b].q, w[b].s, acc[i][b]);
  };
  MxA a0[kMxMI], a1[kMxMI];
  MxB w0[kMxNB], w1[kMxNB];
  const int last = nsteps - 1;
  load(0, a0, w0);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    load(s + 1, a1, w1);
    mma(a0, w0);
    load(min(s + 2, last), a0, w0);
    mma(a1, w1);
  }
  if (s < nsteps) mma(a0, w0);
  // lane holds rows 4 g + j of each row group, column li of each block
#pragma unroll
  for (int i = 0; i < kMxMI; ++i)
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) {
      const int col = c0 + 16 * b + li;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = r0 + 16 * i + 4 * g + j;
        if (row < P.R && col < P.N) P.y[(size_t)row * P.N + col] = acc[i][b][j];
      }
    }
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qquantize_act_mxfp8(const void* x, int x_dtype, int R, int K, uint8_t* codes,
                        uint8_t* scales, void* stream) {
  if (R < 0 || K <= 0 || K % 32)
    return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_mxfp8: R=%d K=%d (K %% 32 != 0)", R, K);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "qquantize_act_mxfp8: unknown x_dtype %d", x_dtype);
  if (R == 0) return QMOE_OK;
  if (!x || !codes || !scales) return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_mxfp8: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(codes, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_mxfp8: misaligned x/codes");
  const long long blocks = (long long)R * (K / 32);
  const dim3 grid((unsigned)((blocks + 255) / 256));
  return QMOE_LAUNCH("quantize_act_mxfp8", quantize_act_mxfp8_kernel, grid, 256, 0,
                     (hipStream_t)stream, x, x_dtype, R, K, codes, scales);
}

int qgemm_mxfp4_mxfp8(const void* W, int N, int K, const uint8_t* codes, const uint8_t* scales,
                      int R, float* y, void* stream) {
  if (N < 0 || R < 0 || K <= 0 || K % 128)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_mxfp4_mxfp8: N=%d R=%d K=%d (K %% 128 != 0)", N,
                R, K);
  if ((long long)N * K >= (1LL << 32) || (long long)R * K >= (1LL << 32))
    return fail(QMOE_ERR_UNSUPPORTED, "qgemm_mxfp4_mxfp8: offsets beyond 32 bits");
  if (N == 0 || R == 0) return QMOE_OK;
  if (!W || !codes || !scales || !y)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_mxfp4_mxfp8: null pointer");
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(codes, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_mxfp4_mxfp8: misaligned W/codes");
  const Layout L = layout_of(QMOE_MXFP4, N, K);
  MxParams P{(const uint8_t*)W + L.off[0], (const uint8_t*)W + L.off[1], codes, scales, y, N, K, R};
  const dim3 grid((unsigned)((N + kMxBN - 1) / kMxBN), (unsigned)((R + kMxBM - 1) / kMxBM));
  if (grid.y > 65535) return fail(QMOE_ERR_UNSUPPORTED, "qgemm_mxfp4_mxfp8: R=%d too large", R);
  return QMOE_LAUNCH("mxfp4_gemm", mxfp4_gemm_kernel, grid, kMxBlock, 0, (hipStream_t)stream, P);
}

}  // extern "C"
