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

// Block (bx, by): rows by * 128 .., columns bx * 128 ..; wave w computes
// the 64 x 64 quarter (w >> 1, w & 1): 4 row groups x 4 column blocks, 16
// matrix ops per K step of 128.  Each step's operand tiles (A: 128 rows x
// 128 bytes, B: 128 columns x 64 bytes, and their scale words) are loaded
// once per block with 16-byte coalesced loads into registers while the
// previous step is multiplied, then written to the other half of a
// double-buffered LDS tile.  16-byte chunk c of A row r sits at chunk
// c ^ (r & 7), chunk c of B column n at c ^ (n & 3), so the 16 rows (or
// columns) one operand read touches spread over the banks.  Rows and columns
// past the ends re-read the last one (never stored).
constexpr int kMxAB = kMxBM * 128, kMxBB = kMxBN * 64;  // operand bytes per step
constexpr size_t kMxLds = 2 * (kMxAB + kMxBB + 4 * (kMxBM + kMxBN));

__global__ __launch_bounds__(kMxBlock, 2) void mxfp4_gemm_kernel(MxParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int K = P.K, nbk = K >> 5, nsteps = K >> 7;
  const int br0 = blockIdx.y * kMxBM, bc0 = blockIdx.x * kMxBN;
  // LDS: [buf] A bytes, B bytes, A scale words, B scale words
  auto As = [&](int buf) { return smem + buf * (kMxAB + kMxBB + 4 * (kMxBM + kMxBN)); };
  auto Bs = [&](int buf) { return As(buf) + kMxAB; };
  auto Asc = [&](int buf) { return (uint32_t*)(Bs(buf) + kMxBB); };
  auto Bsc = [&](int buf) { return Asc(buf) + kMxBM; };
  // staging roles: A chunks tid + 256 j (j < 4): row >> 3, chunk & 7; B chunks
  // tid + 256 j (j < 2): column >> 2, chunk & 3; thread tid < 128 loads the
  // scale word of A row tid, the others that of B column tid - 128
  uint32_t arow_g[4], bcol_g[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) arow_g[j] = (uint32_t)min(br0 + ((tid + 256 * j) >> 3), P.R - 1);
#pragma unroll
  for (int j = 0; j < 2; ++j) bcol_g[j] = (uint32_t)min(bc0 + ((tid + 256 * j) >> 2), P.N - 1);
  const bool sc_a = tid < kMxBM;
  const uint32_t sc_row = (uint32_t)(sc_a ? min(br0 + tid, P.R - 1) : min(bc0 + tid - kMxBM, P.N - 1));
  // two steps of this thread's operand loads in flight, in sets X and Y
  // (named registers: an array here would be placed in scratch)
  struct Set { uint4 a0, a1, a2, a3, b0, b1; uint32_t s; };
  const uint8_t* sp = sc_a ? P.xs : P.ws;
  auto aptr = [&](int j, uint32_t k0) {
    return (const uint4*)(P.xq + arow_g[j] * (uint32_t)K + k0 + 16u * ((tid + 256 * j) & 7));
  };
  auto bptr = [&](int j, uint32_t k0) {
    return (const uint4*)(P.wq + bcol_g[j] * (uint32_t)(K >> 1) + (k0 >> 1) +
                          16u * ((tid + 256 * j) & 3));
  };
  auto gload = [&](int st, Set& v) {
    const uint32_t k0 = (uint32_t)st * 128u;
    v.a0 = *aptr(0, k0); v.a1 = *aptr(1, k0); v.a2 = *aptr(2, k0); v.a3 = *aptr(3, k0);
    v.b0 = *bptr(0, k0); v.b1 = *bptr(1, k0);
    v.s = *(const uint32_t*)(sp + sc_row * (uint32_t)nbk + 4u * st);
  };
  auto awrite = [&](int buf, int j, uint4 v) {
    const int c = tid + 256 * j, r = c >> 3, ch = c & 7;
    *(uint4*)(As(buf) + r * 128 + 16 * (ch ^ (r & 7))) = v;
  };
  auto bwrite = [&](int buf, int j, uint4 v) {
    const int c = tid + 256 * j, n = c >> 2, ch = c & 3;
    *(uint4*)(Bs(buf) + n * 64 + 16 * (ch ^ (n & 3))) = v;
  };
  auto lwrite = [&](int buf, const Set& v) {
    awrite(buf, 0, v.a0); awrite(buf, 1, v.a1); awrite(buf, 2, v.a2); awrite(buf, 3, v.a3);
    bwrite(buf, 0, v.b0); bwrite(buf, 1, v.b1);
    Asc(buf)[tid] = v.s;  // A scale words, then B's (tid - 128) right after
  };
  const int wr0 = (wave >> 1) * (16 * kMxMI), wc0 = (wave & 1) * (16 * kMxNB);
  mx_v4f acc[kMxMI][kMxNB];
#pragma unroll
  for (int i = 0; i < kMxMI; ++i)
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) acc[i][b] = mx_v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    uint4 bq[kMxNB];
    uint32_t bs[kMxNB];
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) {
      const int n = wc0 + 16 * b + li;
      bq[b] = *(const uint4*)(Bs(buf) + n * 64 + 16 * (g ^ (n & 3)));
      bs[b] = (Bsc(buf)[n] >> (8 * g)) & 0xFFu;
    }
#pragma unroll
    for (int i = 0; i < kMxMI; ++i) {
      const int r = wr0 + 16 * i + li;
      const uint4 lo = *(const uint4*)(As(buf) + r * 128 + 16 * (g ^ (r & 7)));
      const uint4 hi = *(const uint4*)(As(buf) + r * 128 + 16 * ((g + 4) ^ (r & 7)));
      const uint32_t as = (Asc(buf)[r] >> (8 * g)) & 0xFFu;
#pragma unroll
      for (int b = 0; b < kMxNB; ++b) acc[i][b] = mx_mma(lo, hi, as, bq[b], bs[b], acc[i][b]);
    }
  };
  // LDS buffer s & 1 holds step s; set X holds the next odd step, Y the
  // next even one.  Prefetches past the last step re-read it and fill a
  // buffer nobody reads any more, so the loop body has no branches.
  const int last = nsteps - 1;
  Set X, Y;
  gload(0, X);
  lwrite(0, X);
  __syncthreads();
  gload(min(1, last), X);
  gload(min(2, last), Y);
  int st = 0;
  for (; st + 2 <= nsteps; st += 2) {
    compute(0);
    lwrite(1, X);
    __syncthreads();
    gload(min(st + 3, last), X);
    compute(1);
    lwrite(0, Y);
    __syncthreads();
    gload(min(st + 4, last), Y);
  }
  if (st < nsteps) compute(0);  // odd step count: the last step is in buffer 0
  // lane holds rows 4 g + j of each row group, column li of each block
#pragma unroll
  for (int i = 0; i < kMxMI; ++i)
#pragma unroll
    for (int b = 0; b < kMxNB; ++b) {
      const int col = bc0 + wc0 + 16 * b + li;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = br0 + wr0 + 16 * i + 4 * g + j;
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
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(codes, 16) || !QMOE_ALIGNED(scales, 4))
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_mxfp4_mxfp8: misaligned W/codes/scales");
  const Layout L = layout_of(QMOE_MXFP4, N, K);
  MxParams P{(const uint8_t*)W + L.off[0], (const uint8_t*)W + L.off[1], codes, scales, y, N, K, R};
  const dim3 grid((unsigned)((N + kMxBN - 1) / kMxBN), (unsigned)((R + kMxBM - 1) / kMxBM));
  if (grid.y > 65535) return fail(QMOE_ERR_UNSUPPORTED, "qgemm_mxfp4_mxfp8: R=%d too large", R);
  return QMOE_LAUNCH("mxfp4_gemm", mxfp4_gemm_kernel, grid, kMxBlock, kMxLds, (hipStream_t)stream,
                     P);
}

}  // extern "C"
