// Q8_0 weights x int8 activations on the int8 matrix cores, for prefill-sized
// row counts ([P1] "NInfer 80 SM port": its int8 artifact runs prefill on the
// int8 tensor cores, with the activations quantized to int8 so that both GEMM
// operands are integers; section 九 items 2-3).
//
// The activations come from qquantize_act_q8 (per 32 values along K: fp32
// scale d = max|x| / 127, codes round-half-away(x / d) in [-127, 127]); the
// weights are used as stored (Q8_0: int8 codes, one fp16 scale per 32).  A
// 32-value block of one activation row against one weight row is then an
// exact integer dot product, so
//   y[r, n] = sum_b (d_x[r, b] * d_w[n, b]) * isum_b[r, n]
// with isum_b from one v_mfma_i32_16x16x32_i8 per 16 x 16 output tile and
// block b (exact int32), and the scaling and the sum over b in fp32.
//
// Block: 128 rows x 128 columns, 4 waves as 2 x 2 quarters of 64 x 64 (4 row
// groups x 4 column blocks of 16 x 16).  K advances 64 values (two blocks)
// per step; each step's operand tiles (A: 128 rows x 64 code bytes and their
// two fp32 scales, B: 128 weight rows x 64 code bytes and two fp16 scales)
// are loaded once per block with 16-byte loads one step ahead in registers
// and written to a double-buffered LDS tile with 80-byte rows (64 + 16 of
// padding: the 16 rows one operand read touches fall on distinct banks).
#include "dequant.hpp"

#pragma clang fp contract(off)

namespace qmoe {

constexpr int kI8Waves = 4;
constexpr int kI8GBlock = 64 * kI8Waves;
constexpr int kI8MI = 4, kI8NB = 4;               // 16-row groups, 16-column blocks per wave
constexpr int kI8BM = 2 * 16 * kI8MI, kI8BN = 2 * 16 * kI8NB;  // 128 x 128 per block
constexpr int kI8Row = 80;                         // LDS bytes per operand row
constexpr int kI8Tile = 128 * kI8Row;              // one operand tile
// [A codes][B codes][A scales: 2 x 128 fp32][B scales: 2 x 128 fp32]
constexpr int kI8Buf = 2 * kI8Tile + 2 * 128 * 2 * 4;
constexpr size_t kI8Lds = 2 * (size_t)kI8Buf;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct I8GemmParams {
  const int8_t* wq;    // [N][K] codes
  const uint16_t* wd;  // [N][K/32] fp16 scales
  const int8_t* xq;    // [R][K] codes
  const float* xd;     // [R][K/32] fp32 scales
  float* y;            // [R][N]
  int N, K, R;
};

__global__ __launch_bounds__(kI8GBlock, 2) void q8_0_i8_gemm_kernel(I8GemmParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int K = P.K, nbk = K >> 5, nsteps = (nbk + 1) >> 1;
  const int br0 = blockIdx.y * kI8BM, bc0 = blockIdx.x * kI8BN;
  auto Ab = [&](int buf) { return smem + buf * kI8Buf; };
  auto Bb = [&](int buf) { return Ab(buf) + kI8Tile; };
  auto Asc = [&](int buf) { return (float*)(Ab(buf) + 2 * kI8Tile); };
  auto Bsc = [&](int buf) { return Asc(buf) + 256; };
  // staging roles: code chunks c = tid + 256 j (j < 2) of A and of B: row
  // c >> 2, 16-byte chunk c & 3; thread tid < 128 loads A row tid's two
  // scales, the others B row tid - 128's
  uint32_t arow[2], brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    arow[j] = (uint32_t)min(br0 + ((tid + 256 * j) >> 2), P.R - 1);
    brow[j] = (uint32_t)min(bc0 + ((tid + 256 * j) >> 2), P.N - 1);
  }
  const bool sc_a = tid < 128;
  const uint32_t sc_row = (uint32_t)(sc_a ? min(br0 + tid, P.R - 1) : min(bc0 + tid - 128, P.N - 1));
  struct Set { uint4 a0, a1, b0, b1; float s0, s1; };
  // step st covers blocks 2 st and 2 st + 1; a block past the last (odd
  // block count) re-reads the last one and gets scale 0
  auto gload = [&](int st, Set& v) {
    const int b0 = 2 * st, b1 = min(2 * st + 1, nbk - 1);
    const uint32_t k0 = (uint32_t)b0 * 32u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ch = 16u * (uint32_t)((tid + 256 * j) & 3);
      // chunks 2, 3 belong to the second block; past the last block they
      // re-read its bytes (their products are scaled by 0)
      const uint32_t kk = ch < 32u ? k0 + ch : (uint32_t)b1 * 32u + ch - 32u;
      const uint4 a = *(const uint4*)(P.xq + arow[j] * (uint32_t)K + kk);
      const uint4 b = *(const uint4*)(P.wq + brow[j] * (uint32_t)K + kk);
      if (j == 0) { v.a0 = a; v.b0 = b; } else { v.a1 = a; v.b1 = b; }
    }
    if (sc_a) {
      v.s0 = P.xd[sc_row * (uint32_t)nbk + b0];
      v.s1 = 2 * st + 1 < nbk ? P.xd[sc_row * (uint32_t)nbk + b1] : 0.f;
    } else {
      v.s0 = f16_bits_to_f32(P.wd[sc_row * (uint32_t)nbk + b0]);
      v.s1 = 2 * st + 1 < nbk ? f16_bits_to_f32(P.wd[sc_row * (uint32_t)nbk + b1]) : 0.f;
    }
  };
  auto lwrite = [&](int buf, const Set& v) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + 256 * j, r = c >> 2, ch = c & 3;
      *(uint4*)(Ab(buf) + r * kI8Row + 16 * ch) = j == 0 ? v.a0 : v.a1;
      *(uint4*)(Bb(buf) + r * kI8Row + 16 * ch) = j == 0 ? v.b0 : v.b1;
    }
    // scales block-major: A [kb][128 rows], then B [kb][128 rows], so that
    // the four rows 4 g + j of a result are one 16-byte read
    float* sc = Asc(buf) + (sc_a ? 0 : 256) + (tid & 127);
    sc[0] = v.s0;
    sc[128] = v.s1;
  };
  const int wr0 = (wave >> 1) * (16 * kI8MI), wc0 = (wave & 1) * (16 * kI8NB);
  f32x4_t acc[kI8MI][kI8NB];
#pragma unroll
  for (int i = 0; i < kI8MI; ++i)
#pragma unroll
    for (int b = 0; b < kI8NB; ++b) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    // (one block at a time: unrolling both keeps twice the operands live and
    // spills)
#pragma unroll 1
    for (int kb = 0; kb < 2; ++kb) {
      // lane (li, g) supplies codes k = 8 g .. 8 g + 7 of block kb of A row
      // (or B row) li of its group; the result holds rows 4 g + j, column li.
      // All 16 products of the block are issued before their scaling, so
      // the matrix cores' latency is covered by the later ones.
      long bq[kI8NB], aq[kI8MI];
      float bs[kI8NB];
#pragma unroll
      for (int b = 0; b < kI8NB; ++b) {
        const int n = wc0 + 16 * b + li;
        bq[b] = *(const long*)(Bb(buf) + n * kI8Row + 32 * kb + 8 * g);
        bs[b] = Bsc(buf)[128 * kb + n];
      }
#pragma unroll
      for (int i = 0; i < kI8MI; ++i)
        aq[i] = *(const long*)(Ab(buf) + (wr0 + 16 * i + li) * kI8Row + 32 * kb + 8 * g);
      i32x4_t is[kI8MI][kI8NB];
#pragma unroll
      for (int i = 0; i < kI8MI; ++i)
#pragma unroll
        for (int b = 0; b < kI8NB; ++b)
          is[i][b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aq[i], bq[b], i32x4_t{0, 0, 0, 0}, 0,
                                                          0, 0);
#pragma unroll
      for (int i = 0; i < kI8MI; ++i) {
        const float4 a4 = *(const float4*)(Asc(buf) + 128 * kb + wr0 + 16 * i + 4 * g);
        const float as[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int b = 0; b < kI8NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][b][j] = fmaf((float)is[i][b][j], as[j] * bs[b], acc[i][b][j]);
      }
    }
  };
  // LDS buffer s & 1 holds step s; one step of loads is in flight in
  // registers while the current one is multiplied.  A prefetch past the last
  // step re-reads it (its buffer is not read again), so the loop has no
  // branches around the loads.
  const int last = nsteps - 1;
  Set X;
  gload(0, X);
  lwrite(0, X);
  __syncthreads();
  gload(min(1, last), X);
  for (int st = 0; st < nsteps; ++st) {
    compute(st & 1);
    lwrite((st + 1) & 1, X);
    __syncthreads();
    gload(min(st + 2, last), X);
  }
#pragma unroll
  for (int i = 0; i < kI8MI; ++i)
#pragma unroll
    for (int b = 0; b < kI8NB; ++b) {
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

extern "C" int qgemm_q8_0_i8(const void* W, int N, int K, const int8_t* q, const float* d,
                             int R, float* y, void* stream) {
  if (N < 0 || R < 0 || K <= 0 || K % 32)
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_q8_0_i8: N=%d R=%d K=%d (K %% 32 != 0)", N, R, K);
  if ((long long)N * K >= (1LL << 32) || (long long)R * K >= (1LL << 32))
    return fail(QMOE_ERR_UNSUPPORTED, "qgemm_q8_0_i8: offsets beyond 32 bits");
  if (N == 0 || R == 0) return QMOE_OK;
  if (!W || !q || !d || !y) return fail(QMOE_ERR_INVALID_ARG, "qgemm_q8_0_i8: null pointer");
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(q, 16) || !QMOE_ALIGNED(d, 4) ||
      !QMOE_ALIGNED(y, 4))
    return fail(QMOE_ERR_INVALID_ARG, "qgemm_q8_0_i8: misaligned W/q/d/y");
  const Layout L = layout_of(QMOE_Q8_0, N, K);
  I8GemmParams P{(const int8_t*)W + L.off[0], (const uint16_t*)((const uint8_t*)W + L.off[1]),
                 q, d, y, N, K, R};
  const dim3 grid((unsigned)((N + kI8BN - 1) / kI8BN), (unsigned)((R + kI8BM - 1) / kI8BM));
  if (grid.y > 65535) return fail(QMOE_ERR_UNSUPPORTED, "qgemm_q8_0_i8: R=%d too large", R);
  return QMOE_LAUNCH("q8_0_i8_gemm", q8_0_i8_gemm_kernel, grid, kI8GBlock, kI8Lds,
                     (hipStream_t)stream, P);
}
