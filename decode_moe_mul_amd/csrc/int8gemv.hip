// Int8 activations against Q8_0 weights with integer dot products for decode
// rows ([P1] "NInfer 80 SM port": its int8 artifact quantizes the
// activations so that both operands are integers, and decode takes
// dp4a-class dot products, section 八.2).
//  * qquantize_act_q8: per 32 values along K, d = max|x| / 127 and
//    q = round-half-away(x / d) clamped to [-127, 127] (both divisions fp32,
//    correctly rounded); an all-zero block has d = 0, q = 0.
//  * qgemv_q8_0_i8: y[r, n] = sum_b d_w[n, b] d[r, b] sum_{k in b} q_w q_x:
//    each 32-value unit is 8 v_dot4_i32_i8 (exact int32), then one fp32
//    multiply-add by the two scales.  The int8 activation rows are staged in
//    LDS (up to 16 rows per pass, fewer when K is long); G lanes share a
//    weight row, each owning whole units, and the row sums meet in a DPP
//    reduction.
#include "decode.hpp"

namespace qmoe {

// ------------------------------------------------ activation quantizer ----
__global__ __launch_bounds__(256) void quantize_act_q8_kernel(const void* x, int x_dtype, int R,
                                                              int K, int8_t* q, float* d) {
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
      const uint4 b = p[i];
      const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
        v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float dd = amax / 127.f;
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = 0;
      if (dd > 0.f) {
        const float r = v[4 * i + j] / dd;
        const float t = truncf(r);
        c = (int)t + (fabsf(r - t) >= 0.5f ? (r < 0.f ? -1 : 1) : 0);
        c = min(max(c, -127), 127);
      }
      word |= ((uint32_t)c & 0xFFu) << (8 * j);
    }
    out[i] = word;
  }
  uint4* dst = (uint4*)(q + at);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  d[blk] = dd;
}

// ----------------------------------------------------------- the GEMV ----
constexpr int kI8Batch = 4;  // units per lane whose loads are in flight together

struct I8Params {
  const int8_t* wq;       // [N][K]
  const uint16_t* wd;     // [N][K/32] fp16
  const int8_t* xq;       // [R][K]
  const float* xd;        // [R][K/32]
  float* y;               // [R][N]
  int N, K, R, G, tile_rows, rc;
};

// Block b: weight rows [b tile_rows, (b + 1) tile_rows); rc activation rows
// per pass (the last pass may hold fewer).  Every lane runs the same loop
// count (rows past the tile re-read its last row and are not stored).
template <int RC>
__global__ __launch_bounds__(256) void qgemv_q8_0_i8_kernel(I8Params P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = P.K, U = K >> 5, G = P.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = 64 / G, g = lane & (G - 1), slot = lane / G;
  const int rb = blockIdx.x * P.tile_rows, re = min(P.N, rb + P.tile_rows);
  const int step = 4 * sub;
  int8_t* xs = (int8_t*)smem;                       // [rc][K]
  float* xds = (float*)(smem + (size_t)P.rc * K);   // [rc][U]
  for (int c0 = 0; c0 < P.R; c0 += P.rc) {
    const int rc = min(P.rc, P.R - c0);
    __syncthreads();  // earlier readers of the staged rows are done
    for (int i = threadIdx.x; i < rc * (K >> 4); i += 256)
      ((uint4*)xs)[i] = ((const uint4*)(P.xq + (size_t)c0 * K))[i];
    for (int i = threadIdx.x; i < rc * U; i += 256) xds[i] = P.xd[(size_t)c0 * U + i];
    __syncthreads();
    for (int row0 = rb + wave * sub; row0 < re; row0 += step) {
      const int row = min(row0 + slot, re - 1);
      const int8_t* wr = P.wq + (size_t)row * K;
      const uint16_t* wdr = P.wd + (size_t)row * U;
      float acc[RC];
#pragma unroll
      for (int r = 0; r < RC; ++r) acc[r] = 0.f;
      // the lane's units g, g + G, ... in batches of kI8Batch whose loads are
      // all issued before the first is used (a batch past the lane's last
      // unit re-reads that unit and adds nothing)
      const int nu = U / G;
      for (int i0 = 0; i0 < nu; i0 += kI8Batch) {
        uint4 w0[kI8Batch], w1[kI8Batch];
        uint16_t sc[kI8Batch];
#pragma unroll
        for (int j = 0; j < kI8Batch; ++j) {
          const int u = g + G * min(i0 + j, nu - 1);
          w0[j] = load_stream((const uint4*)(wr + 32 * u));
          w1[j] = load_stream((const uint4*)(wr + 32 * u + 16));
          sc[j] = wdr[u];
        }
#pragma unroll
        for (int j = 0; j < kI8Batch; ++j) {
          if (i0 + j >= nu) break;
          const int u = g + G * (i0 + j);
          const float dw = f16_bits_to_f32(sc[j]);
          const int wv[8] = {(int)w0[j].x, (int)w0[j].y, (int)w0[j].z, (int)w0[j].w,
                             (int)w1[j].x, (int)w1[j].y, (int)w1[j].z, (int)w1[j].w};
#pragma unroll
          for (int r = 0; r < RC; ++r) {
            if (r < rc) {
              const uint4 a0 = *(const uint4*)(xs + (size_t)r * K + 32 * u);
              const uint4 a1 = *(const uint4*)(xs + (size_t)r * K + 32 * u + 16);
              const int av[8] = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                 (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
              int s = 0;
#pragma unroll
              for (int q = 0; q < 8; ++q) s = __builtin_amdgcn_sdot4(wv[q], av[q], s, false);
              acc[r] = fmaf((float)s, dw * xds[r * U + u], acc[r]);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RC; ++r) {
        const float v = group_reduce(acc[r], G);
        if (r < rc && g == G - 1 && row0 + slot < re) P.y[(size_t)(c0 + r) * P.N + row] = v;
      }
    }
  }
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qquantize_act_q8(const void* x, int x_dtype, int R, int K, int8_t* q, float* d,
                     void* stream) {
  if (R < 0 || K <= 0 || K % 32)
    return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_q8: R=%d K=%d (K %% 32 != 0)", R, K);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "qquantize_act_q8: unknown x_dtype %d", x_dtype);
  if (R == 0) return QMOE_OK;
  if (!x || !q || !d) return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_q8: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(q, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qquantize_act_q8: misaligned x/q");
  const long long blocks = (long long)R * (K / 32);
  return QMOE_LAUNCH("quantize_act_q8", quantize_act_q8_kernel,
                     dim3((unsigned)((blocks + 255) / 256)), 256, 0, (hipStream_t)stream, x,
                     x_dtype, R, K, q, d);
}

int qgemv_q8_0_i8(const void* W, int N, int K, const int8_t* q, const float* d, int R, float* y,
                  void* stream) {
  if (N < 0 || R < 0 || R > 16 || K <= 0 || K % 32)
    return fail(QMOE_ERR_INVALID_ARG, "qgemv_q8_0_i8: N=%d R=%d K=%d (R <= 16, K %% 32 == 0)",
                N, R, K);
  if (N == 0 || R == 0) return QMOE_OK;
  if (!W || !q || !d || !y) return fail(QMOE_ERR_INVALID_ARG, "qgemv_q8_0_i8: null pointer");
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(q, 16))
    return fail(QMOE_ERR_INVALID_ARG, "qgemv_q8_0_i8: misaligned W/q");
  const Layout L = layout_of(QMOE_Q8_0, N, K);
  I8Params P{(const int8_t*)W + L.off[0], (const uint16_t*)((const uint8_t*)W + L.off[1]), q, d,
             y, N, K, R, 0, 0, 0};
  // staged rows per pass: as many as fit 64 KB with their scales
  const size_t per_row = (size_t)K + (size_t)(K / 32) * sizeof(float);
  P.rc = (int)std::min<size_t>(R, (size_t)kLdsCap / per_row);
  if (P.rc < 1) return fail(QMOE_ERR_UNSUPPORTED, "qgemv_q8_0_i8: K=%d too long to stage", K);
  P.G = lanes_per_row(K);
  P.tile_rows = pick_tile_rows(N, P.G, 1);
  const dim3 grid((unsigned)((N + P.tile_rows - 1) / P.tile_rows));
  const size_t lds = (size_t)P.rc * per_row;
  hipStream_t s = (hipStream_t)stream;
  const int rc = P.rc;
  if (rc <= 1) return QMOE_LAUNCH("qgemv_q8_0_i8", qgemv_q8_0_i8_kernel<1>, grid, 256, lds, s, P);
  if (rc <= 2) return QMOE_LAUNCH("qgemv_q8_0_i8", qgemv_q8_0_i8_kernel<2>, grid, 256, lds, s, P);
  if (rc <= 4) return QMOE_LAUNCH("qgemv_q8_0_i8", qgemv_q8_0_i8_kernel<4>, grid, 256, lds, s, P);
  if (rc <= 8) return QMOE_LAUNCH("qgemv_q8_0_i8", qgemv_q8_0_i8_kernel<8>, grid, 256, lds, s, P);
  return QMOE_LAUNCH("qgemv_q8_0_i8", qgemv_q8_0_i8_kernel<16>, grid, 256, lds, s, P);
}

}  // extern "C"
