// Decode-side quantized GEMV: qgemv_<fmt> (dense, [P3] "RTX 3090 Llama 70B
// three-tier cache" section 4.4) and the two phases of moe_ffn_tiered (routed
// experts in mixed-precision tiers, [P2] "Three RTX 3090 Qwen3.8-Flash-Next
// guide" sections 优化策略二/三 and bug item 4; many session rows per launch,
// [P4] "DwarfStar on 8x L40S" section "120 t/s 的秘密微批次分组解码").
//
// Decode is a weight stream: every weight byte is read once per call and
// meets only a few activation rows, so the kernel is organised around HBM
// streaming.
//  * Schedule.  One launch per phase.  Block b serves (rank b / ntiles, row
//    tile b % ntiles).  Every block ranks the experts that received rows
//    (from the permutation offsets, staged in LDS): experts with more rows
//    than the register blocking RC come first, then the others, so blocks
//    are never wasted on empty experts and the heavy ones start first.
//  * Few rows (<= RC, the common case): fp16 dot products.  The expert's
//    activation rows are staged once per block in LDS (fp16, in the weight
//    format's pair order, in a bank-conflict-free padded layout).  A weight
//    row is reduced by G lanes (G a power of two, every lane owning >= 4
//    whole 32-value units); a wave covers 64/G rows at a time.  Each lane
//    streams its (row, unit) sequence through a 3-4 deep load pipeline that
//    runs across row boundaries, decodes each unit once to exact fp16 pairs,
//    and dots it against all staged rows with v_dot2_f32_f16; the unit scale
//    is applied once per unit in fp32; row sums are reduced with DPP.
//  * Many rows (a shared expert that sees every session row): the same row
//    tile runs on the matrix cores, 16 rows at a time, fp16 operands
//    dequantized in registers, v_mfma_f32_16x16x32_f16.
//  * Gate and up rows of the same output are handled by the same lanes, so
//    SiLU(g) * u is applied in registers before anything is stored.
#include <algorithm>
#include <cmath>
#include <cstdio>

#include "decode.hpp"

namespace qmoe {

// ----------------------------------------------------------- qgemv ------
struct GemvParams {
  const void* W;
  int N, K;
  const void* x;
  int x_dtype, R;
  float* y;
  int G, tile_rows;
};

template <int FMT, int RC, bool MFMA>
__global__ __launch_bounds__(kBlock) void qgemv_kernel(GemvParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int N = P.N, K = P.K, dtype = P.x_dtype;
  const char* xb = (const char*)P.x;
  float* y = P.y;
  const Mat mats[1] = {mat_of(P.W, FMT, N, K)};
  const int rb = blockIdx.x * P.tile_rows, re = min(N, rb + P.tile_rows);
  const size_t xrow_bytes = (size_t)K * (dtype == QMOE_F32 ? 4 : 2);
  auto src = [=](int r) { return (const void*)(xb + (size_t)r * xrow_bytes); };
  auto sink = [=](int n, int r, const float* a) { y[(size_t)r * N + n] = a[0]; };
  if (MFMA) {
    if (dtype == QMOE_F32)
      mfma_cols<FMT, 1, QMOE_F32>(mats, K, rb, re, P.R, smem, src, sink);
    else
      mfma_cols<FMT, 1, QMOE_BF16>(mats, K, rb, re, P.R, smem, src, sink);
  }
  else
    valu_rows<FMT, 1, RC>(mats, K, rb, re, P.G, P.R, dtype, smem, src, sink);
}

// ------------------------------------------------ batched dense GEMV ----
// Several independent matrices in one launch: block b serves matrix i with
// block_off[i] <= b < block_off[i + 1] and row tile b - block_off[i].  Each
// matrix is processed exactly as qgemv would (same lanes per row, same
// register blocking), so its output equals qgemv's bit for bit.
struct GemvBatchParams {
  qmoe_gemv_desc d[QMOE_MAX_BATCH];
  int G[QMOE_MAX_BATCH], tile_rows[QMOE_MAX_BATCH];
  int rc[QMOE_MAX_BATCH];  // rows per dot-product chunk; 0: matrix cores
  int block_off[QMOE_MAX_BATCH + 1];
  int n;
};

template <int RC, bool MFMA>
__global__ __launch_bounds__(kBlock) void qgemv_batch_kernel(GemvBatchParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  // matrix of this block, its fields taken with constant indices only (a
  // runtime index into the by-value argument would spill it to scratch)
  const int b = blockIdx.x;
  int fmt = 0, N = 0, K = 0, dtype = 0, R = 0, G = 1, tr = 1, boff = 0, rc = 1;
  const void* W = nullptr;
  const void* x = nullptr;
  float* y = nullptr;
#pragma unroll
  for (int i = 0; i < QMOE_MAX_BATCH; ++i) {
    if (i < P.n && b >= P.block_off[i] && b < P.block_off[i + 1]) {
      fmt = P.d[i].fmt; N = P.d[i].N; K = P.d[i].K; dtype = P.d[i].x_dtype; R = P.d[i].R;
      W = P.d[i].W; x = P.d[i].x; y = P.d[i].y;
      G = P.G[i]; tr = P.tile_rows[i]; boff = P.block_off[i]; rc = P.rc[i];
    }
  }
  if (!W) return;
  const int rb = (b - boff) * tr, re = min(N, rb + tr);
  if (rb >= re) return;
  const char* xb = (const char*)x;
  const size_t xrow_bytes = (size_t)K * (dtype == QMOE_F32 ? 4 : 2);
  auto src = [=](int r) { return (const void*)(xb + (size_t)r * xrow_bytes); };
  auto sink = [=](int n, int r, const float* a) { y[(size_t)r * N + n] = a[0]; };
#define QMOE_BATCH_CASE(FM)                                                      \
  case FM: {                                                                     \
    const Mat mats[1] = {mat_of(W, FM, N, K)};                                   \
    if (MFMA && rc == 0 && dtype == QMOE_F32)                                    \
      mfma_cols<FM, 1, QMOE_F32>(mats, K, rb, re, R, smem, src, sink);           \
    else if (MFMA && rc == 0)                                                    \
      mfma_cols<FM, 1, QMOE_BF16>(mats, K, rb, re, R, smem, src, sink);          \
    else                                                                         \
      valu_rows<FM, 1, RC>(mats, K, rb, re, G, R, dtype, smem, src, sink, rc);   \
  } break;
  switch (fmt) {
    QMOE_BATCH_CASE(QMOE_Q8_0)
    QMOE_BATCH_CASE(QMOE_Q4_0)
    QMOE_BATCH_CASE(QMOE_MXFP4)
    QMOE_BATCH_CASE(QMOE_Q4_K)
    QMOE_BATCH_CASE(QMOE_Q6_K)
    default: break;
  }
#undef QMOE_BATCH_CASE
}

// PHASE 0: gate/up + SwiGLU -> h;  PHASE 1: down -> o.  MFMA: whether
// experts with more than m_max rows can occur (the matrix-core branch costs
// registers, so launches that cannot use it leave it out).  Gate/up blocks
// take the registers of two blocks per compute unit (gate and up tiles at
// once, or a deep ring of weight loads for one row), down blocks of three.
template <int PHASE, int RC, bool MFMA>
__global__ __launch_bounds__(kBlock, PHASE == 1 ? 3 : 2) void ffn_decode_kernel(FfnParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int32_t* perm = P.perm;
  int* red = (int*)smem;
  int tile = 0, pos0 = 0, m = 0;
  bool big = false;
  // block-uniform values read from LDS, moved to scalar registers so that
  // the weight bases derived from them stay scalar (loads then take a
  // scalar base and a 32-bit vector offset)
  const int e = __builtin_amdgcn_readfirstlane(scheduled_expert(
      P.offsets, P.E, P.m_max, blockIdx.x, P.ntiles, P.ntiles_big, red, tile, big, pos0, m));
  if (e < 0) return;
  tile = __builtin_amdgcn_readfirstlane(tile);
  big = __builtin_amdgcn_readfirstlane((int)big) != 0;
  pos0 = __builtin_amdgcn_readfirstlane(pos0);
  m = __builtin_amdgcn_readfirstlane(m);
  ffn_item<PHASE, RC, MFMA, false, false>(P, e, tile, big, pos0, m, smem,
                                          [=](int i) { return perm[i]; });
}

// ------------------------------------------------------ host helpers ----
int t5_check(const char* who, const qmoe_gemv_desc& q);             // ternary.hip
int t5_batch_launch(const qmoe_gemv_desc* d, int n, void* stream);  // ternary.hip

// Rows per block for a dense matrix of mat_bytes in a launch that streams
// total_bytes: per_cu blocks per compute unit overall, but no fewer than
// kMinBlockBytes of weights per block, since every block stages its own copy
// of the activation rows; each matrix gets blocks in proportion to its bytes.
// A multiple of a wave pass and of the 16-row matrix-core blocks.
constexpr size_t kMinBlockBytes = 64 << 10;
constexpr size_t kLdsPerCu = 160 << 10;  // LDS of one CDNA4 compute unit
static int pick_tile_rows_bytes(int N, int G, size_t mat_bytes, size_t total_bytes,
                                int per_cu = 8) {
  int group = kWaves * (64 / G);
  if (group < 16) group = 16;
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const long long by_bytes = (long long)(total_bytes / kMinBlockBytes);
  const long long blocks =
      std::min<long long>((long long)per_cu * cus, std::max<long long>(cus, by_bytes));
  long long tiles = total_bytes ? (long long)((double)blocks * mat_bytes / total_bytes) : 1;
  const long long max_tiles = (N + group - 1) / group;
  tiles = std::max<long long>(1, std::min(tiles, max_tiles));
  const int rows = (int)((N + tiles - 1) / tiles);
  return (rows + group - 1) / group * group;
}

template <int FMT>
static int qgemv_dispatch(const GemvParams& P, int RC, dim3 grid, size_t lds, hipStream_t s) {
  if (P.R > RC) return QMOE_LAUNCH("qgemv", (qgemv_kernel<FMT, 4, true>), grid, kBlock, lds, s, P);
  if (RC == 1) return QMOE_LAUNCH("qgemv", (qgemv_kernel<FMT, 1, false>), grid, kBlock, lds, s, P);
  if (RC == 2) return QMOE_LAUNCH("qgemv", (qgemv_kernel<FMT, 2, false>), grid, kBlock, lds, s, P);
  return QMOE_LAUNCH("qgemv", (qgemv_kernel<FMT, 4, false>), grid, kBlock, lds, s, P);
}

static int qgemv_launch(int FMT, const void* W, int N, int K, const void* x, int x_dtype,
                        int R, float* y, void* stream) {
  if (!W || !x || !y) return fail(QMOE_ERR_INVALID_ARG, "qgemv: null pointer");
  if (N < 0 || K <= 0 || R < 0 || K % block_of(FMT) || K > 65536)
    return fail(QMOE_ERR_INVALID_ARG, "qgemv: bad sizes N=%d K=%d R=%d", N, K, R);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "qgemv: unknown x_dtype %d", x_dtype);
  if (!QMOE_ALIGNED(W, 256) || !QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(y, 4))
    return fail(QMOE_ERR_INVALID_ARG, "qgemv: misaligned pointer");
  if (N == 0 || R == 0) return QMOE_OK;
  // RC = 0: one staged row does not fit in LDS (K > 27456); such rows (and
  // more rows than RC) take the matrix-core path, which stages nothing
  const int RC = pick_rc(R, K);
  GemvParams P{W, N, K, x, x_dtype, R, y, lanes_per_row(K), 0};
  const size_t wbytes = layout_of(FMT, N, K).total;
  P.tile_rows = pick_tile_rows_bytes(N, P.G, wbytes, wbytes);
  if (R > RC) {  // matrix-core tiles: whole 64-column passes
    const int pass = 16 * mfma_cols_per_pass(1);
    P.tile_rows = (P.tile_rows + pass - 1) / pass * pass;
  }
  const dim3 grid((N + P.tile_rows - 1) / P.tile_rows);
  const size_t lds = R > RC ? mfma_red_bytes(1) : stage_bytes(RC, K);
  hipStream_t s = (hipStream_t)stream;
  switch (FMT) {
    case QMOE_Q8_0: return qgemv_dispatch<QMOE_Q8_0>(P, RC, grid, lds, s);
    case QMOE_Q4_0: return qgemv_dispatch<QMOE_Q4_0>(P, RC, grid, lds, s);
    case QMOE_MXFP4: return qgemv_dispatch<QMOE_MXFP4>(P, RC, grid, lds, s);
    case QMOE_Q4_K: return qgemv_dispatch<QMOE_Q4_K>(P, RC, grid, lds, s);
    default: return qgemv_dispatch<QMOE_Q6_K>(P, RC, grid, lds, s);
  }
}

// Batched GEMV: each matrix is checked as qgemv checks it and takes the path
// qgemv would take for it (dot products in chunks of pick_rc(R, K) rows, or
// the matrix cores beyond), with qgemv's lanes per row, so its arithmetic
// matches qgemv's exactly.  The kernel's register blocking is the largest
// chunk of the batch, its LDS the largest staging.
static int qgemv_batch_launch(const qmoe_gemv_desc* d, int n, void* stream) {
  if (n < 0 || n > QMOE_MAX_BATCH)
    return fail(QMOE_ERR_INVALID_ARG, "qgemv_batch: n=%d outside [0, %d]", n, QMOE_MAX_BATCH);
  if (n == 0) return QMOE_OK;
  if (!d) return fail(QMOE_ERR_INVALID_ARG, "qgemv_batch: null descriptors");
  int n_t5 = 0;
  for (int i = 0; i < n; ++i) n_t5 += d[i].fmt == QMOE_T5;
  if (n_t5 == n) {  // a batch of ternary matrices: the T5 kernel
    for (int i = 0; i < n; ++i) {
      char who[32];
      snprintf(who, sizeof who, "qgemv_batch: matrix %d", i);
      const int st = t5_check(who, d[i]);
      if (st) return st;
    }
    return t5_batch_launch(d, n, stream);
  }
  GemvBatchParams P{};
  P.n = n;
  bool any_mfma = false;
  long long blocks = 0;
  for (int i = 0; i < n; ++i) {
    const qmoe_gemv_desc& q = d[i];
    if (!tier_format(q.fmt))  // (T5 only in batches of T5 matrices)
      return fail(QMOE_ERR_UNSUPPORTED, "qgemv_batch: matrix %d: format %d not in this batch", i,
                  q.fmt);
    const bool work = q.N > 0 && q.R > 0;  // empty products touch no memory
    if (work && (!q.W || !q.x || !q.y))
      return fail(QMOE_ERR_INVALID_ARG, "qgemv_batch: matrix %d null pointer", i);
    if (q.N < 0 || q.K <= 0 || q.R < 0 || q.R > 16 || q.K % block_of(q.fmt) || q.K > 65536)
      return fail(QMOE_ERR_INVALID_ARG, "qgemv_batch: matrix %d bad sizes N=%d K=%d R=%d", i, q.N,
                  q.K, q.R);
    if (q.x_dtype != QMOE_F32 && q.x_dtype != QMOE_BF16)
      return fail(QMOE_ERR_UNSUPPORTED, "qgemv_batch: matrix %d unknown x_dtype %d", i, q.x_dtype);
    if (work && (!QMOE_ALIGNED(q.W, 256) || !QMOE_ALIGNED(q.x, 16) || !QMOE_ALIGNED(q.y, 4)))
      return fail(QMOE_ERR_INVALID_ARG, "qgemv_batch: matrix %d misaligned pointer", i);
    P.d[i] = q;
  }
  int RC = 1;
  size_t lds = 0, total_bytes = 0;
  for (int i = 0; i < n; ++i)
    if (d[i].N > 0 && d[i].R > 0) total_bytes += layout_of(d[i].fmt, d[i].N, d[i].K).total;
  // One round of blocks: as many per compute unit as the largest staging
  // lets its 160 KB of LDS hold at once, at most eight (a second round of
  // blocks would start behind a ragged first one).
  size_t lds_max = 0;
  for (int i = 0; i < n; ++i)
    if (d[i].N > 0 && d[i].R > 0)
      lds_max = std::max(lds_max, d[i].R > pick_rc(d[i].R, d[i].K)
                                      ? mfma_red_bytes(1)
                                      : stage_bytes(pick_rc(d[i].R, d[i].K), d[i].K));
  const int per_cu = lds_max ? (int)std::max<size_t>(1, std::min<size_t>(8, kLdsPerCu / lds_max)) : 8;
  for (int i = 0; i < n; ++i) {
    const qmoe_gemv_desc& q = d[i];
    const int rc = pick_rc(q.R, q.K);
    P.G[i] = lanes_per_row(q.K);
    int tr = pick_tile_rows_bytes(q.N, P.G[i], layout_of(q.fmt, q.N, q.K).total, total_bytes,
                                  per_cu);
    const bool mc = q.R > rc;
    P.rc[i] = mc ? 0 : rc;
    any_mfma |= mc;
    if (!mc) {
      RC = std::max(RC, rc);
      lds = std::max(lds, stage_bytes(rc, q.K));
    } else {
      lds = std::max(lds, mfma_red_bytes(1));
    }
    if (mc) {
      const int pass = 16 * mfma_cols_per_pass(1);
      tr = (tr + pass - 1) / pass * pass;
    }
    P.tile_rows[i] = tr;
    P.block_off[i] = (int)blocks;
    blocks += (q.N == 0 || q.R == 0) ? 0 : (q.N + tr - 1) / tr;
  }
  P.block_off[n] = (int)blocks;
  if (blocks == 0) return QMOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks);
  if (any_mfma)
    return QMOE_LAUNCH("qgemv", (qgemv_batch_kernel<4, true>), grid, kBlock, lds, s, P);
  if (RC == 1) return QMOE_LAUNCH("qgemv", (qgemv_batch_kernel<1, false>), grid, kBlock, lds, s, P);
  if (RC == 2) return QMOE_LAUNCH("qgemv", (qgemv_batch_kernel<2, false>), grid, kBlock, lds, s, P);
  return QMOE_LAUNCH("qgemv", (qgemv_batch_kernel<4, false>), grid, kBlock, lds, s, P);
}

template <int PHASE, bool MFMA>
static int ffn_dispatch2(const FfnParams& P, int RC, dim3 grid, size_t lds, hipStream_t s) {
  const char* name = PHASE == 0 ? "ffn_gate_up" : "ffn_down";
  if (RC == 1) return QMOE_LAUNCH(name, (ffn_decode_kernel<PHASE, 1, MFMA>), grid, kBlock, lds, s, P);
  if (RC == 2) {
    allow_lds(ffn_decode_kernel<PHASE, 2, MFMA>, lds);
    return QMOE_LAUNCH(name, (ffn_decode_kernel<PHASE, 2, MFMA>), grid, kBlock, lds, s, P);
  }
  allow_lds(ffn_decode_kernel<PHASE, 4, MFMA>, lds);
  return QMOE_LAUNCH(name, (ffn_decode_kernel<PHASE, 4, MFMA>), grid, kBlock, lds, s, P);
}

template <int PHASE>
static int ffn_dispatch(const FfnParams& P, int RC, dim3 grid, size_t lds, hipStream_t s) {
  return P.m_max < 0x7FFFFFFF ? ffn_dispatch2<PHASE, true>(P, RC, grid, lds, s)
                              : ffn_dispatch2<PHASE, false>(P, RC, grid, lds, s);
}

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);

// Blocks per CU for one phase of the routed FFN: 8 per 256 KB of weights a
// block would stream at 8 per CU (ranks experts of the phase's largest tier),
// between 4 and 24.  Long blocks leave a long tail once the last ones start
// (16 rows through 256 experts of [2048, 7168] Q4_K, about 2 MB per block at
// 8 per CU; 8 / 12 / 16 / 24 / 32 / 48 per CU: gate/up 376 / 367 / 365 / 354
// / 355 / 367 us per step of the three decode calls); a few rows through
// small experts (about 60 KB per block at 8) run faster as fewer, longer
// blocks (the 6-row tiered call 79.4 -> 75.1 us at 4 per CU).
int ffn_blocks_per_cu(const qmoe_tier* tiers, int n_tiers, int H, int F, int phase,
                      int ranks) {
  size_t worst = 0;
  for (int i = 0; i < n_tiers; ++i) {
    const size_t b = phase == 0 ? 2 * layout_of(tiers[i].fmt_gate_up, F, H).total
                                : layout_of(tiers[i].fmt_down, H, F).total;
    worst = std::max(worst, b);
  }
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const double per_block = (double)ranks * (double)worst / (8.0 * cus);
  return std::min(24, std::max(4, (int)(8.0 * per_block / (double)(256 << 10))));
}



}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qgemv_q8_0(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q8_0, W, N, K, x, d, R, y, s);
}
int qgemv_q4_0(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q4_0, W, N, K, x, d, R, y, s);
}
int qgemv_mxfp4(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_MXFP4, W, N, K, x, d, R, y, s);
}
int qgemv_q4_k(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q4_K, W, N, K, x, d, R, y, s);
}
int qgemv_q6_k(const void* W, int N, int K, const void* x, int d, int R, float* y, void* s) {
  return qgemv_launch(QMOE_Q6_K, W, N, K, x, d, R, y, s);
}

int qgemv_batch(const qmoe_gemv_desc* descs, int n, void* stream) {
  return qgemv_batch_launch(descs, n, stream);
}

size_t moe_ffn_workspace_size(int T, int k, int F) {
  if (T < 0 || k < 0 || F < 0) return 0;
  return round_up256((size_t)T * k * F * sizeof(float)) + 256;
}

int moe_ffn_tiered(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, const void* x,
                   int x_dtype, int T, int k, const int32_t* offsets, const int32_t* perm,
                   float* o, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 0) return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: T=%d k=%d", T, k);
  if (T == 0 || k == 0) return QMOE_OK;
  int st = validate_tiers(tiers, n_tiers, E, H, F, false);
  if (st) return st;
  if (E > 8192) return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: E=%d > 8192", E);
  if (!x || !offsets || !perm || !o)
    return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: null pointer");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: unknown x_dtype %d", x_dtype);
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(o, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_ffn_tiered: misaligned x/o");
  const size_t need = moe_ffn_workspace_size(T, k, F);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_ffn_tiered: workspace %zu < %zu (or misaligned)",
                ws_bytes, need);
  const long long A = (long long)T * k;
  if (A > (1 << 24)) return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: T*k too large");
  // rc = 0: not even one row of that K fits in LDS; then every expert of
  // that phase takes the matrix-core path (m_max = 0)
  const int rc1 = pick_rc(T, H, kFfnStageBudget), rc2 = pick_rc(T, F, kFfnStageBudget);
  hipStream_t s = (hipStream_t)stream;
  FfnParams P{};
  for (int i = 0; i < n_tiers; ++i) P.tiers[i] = tiers[i];
  P.n_tiers = n_tiers; P.E = E; P.H = H; P.F = F; P.T = T; P.k = k;
  P.x = x; P.x_dtype = x_dtype; P.offsets = offsets; P.perm = perm;
  P.h = (float*)ws; P.o = o;
  const int ranks = (int)(A < E ? A : E);  // experts that can receive rows
  const size_t sched_bytes = (size_t)kSchedRedInts * 4;
  // Experts with more rows than the dot-product path blocks in registers
  // use the matrix cores, when the row count allows that to happen (with
  // duplicate ids the dot-product path loops over row chunks instead).
  for (int phase = 0; phase < 2; ++phase) {
    const int N = phase == 0 ? F : H, K = phase == 0 ? H : F, rc = phase == 0 ? rc1 : rc2;
    P.G = lanes_per_row(K);
    P.tile_rows =
        pick_tile_rows(N, P.G, ranks, ffn_blocks_per_cu(tiers, n_tiers, H, F, phase, ranks));
    P.ntiles = (N + P.tile_rows - 1) / P.tile_rows;
    P.m_max = rc == 0 ? 0 : T > rc ? rc : 0x7FFFFFFF;
    // A many-row expert gets up to (m_max + 1) * ntiles blocks and holds at
    // least m_max + 1 of the A row assignments, so no routing needs more
    // than min(A * ntiles, E * max(ntiles, ntiles_big)) blocks.
    const long long big_cap = (long long)(rc + 1) * P.ntiles, cols16 = (N + 15) / 16;
    P.ntiles_big = (int)(big_cap < cols16 ? big_cap : cols16);
    const long long need_a = A * P.ntiles;
    const long long need_e = (long long)E * (P.ntiles > P.ntiles_big ? P.ntiles : P.ntiles_big);
    const long long nblocks = need_a < need_e ? need_a : need_e;
    if (nblocks >= (1LL << 31)) return fail(QMOE_ERR_UNSUPPORTED, "moe_ffn_tiered: grid too large");
    size_t lds = rc ? stage_bytes(rc, K) : 0;
    if (lds < sched_bytes) lds = sched_bytes;
    if (lds < mfma_red_bytes(2 - phase)) lds = mfma_red_bytes(2 - phase);
    const dim3 grid((unsigned)nblocks);
    const int rc_t = rc ? rc : 1;  // register blocking of the (unused) dot-product path
    st = phase == 0 ? ffn_dispatch<0>(P, rc_t, grid, lds, s) : ffn_dispatch<1>(P, rc_t, grid, lds, s);
    if (st) return st;
  }
  return QMOE_OK;
}

}  // extern "C"
