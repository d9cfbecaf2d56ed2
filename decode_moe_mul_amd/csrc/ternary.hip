// qgemv_t5: dense GEMV over ternary weights in the "t5_g128_fp16" format of
// [P1] "RTX 4080 SUPER native Windows 27B: NInfer 80 SM port", section 九.2
// (base-3 codes, five weights per byte, one FP16 scale per 128 weights; its
// decode is memory-bound), y[r, n] = sum_k d * t[n, k] * x[r, k].
//
// At 1.75 bits per weight the stream is 4.6 weights per byte, so the decode
// has to be cheap and free of LDS traffic: two code bytes at a time sit in the
// two 16-bit halves of a register, and the five base-3 digits come out of
// packed 16-bit arithmetic (q / 3 = (q * 171) >> 9 for q <= 242, digit =
// q - 3 (q / 3)); OR-ing a digit c into the fp16 pattern of 1024 and adding
// -1025 gives t = c - 1 exactly, so each digit pair is one fp16 pair (t of
// byte 2p, t of byte 2p + 1) for v_dot2_f32_f16.  The activations are staged
// in LDS in the same pairing (x[10p + r], x[10p + 5 + r]), r < 5, zero past the
// group's 128 values; every row slot of a wave reads the same staged words (a
// broadcast).  Products of {-1, 0, 1} with fp16 activations are exact in the
// fp32 accumulation; the group's sum is scaled by d once.
//
// Lanes: G lanes per weight row (G <= 8), lane g owns groups g, g + G, ...;
// a wave covers 64 / G rows at a time.  Each lane streams its flattened
// (row, group) sequence through a ring of kT5Ring register slots of one
// 28-byte group each; every load is unconditional (positions past the lane's
// last group or the tile's last row re-read a valid group and are weighted
// by zero or never stored).
#include <algorithm>

#include "common.hpp"

#pragma clang fp contract(off)

namespace qmoe {

constexpr int kT5Block = 256;
constexpr int kT5Waves = kT5Block / 64;
constexpr int kT5Ring = 4;
constexpr int kT5StageCap = 65536;
constexpr uint32_t kH2Neg1025 = 0xE401E401u;  // fp16 -1025 in both halves

// Staged activation words of one row: [nb][13] pairs of uint4, words r < 5 =
// (x[10p + r], x[10p + 5 + r]) of group j as fp16 pairs, words 5..7 zero.
QMOE_HD size_t t5_stage_row_bytes(int K) { return (size_t)(K / 128) * 13 * 32; }

struct T5Group {
  uint32_t w[7];
};

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// One or several T5 matrices in one launch: block b serves matrix i with
// block_off[i] <= b < block_off[i + 1], rows [tile_rows * (b - block_off[i]),
// ...) of it.  Each matrix is processed exactly as a launch of its own would.
struct T5BatchParams {
  qmoe_gemv_desc d[QMOE_MAX_BATCH];
  int G[QMOE_MAX_BATCH], tile_rows[QMOE_MAX_BATCH], rc[QMOE_MAX_BATCH];
  int block_off[QMOE_MAX_BATCH + 1];
  int n;
};

template <int RC>
__global__ __launch_bounds__(kT5Block) void qgemv_t5_kernel(T5BatchParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint4* xs = (uint4*)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the block's matrix, its fields taken with constant indices only
  const int bid = blockIdx.x;
  int N = 0, K = 128, x_dtype = 0, R = 0, G = 1, tr = 1, boff = 0, rcmax = 1;
  const uint8_t* W = nullptr;
  const void* x = nullptr;
  float* y = nullptr;
#pragma unroll
  for (int i = 0; i < QMOE_MAX_BATCH; ++i) {
    if (i < P.n && bid >= P.block_off[i] && bid < P.block_off[i + 1]) {
      N = P.d[i].N; K = P.d[i].K; x_dtype = P.d[i].x_dtype; R = P.d[i].R;
      W = (const uint8_t*)P.d[i].W; x = P.d[i].x; y = P.d[i].y;
      G = P.G[i]; tr = P.tile_rows[i]; boff = P.block_off[i]; rcmax = P.rc[i];
    }
  }
  if (!W) return;  // block-uniform
  const int nb = K / 128;
  const int rb = (bid - boff) * tr, re = min(N, rb + tr);
  const int sub = 64 / G, g = lane & (G - 1), slot = lane / G;
  const int first = rb + wave * sub, step = kT5Waves * sub;
  const int n_rg = first < re ? (re - first + step - 1) / step : 0;  // wave-uniform
  const int ng = (nb + G - 1) / G;                                    // groups per lane and row
  const int nflat = n_rg * ng;
  const size_t row_bytes = (size_t)nb * kT5GroupBytes;

  for (int r0 = 0; r0 < R; r0 += rcmax) {
    const int rc = min(rcmax, R - r0);
    // the chunk's first weight loads go out before its activations are staged
    T5Group ring[kT5Ring];
    int irg = 0, it = 0;  // next (row group, group slot) to load
    auto issue = [&](T5Group& sl) {
      const int row = min(first + irg * step + slot, re - 1);
      const int j = min(g + it * G, nb - 1);
      const uint32_t* p = (const uint32_t*)(W + (size_t)row * row_bytes + (size_t)j * kT5GroupBytes);
#pragma unroll
      for (int i = 0; i < 7; ++i) sl.w[i] = __builtin_nontemporal_load(p + i);
      if (++it == ng) { it = 0; ++irg; }
    };
    if (nflat > 0) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < kT5Ring; ++i) issue(ring[i]);
    }
    __syncthreads();  // earlier readers of the staged rows
    const int items = rc * nb * 13;
    // item (r, j, p): values 10p .. 10p + 9 of group j (8-byte aligned pairs;
    // the last pair of a group, values 128 and 129, is not read)
    auto stage = [&](auto load2) {
#pragma unroll 2
      for (int idx = tid; idx < items; idx += kT5Block) {
        const int r = idx / (nb * 13), rem = idx - r * (nb * 13);
        const int j = rem / 13, p = rem - j * 13;
        const size_t base = (size_t)(r0 + r) * K + 128 * j + 10 * p;
        float2 v[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) v[i] = (p < 12 || i < 4) ? load2(base + 2 * i) : make_float2(0.f, 0.f);
        xs[2 * idx] = make_uint4(pack_h2(v[0].x, v[2].y), pack_h2(v[0].y, v[3].x),
                                 pack_h2(v[1].x, v[3].y), pack_h2(v[1].y, v[4].x));
        xs[2 * idx + 1] = make_uint4(pack_h2(v[2].x, v[4].y), 0u, 0u, 0u);
      }
    };
    if (x_dtype == QMOE_F32)
      stage([&](size_t i) { return *(const float2*)((const float*)x + i); });
    else
      stage([&](size_t i) {
        const uint32_t w = *(const uint32_t*)((const uint16_t*)x + i);
        return make_float2(bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16));
      });
    __syncthreads();
    if (nflat == 0) continue;  // wave-uniform

    float acc[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[r] = 0.f;
    int crg = 0, ct = 0;  // (row group, group slot) being computed
    for (int f0 = 0; f0 < nflat; f0 += kT5Ring) {
#pragma unroll
      for (int q = 0; q < kT5Ring; ++q) {
        const T5Group& cur = ring[q];
        const int jr = g + ct * G;
        const bool keep = jr < nb;  // lanes past the row's last group add zero
        const int j = min(jr, nb - 1);
        const float d = keep ? f16_bits_to_f32(cur.w[6] >> 16) : 0.f;
        float s[RC];
#pragma unroll
        for (int r = 0; r < RC; ++r) s[r] = 0.f;
#pragma unroll
        for (int p = 0; p < 13; ++p) {
          // code bytes 2p, 2p + 1 in the two halves of one register
          const uint32_t word = cur.w[p >> 1];
          u16x2 q = __builtin_bit_cast(
              u16x2, __builtin_amdgcn_perm(0u, word, (p & 1) ? 0x0C030C02u : 0x0C010C00u));
          uint32_t tw[5];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const u16x2 qn = (q * (uint16_t)171) >> (uint16_t)9;  // q / 3 (q <= 242)
            const u16x2 dg = q - qn * (uint16_t)3;
            tw[r] = pk_add_h2(__builtin_bit_cast(uint32_t, dg) | H2_MAGIC, kH2Neg1025);
            q = qn;
          }
          tw[4] = pk_add_h2(__builtin_bit_cast(uint32_t, q) | H2_MAGIC, kH2Neg1025);
#pragma unroll
          for (int r = 0; r < RC; ++r) {
            if (r < rc) {
              const uint4* xp = xs + 2 * (((size_t)r * nb + j) * 13 + p);
              const uint4 x0 = xp[0], x1 = xp[1];
              s[r] = fdot2(tw[0], x0.x, s[r]);
              s[r] = fdot2(tw[1], x0.y, s[r]);
              s[r] = fdot2(tw[2], x0.z, s[r]);
              s[r] = fdot2(tw[3], x0.w, s[r]);
              s[r] = fdot2(tw[4], x1.x, s[r]);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < RC; ++r) acc[r] = fmaf(d, s[r], acc[r]);
        issue(ring[q]);  // the slot's next group, in flight for kT5Ring positions
        if (++ct == ng) {  // wave-uniform: the row group is complete
#pragma unroll
          for (int r = 0; r < RC; ++r)
            for (int off = 1; off < G; off <<= 1) acc[r] += __shfl_xor(acc[r], off, 64);
          const int row = first + crg * step + slot;
          if (crg < n_rg && row < re && g == 0) {
#pragma unroll
            for (int r = 0; r < RC; ++r)
              if (r < rc) y[(size_t)(r0 + r) * N + row] = acc[r];
          }
#pragma unroll
          for (int r = 0; r < RC; ++r) acc[r] = 0.f;
          ct = 0;
          ++crg;
        }
      }
    }
  }
}

// Host checks of one T5 matrix (as qgemv_t5 states them); 0 or a status.
int t5_check(const char* who, const qmoe_gemv_desc& q) {
  const bool work = q.N > 0 && q.R > 0;
  if (work && (!q.W || !q.x || !q.y)) return fail(QMOE_ERR_INVALID_ARG, "%s: null pointer", who);
  if (q.N < 0 || q.K <= 0 || q.R < 0 || q.R > 16 || q.K % 128 || q.K > 65536)
    return fail(QMOE_ERR_INVALID_ARG, "%s: bad sizes N=%d K=%d R=%d", who, q.N, q.K, q.R);
  if (q.x_dtype != QMOE_F32 && q.x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: unknown x_dtype %d", who, q.x_dtype);
  if (t5_stage_row_bytes(q.K) > (size_t)kT5StageCap)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: K=%d > %d (one staged row must fit in LDS)", who, q.K,
                (int)(kT5StageCap / (13 * 32)) * 128);
  if (work && (!QMOE_ALIGNED(q.W, 256) || !QMOE_ALIGNED(q.x, 16) || !QMOE_ALIGNED(q.y, 4)))
    return fail(QMOE_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return QMOE_OK;
}

// Lanes per row, rows per staged chunk and rows per block of matrix q when
// the launch streams total_bytes: about 8 blocks per CU overall, at least
// 32 KiB of weights per block, each matrix's share in proportion to its
// bytes, rows in whole wave passes.
static void t5_plan(const qmoe_gemv_desc& q, size_t total_bytes, int& G, int& rc, int& tile_rows) {
  const int nb = q.K / 128;
  G = 1;
  while (G < 8 && 2 * G <= nb) G *= 2;
  // 2 rows per staged chunk when two rows fit in LDS (K <= 9984), else 1
  rc = 2 * t5_stage_row_bytes(q.K) <= (size_t)kT5StageCap ? 2 : 1;
  int cus = cu_count();
  if (cus <= 0) cus = 256;
  const size_t bytes = (size_t)q.N * nb * kT5GroupBytes;
  const long long blocks_all =
      std::min<long long>(8LL * cus, std::max<long long>(cus, (long long)(total_bytes >> 15)));
  long long blocks = total_bytes ? (long long)((double)blocks_all * bytes / total_bytes) : 1;
  if (blocks < 1) blocks = 1;
  const int group = kT5Waves * (64 / G);
  long long rows = (q.N + blocks - 1) / blocks;
  tile_rows = (int)((rows + group - 1) / group * group);
}

// One launch over n T5 matrices (n <= QMOE_MAX_BATCH), after t5_check.
int t5_batch_launch(const qmoe_gemv_desc* d, int n, void* stream) {
  T5BatchParams P{};
  P.n = n;
  size_t total = 0;
  for (int i = 0; i < n; ++i)
    if (d[i].N > 0 && d[i].R > 0) total += (size_t)d[i].N * (d[i].K / 128) * kT5GroupBytes;
  long long blocks = 0;
  size_t lds = 0;
  bool two = false;
  for (int i = 0; i < n; ++i) {
    P.d[i] = d[i];
    t5_plan(d[i], total, P.G[i], P.rc[i], P.tile_rows[i]);
    P.block_off[i] = (int)blocks;
    if (d[i].N > 0 && d[i].R > 0) {
      blocks += (d[i].N + P.tile_rows[i] - 1) / P.tile_rows[i];
      lds = std::max(lds, P.rc[i] * t5_stage_row_bytes(d[i].K));
      two |= P.rc[i] == 2;
    }
  }
  P.block_off[n] = (int)blocks;
  if (blocks == 0) return QMOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (two) return QMOE_LAUNCH("qgemv_t5", qgemv_t5_kernel<2>, dim3((unsigned)blocks), kT5Block, lds, s, P);
  return QMOE_LAUNCH("qgemv_t5", qgemv_t5_kernel<1>, dim3((unsigned)blocks), kT5Block, lds, s, P);
}

}  // namespace qmoe

using namespace qmoe;

extern "C" int qgemv_t5(const void* W, int N, int K, const void* x, int x_dtype, int R, float* y,
                        void* stream) {
  if (!W || !x || !y) return fail(QMOE_ERR_INVALID_ARG, "qgemv_t5: null pointer");
  qmoe_gemv_desc q{QMOE_T5, N, K, x_dtype, R, 0, W, x, y};
  const int st = t5_check("qgemv_t5", q);
  if (st) return st;
  if (N == 0 || R == 0) return QMOE_OK;
  return t5_batch_launch(&q, 1, stream);
}
