// moe_route: router logits, top-k with ties to the lower id, renormalised
// softmax over the kept logits, always-on shared experts appended.
// ([P2] "Three RTX 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析: a light
// router picks 10 of 512 experts per token; [P4] "DwarfStar on 8x L40S",
// section 快速上手: a shared expert beside the routed ones.)
//
// Kernels:
//  router_gemv_kernel  rows <= 16: 16 waves per block, each streaming one
//                      expert row of Wr over a K-slice against all rows
//                      staged in LDS; split-K partials go to the workspace.
//  router_gemm_kernel  longer chunks: 64x64 output tiles on the matrix cores
//                      (fp32 operands and sums).
//  topk_kernel         one wave per row: sums the split-K partials in fixed
//                      order, adds the bias, selects k by repeated wave
//                      arg-max, softmax over the kept logits.
#include <algorithm>
#include <mutex>

#include "route.hpp"

namespace qmoe {

__global__ __launch_bounds__(kGemvBlock) void router_gemv_kernel(RouteParams P) {
  extern __shared__ __align__(16) float xsl[];  // [T][ks_len]
  router_partials<false, kGemvBlock>(P, xsl, blockIdx.x, blockIdx.y);
}

// 128 x 128 tile of logits (rows x experts) over one K slice on the matrix
// cores in fp32 (v_mfma_f32_16x16x4_f32, fp32 products and sums).  Wave w
// computes rows 64 (w >> 1) .. and experts 64 (w & 1) .. of the tile as
// 4 x 4 blocks of 16 x 16, so each operand value a lane loads feeds four
// blocks (with 2 x 2 blocks per wave the operand loads, not the matrix cores,
// bounded the kernel).  Per 16-wide chunk of the slice each lane loads 4
// consecutive values of its rows of x and of its experts' rows of Wr; op s of
// the chunk takes value s of every lane group, so both operands walk the
// chunk's 16 indices in the same interleaved order.  Two chunks of loads are
// in flight.  Slice blockIdx.z writes part[z][t][e].
constexpr int kGT = 128, kGE = 128, kGDepth = 2;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
QMOE_D void rg_load(const RouteParams& P, const int (&trow)[4], const int (&erow)[4], int k,
                    float4 (&a)[4], float4 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = load_act4<DT>(P.x, (size_t)trow[i] * P.H + k);
    b[i] = *(const float4*)(P.Wr + (size_t)erow[i] * P.H + k);
  }
}

template <int DT>
__global__ __launch_bounds__(kRouteBlock) void router_gemm_kernel(RouteParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int tb = blockIdx.y * kGT + 64 * (wave >> 1), eb = blockIdx.x * kGE + 64 * (wave & 1);
  // operand rows, clamped: rows past the end re-read the last one (dropped)
  int trow[4], erow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    trow[i] = min(tb + 16 * i + r, P.T - 1);
    erow[i] = min(eb + 16 * i + r, P.E - 1);
  }
  const int k0 = blockIdx.z * P.ks_len, klen = min(P.ks_len, P.H - k0);  // klen % 4 == 0
  const int nch = (klen + 15) / 16;
  // this lane's 4 values of chunk c start at k; past the slice (when its
  // length is not a multiple of 16) the load re-reads the last 4 and the
  // values are zeroed
  auto k_of = [&](int c) { return k0 + min(16 * c + 4 * kg, klen - 4); };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float4 ra[kGDepth][4], rb[kGDepth][4];
#pragma unroll
  for (int u = 0; u < kGDepth; ++u) rg_load<DT>(P, trow, erow, k_of(min(u, nch - 1)), ra[u], rb[u]);
  for (int c0 = 0; c0 < nch; c0 += kGDepth) {
#pragma unroll
    for (int u = 0; u < kGDepth; ++u) {
      const int c = c0 + u;
      const bool valid = c < nch && 16 * c + 4 * kg < klen;
      float4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = valid ? ra[u][i] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[i] = rb[u][i];
      }
      rg_load<DT>(P, trow, erow, k_of(min(c + kGDepth, nch - 1)), ra[u], rb[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].x, b[j].x, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].y, b[j].y, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].z, b[j].z, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].w, b[j].w, acc[i][j], 0, 0, 0);
        }
    }
  }
  // lane holds rows 4 kg + q of each 16 x 16 block, column r
  float* part = P.part + (size_t)blockIdx.z * P.T * P.E;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = tb + 16 * i + 4 * kg + q, e = eb + 16 * j + r;
        if (t < P.T && e < P.E) part[(size_t)t * P.E + e] = acc[i][j][q];
      }
}

// K split of the matrix-core router (more than kGemvRowsMax rows): slices of
// whole 16-value chunks, as many as bring the launch to about 256 blocks of
// 128 x 128 tiles (at most 8).
static void gemm_split(int T, int H, int E, int& KS, int& ks_len) {
  const long long tiles = (long long)((E + kGE - 1) / kGE) * ((T + kGT - 1) / kGT);
  const int want = (int)std::max<long long>(1, std::min<long long>(8, (256 + tiles - 1) / tiles));
  ks_len = ((H + want - 1) / want + 15) / 16 * 16;
  KS = (H + ks_len - 1) / ks_len;
}

// The router's K split for T rows: route_split up to kGemvRowsMax rows, the
// matrix-core split beyond.
static void router_split(int T, int H, int E, int& KS, int& ks_len) {
  if (T > kGemvRowsMax) gemm_split(T, H, E, KS, ks_len);
  else route_split(T, H, KS, ks_len);
}


// One wave per row: the row's final logits (split-K partials summed in slice
// order, then the bias: row_logits, whose loads for all the lane's experts
// are in flight together), then its top-k.
template <int PER>  // values per lane: E <= 64 * PER
__global__ __launch_bounds__(kRouteBlock) void topk_kernel(RouteParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= P.T) return;
  float raw[PER];
  row_logits<PER>(P, t, raw);
  if (P.logits) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < P.E) P.logits[(size_t)t * P.E + lane + 64 * i] = raw[i];
  }
  int my_id;
  float my_raw;
  wave_topk<PER>(raw, P.E, P.k, my_id, my_raw);
  write_topk(P, t, my_id, my_raw, nullptr);
}

// ------------------------------------------- fused decode routing -------
// router_partials -> final logits -> top-k -> permutation in one launch for
// up to 16 rows.  The block that completes last (a device-scope counter in
// the workspace decides) gives one wave to each row: the wave sums that row's
// split-K partials in slice order (as moe_route's top-k does), takes its top-k and
// writes ids/p; the block then sorts the assignments (by the rows' expert
// masks, since a row names an expert at most once).  Partials are written
// through and read past L2 (store_coherent/load_coherent) and each thread
// drains its stores before the block's counter increment, so no device-wide
// fence (an L2 write-back plus invalidate per wave) is needed.  The finishing
// block resets the counter, so it starts and ends at zero.
struct RouteDecodeParams {
  RouteParams r;
  unsigned* ctr;       // [1]
  int32_t* offsets;    // [E_total + 1]
  int32_t* perm;       // [T * kt]
  int32_t* inv;        // [T * kt]
  int E_total, W, nbits;
  int rows_fit;  // permute_rows' LDS fits (else the counting sorts)
};

constexpr int kDecodeLdsInts = 8192;  // LDS ints of the fused kernel (32 KiB)

template <int PER>
__global__ __launch_bounds__(kGemvBlock) void route_decode_kernel(RouteDecodeParams D) {
  extern __shared__ __align__(16) float smem[];
  __shared__ int last;
  const RouteParams& P = D.r;
  router_partials<true, kGemvBlock>(P, smem, blockIdx.x, blockIdx.y);
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0)
    last = atomicAdd(&D.ctr[0], 1u) == gridDim.x * gridDim.y - 1u;
  __syncthreads();
  if (!last) return;
  const int kt = P.k + P.n_shared, A = P.T * kt;
  int32_t* ids_l = (int32_t*)smem;  // [A]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = wave; t < P.T; t += kGemvBlock / 64) {  // one row per wave
    float raw[PER];
    row_logits<PER>(P, t, raw);
    if (P.logits) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (lane + 64 * i < P.E) P.logits[(size_t)t * P.E + lane + 64 * i] = raw[i];
    }
    int my_id;
    float my_raw;
    wave_topk<PER>(raw, P.E, P.k, my_id, my_raw);
    write_topk(P, t, my_id, my_raw, ids_l);
  }
  __syncthreads();
  int* hist = (int*)smem + ((A + 63) & ~63);
  if (D.rows_fit)
    permute_rows<kGemvBlock>(ids_l, P.T, kt, D.E_total, D.offsets, D.perm, D.inv, hist);
  else if (A <= kGemvBlock)
    permute_small<kGemvBlock>(ids_l, A, D.E_total, D.offsets, D.perm, D.inv, hist);
  else
    permute_block<kGemvBlock>(ids_l, A, D.E_total, D.W, D.nbits, D.offsets, D.perm, D.inv,
                               hist, hist + D.W * D.E_total);
  if (threadIdx.x == 0)
    __hip_atomic_store(&D.ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

size_t moe_route_workspace_size(int T, int H, int E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  int KS, ks_len;
  router_split(T, H, E, KS, ks_len);
  return round_up256((size_t)KS * T * E * sizeof(float)) + 256;
}

int moe_route(const void* x, int x_dtype, int T, int H, const float* Wr, const float* bias,
              int E, int k, int n_shared, int32_t* ids, float* p, float* logits, void* ws,
              size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || k > 64 || n_shared < 0)
    return fail(QMOE_ERR_INVALID_ARG, "moe_route: bad sizes T=%d H=%d E=%d k=%d n_shared=%d",
                T, H, E, k, n_shared);
  if (E > 4096) return fail(QMOE_ERR_UNSUPPORTED, "moe_route: E=%d > 4096", E);
  if (H % 4) return fail(QMOE_ERR_INVALID_ARG, "moe_route: H %% 4 != 0");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_route: unknown x_dtype %d", x_dtype);
  if (T == 0) return QMOE_OK;
  if (!x || !Wr || !ids || !p) return fail(QMOE_ERR_INVALID_ARG, "moe_route: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(Wr, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_route: misaligned x/Wr");
  const size_t need = moe_route_workspace_size(T, H, E);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu (or misaligned)", ws_bytes,
                need);
  RouteParams P{x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids, p, logits, (float*)ws, 0, 0};
  router_split(T, H, E, P.KS, P.ks_len);
  hipStream_t s = (hipStream_t)stream;
  int st;
  if (T <= kGemvRowsMax) {
    const dim3 grid((E + kGemvExperts - 1) / kGemvExperts, P.KS);
    st = QMOE_LAUNCH("router_gemv", router_gemv_kernel, grid, kGemvBlock,
                     (size_t)T * P.ks_len * sizeof(float), s, P);
  } else {
    const dim3 grid((E + kGE - 1) / kGE, (T + kGT - 1) / kGT, P.KS);
    st = x_dtype == QMOE_F32
             ? QMOE_LAUNCH("router_gemm", router_gemm_kernel<QMOE_F32>, grid, kRouteBlock, 0, s, P)
             : QMOE_LAUNCH("router_gemm", router_gemm_kernel<QMOE_BF16>, grid, kRouteBlock, 0, s, P);
  }
  if (st) return st;
  const dim3 tgrid((T + 3) / 4);
  const int per = (E + 63) / 64;
  if (per <= 1) return QMOE_LAUNCH("topk", topk_kernel<1>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 2) return QMOE_LAUNCH("topk", topk_kernel<2>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 4) return QMOE_LAUNCH("topk", topk_kernel<4>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 8) return QMOE_LAUNCH("topk", topk_kernel<8>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 16) return QMOE_LAUNCH("topk", topk_kernel<16>, tgrid, kRouteBlock, 0, s, P);
  if (per <= 32) return QMOE_LAUNCH("topk", topk_kernel<32>, tgrid, kRouteBlock, 0, s, P);
  return QMOE_LAUNCH("topk", topk_kernel<64>, tgrid, kRouteBlock, 0, s, P);
}

// Fused decode routing: the block counter, then the split-K partials
constexpr size_t kDecodeCtrBytes = 256;

size_t moe_route_decode_workspace_size(int T, int H, int E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  return kDecodeCtrBytes + round_up256((size_t)KS * T * E * sizeof(float));
}

}  // extern "C"

namespace qmoe {

__global__ void zero_words_kernel(unsigned* w, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

// The size checks of the fused decode routing (host only, before any device
// call).
static int route_decode_sizes(const char* who, int x_dtype, int T, int H, int E, int k,
                              int n_shared) {
  if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || k > 64 || n_shared < 0)
    return fail(QMOE_ERR_INVALID_ARG, "%s: bad sizes T=%d H=%d E=%d k=%d n_shared=%d", who, T,
                H, E, k, n_shared);
  if (T > kGemvRowsMax)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: T=%d > %d rows", who, T, kGemvRowsMax);
  if (E > 512) return fail(QMOE_ERR_UNSUPPORTED, "%s: E=%d > 512", who, E);
  if (H % 4) return fail(QMOE_ERR_INVALID_ARG, "%s: H %% 4 != 0", who);
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: unknown x_dtype %d", who, x_dtype);
  return QMOE_OK;
}

// moe_route_decode on the workspace ws; `who` names the entry point in error
// texts; clear_ctr: zero the block counter first (one small kernel).
static int route_decode_impl(const char* who, const void* x, int x_dtype, int T, int H,
                             const float* Wr, const float* bias, int E, int k, int n_shared,
                             int32_t* ids, float* p, float* logits, int32_t* offsets,
                             int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes,
                             bool clear_ctr, void* stream) {
  const int sz = route_decode_sizes(who, x_dtype, T, H, E, k, n_shared);
  if (sz) return sz;
  const int kt = k + n_shared, E_total = E + n_shared, A = T * kt;
  const int hist_ints = kDecodeLdsInts - ((A + 63) & ~63) - kGemvBlock / 64;
  if (hist_ints < E_total)
    return fail(QMOE_ERR_UNSUPPORTED, "%s: T*(k+n_shared)=%d with %d experts "
                "does not fit the fused permutation", who, A, E_total);
  if (!offsets) return fail(QMOE_ERR_INVALID_ARG, "%s: null offsets", who);
  if (T == 0)  // nothing to route; the empty permutation still zeroes offsets
    return moe_permute(nullptr, 0, kt, E_total, offsets, nullptr, nullptr, stream);
  if (!x || !Wr || !ids || !p || !perm || !inv_perm)
    return fail(QMOE_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(Wr, 16))
    return fail(QMOE_ERR_INVALID_ARG, "%s: misaligned x/Wr", who);
  const size_t need = moe_route_decode_workspace_size(T, H, E);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "%s: workspace %zu < %zu (or misaligned)", who, ws_bytes,
                need);
  uint8_t* w = (uint8_t*)ws;
  RouteDecodeParams D{};
  D.r = RouteParams{x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids, p, logits, nullptr, 0, 0};
  route_split(T, H, D.r.KS, D.r.ks_len);
  D.ctr = (unsigned*)w;
  D.r.part = (float*)(w + kDecodeCtrBytes);
  D.offsets = offsets;
  D.perm = perm;
  D.inv = inv_perm;
  D.E_total = E_total;
  D.W = permute_waves(A, E_total, hist_ints, kGemvBlock / 64);
  D.nbits = id_bits(E_total);
  D.rows_fit = hist_ints >= 2 * E_total + 1 + kGemvBlock / 64;
  const dim3 grid((E + kGemvExperts - 1) / kGemvExperts, D.r.KS);
  const size_t lds = std::max((size_t)kDecodeLdsInts * 4, (size_t)T * D.r.ks_len * 4);
  hipStream_t s = (hipStream_t)stream;
  if (clear_ctr) {
    const int st = QMOE_LAUNCH("zero_words", zero_words_kernel, dim3(1), 64, 0, s, D.ctr,
                               (int)(kDecodeCtrBytes / 4));
    if (st) return st;
  }
  const int per = (E + 63) / 64;
#define QMOE_ROUTE_DECODE(PERV) \
  return QMOE_LAUNCH("route_decode", route_decode_kernel<PERV>, grid, kGemvBlock, lds, s, D)
  if (per <= 1) QMOE_ROUTE_DECODE(1);
  if (per <= 2) QMOE_ROUTE_DECODE(2);
  if (per <= 4) QMOE_ROUTE_DECODE(4);
  QMOE_ROUTE_DECODE(8);
#undef QMOE_ROUTE_DECODE
}

// ------------------------------------------- no-allocation variant ------
// The workspace of moe_route_decode_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes its
// name to a kernel (on the host it is only a stand-in symbol): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
constexpr size_t kRouteScratchBytes = (size_t)1 << 20;  // 1 MiB
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];
static bool g_scratch_cleared[kMaxDevices];

// Device address of this device's scratch, looked up with the device current
// on the first call on it; *cleared says whether a call has already zeroed
// its counter.
static int scratch_of_device(int* dev_out, void** out, bool* cleared) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QMOE_ERR_HIP, "moe_route_decode_noalloc: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QMOE_ERR_HIP, "moe_route_decode_noalloc: hipGetSymbolAddress: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *dev_out = dev;
  *out = g_scratch_ptr[dev];
  *cleared = g_scratch_cleared[dev];
  return QMOE_OK;
}

static void scratch_mark_cleared(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch_cleared[dev] = true;
}

}  // namespace qmoe

extern "C" {

int moe_route_decode(const void* x, int x_dtype, int T, int H, const float* Wr,
                     const float* bias, int E, int k, int n_shared, int32_t* ids, float* p,
                     float* logits, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                     size_t ws_bytes, void* stream) {
  return route_decode_impl("moe_route_decode", x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids,
                           p, logits, offsets, perm, inv_perm, ws, ws_bytes, false, stream);
}

size_t moe_route_decode_noalloc_max_bytes(void) { return kRouteScratchBytes; }

int moe_route_decode_noalloc(const void* x, int x_dtype, int T, int H, const float* Wr,
                             const float* bias, int E, int k, int n_shared, int32_t* ids,
                             float* p, float* logits, int32_t* offsets, int32_t* perm,
                             int32_t* inv_perm, void* stream) {
  const int sz = route_decode_sizes("moe_route_decode_noalloc", x_dtype, T, H, E, k, n_shared);
  if (sz) return sz;
  const size_t need = moe_route_decode_workspace_size(T, H, E);
  if (need > kRouteScratchBytes)
    return fail(QMOE_ERR_UNSUPPORTED,
                "moe_route_decode_noalloc: T=%d H=%d E=%d needs %zu bytes of scratch, more "
                "than the %zu it holds",
                T, H, E, need, kRouteScratchBytes);
  void* ws = nullptr;
  bool cleared = false;
  int dev = 0;
  int st = scratch_of_device(&dev, &ws, &cleared);
  if (st) return st;
  // the counter starts at zero: the array is zero when the code object
  // loads, the first successful call on a device clears it once more with a
  // kernel (no memset), and every call leaves it at zero
  st = route_decode_impl("moe_route_decode_noalloc", x, x_dtype, T, H, Wr, bias, E, k,
                         n_shared, ids, p, logits, offsets, perm, inv_perm, ws,
                         kRouteScratchBytes, !cleared, stream);
  if (st == QMOE_OK && !cleared && T > 0) scratch_mark_cleared(dev);
  return st;
}

}  // extern "C"
