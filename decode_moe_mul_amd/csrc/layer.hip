// moe_layer_decode: one decode step of the routed-expert layer in a single
// launch -- router, top-k with the renormalised softmax, expert permutation,
// gate/up + SwiGLU, down projection and the weighted combine ([P2] "Three RTX
// 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析: a light router picks 10 of
// 512 experts per token and the layer returns their weighted sum; sections
// 优化策略二/三: experts of three precision tiers in one layer).
//
// At one to a few rows the separate launches of the layer (routing, the two
// FFN phases, the combine) each stream only a few MB, so their time goes to
// launch and dependency latency: every launch waits for the previous one to
// drain, then re-reads its inputs from memory before its first weight load.
// Here a grid of co-resident persistent blocks (a cooperative launch) runs
// the layer's phases back to back, separated by three grid-wide barriers:
//   1. router split-K partials (items: 4 experts x one K-slice), written
//      through the L2 so that every block can read them;
//   -- barrier --
//   2. every block sums the partials, takes the top-k of every row and sorts
//      the assignments by expert in its own LDS (identical arithmetic in every
//      block, so all blocks hold the same routing); block 0 publishes ids, p,
//      offsets, perm and inv_perm;
//   3. gate/up + SwiGLU items of the routed-FFN block schedule, h written
//      through;
//   -- barrier --
//   4. down items, o written through;
//   -- barrier --
//   5. the weighted combine of every output element, in slot order.
// Every phase uses the arithmetic of moe_route_decode, moe_ffn_tiered and
// moe_combine, so the outputs equal that sequence of calls bit for bit when
// both choose the same register blocking (they do whenever the staged rows
// of length H and F fit the same blocking).
//
// Barriers: device-scope atomics on a single address serialise (about 14 ns
// each), so 512 arrivals on one counter would take 7 us.  Blocks are split
// into kGroups groups (block b in group b % kGroups), each with its own
// arrival counter per barrier on its own 256-byte line; the last arrival of
// a group counts the group in on a global counter, and the last group's last
// arrival writes a release word per group, which that group's blocks poll.
// The same arrival scheme at the end lets the last block out reset every
// word.  Waits are bounded (about a second); a block that gives up sets an
// error word in the workspace and carries on, so a launch always ends.
#include "route.hpp"
#include "decode.hpp"

namespace qmoe {

constexpr int kLayerRowsMax = kGemvRowsMax;  // 16
constexpr int kLayerPer = 8;                 // E <= 64 * 8
constexpr unsigned kSpinLimit = 1u << 20;
constexpr int kGroups = 8;
constexpr int kSyncs = 4;                    // three barriers and the exit
constexpr int kLine = 64;                    // uint32 words per 256-byte line
// counter words, one per line: error, group arrivals [kSyncs][kGroups],
// global arrivals [kSyncs], release [kGroups]
constexpr int kErrLine = 0, kGrpLine = 1, kGlbLine = kGrpLine + kSyncs * kGroups,
              kRelLine = kGlbLine + kSyncs, kCtrLines = kRelLine + kGroups;
constexpr size_t kLayerCtrBytes = 12288;
static_assert((size_t)kCtrLines * kLine * 4 <= kLayerCtrBytes, "counter lines");

struct LayerParams {
  RouteParams r;   // ids and p are the published outputs (block 0)
  FfnParams f[2];  // gate/up and down schedules (offsets/perm live in LDS)
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  float* y;
  unsigned* ctr;
  int E_total, kt, A, W, nbits, eblocks, route_items, stage_off;
};

QMOE_D unsigned* ctr_word(unsigned* ctr, int line) { return ctr + line * kLine; }

// Counts this block in at sync point j (thread 0); true for the very last
// arrival of the grid.
QMOE_D bool sync_arrive(unsigned* ctr, int j) {
  const int g = blockIdx.x % kGroups;
  const unsigned nb = gridDim.x;
  const unsigned gsize = nb / kGroups + ((unsigned)g < nb % kGroups ? 1u : 0u);
  const unsigned ngroups = nb < (unsigned)kGroups ? nb : (unsigned)kGroups;
  const unsigned a = __hip_atomic_fetch_add(ctr_word(ctr, kGrpLine + j * kGroups + g), 1u,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a != gsize - 1) return false;
  const unsigned b = __hip_atomic_fetch_add(ctr_word(ctr, kGlbLine + j), 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  return b == ngroups - 1;
}

// Grid-wide barrier j (0, 1, 2).  Every thread first waits for its own
// written-through stores, so they are visible device-wide before the block's
// arrival is counted.
QMOE_D void grid_sync(unsigned* ctr, int j) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (sync_arrive(ctr, j)) {
      for (int g = 0; g < kGroups; ++g)
        __hip_atomic_store(ctr_word(ctr, kRelLine + g), (unsigned)(j + 1), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    unsigned* rel = ctr_word(ctr, kRelLine + blockIdx.x % kGroups);
    for (unsigned n = 0;
         __hip_atomic_load(rel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)(j + 1);
         ++n) {
      if (n == kSpinLimit) {
        __hip_atomic_store(ctr_word(ctr, kErrLine), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// One FFN phase over the schedule held in LDS: block b takes items b,
// b + gridDim.x, ... until the schedule runs out.
template <int PHASE, int RC, bool MFMA>
QMOE_D void layer_ffn_phase(const FfnParams& F, const int* offs, const int32_t* perm_l, int* red,
                            uint8_t* stage) {
  for (int vb = blockIdx.x;; vb += gridDim.x) {
    int tile = 0;
    bool big = false;
    const int e = __builtin_amdgcn_readfirstlane(
        scheduled_expert(offs, F.E, F.m_max, vb, F.ntiles, F.ntiles_big, red, tile, big));
    if (e < 0) break;
    tile = __builtin_amdgcn_readfirstlane(tile);
    big = __builtin_amdgcn_readfirstlane((int)big) != 0;
    const int pos0 = __builtin_amdgcn_readfirstlane(offs[e]);
    const int m = __builtin_amdgcn_readfirstlane(offs[e + 1]) - pos0;
    ffn_item<PHASE, RC, MFMA, true>(F, e, tile, big, pos0, m, stage,
                                    [=](int i) { return perm_l[i]; });
    __syncthreads();  // the staged rows and the schedule scratch are reused
  }
}

template <int RC, bool MFMA>
__global__ __launch_bounds__(kBlock, 2) void layer_decode_kernel(LayerParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = P.r.T, E_total = P.E_total, kt = P.kt, A = P.A;
  const int nb = gridDim.x;
  int* offs = (int*)smem;                // [E_total + 1]
  int32_t* perm_l = offs + E_total + 1;  // [A]
  int32_t* inv_l = perm_l + A;           // [A]
  int32_t* ids_l = inv_l + A;            // [A]
  float* p_l = (float*)(ids_l + A);      // [A]
  int* red = (int*)(p_l + A);            // [2 * kWaves + 2]
  uint8_t* stage = smem + P.stage_off;

  // 1. router partials
  for (int b = blockIdx.x; b < P.route_items; b += nb) {
    const int ks = b / P.eblocks;
    router_partials<true, kBlock>(P.r, (float*)stage, b - ks * P.eblocks, ks);
    __syncthreads();  // the staged x slice is reused by the next item
  }
  grid_sync(P.ctr, 0);

  // 2. routing of every row, in this block's LDS
  {
    RouteParams R{};
    R.T = T;
    R.H = P.r.H;
    R.bias = P.r.bias;
    R.E = P.r.E;
    R.k = P.r.k;
    R.n_shared = P.r.n_shared;
    R.ids = ids_l;
    R.p = p_l;
    R.part = P.r.part;
    R.KS = P.r.KS;
    R.ks_len = P.r.ks_len;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int t = wave; t < T; t += kWaves) {
      float raw[kLayerPer];
      row_logits<kLayerPer>(R, t, raw);
      int my_id;
      float my_raw;
      wave_topk<kLayerPer>(raw, R.E, R.k, my_id, my_raw);
      write_topk(R, t, my_id, my_raw, nullptr);
    }
    __syncthreads();
    permute_block<kBlock>(ids_l, A, E_total, P.W, P.nbits, offs, perm_l, inv_l, (int*)stage,
                          red);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < A; i += kBlock) {
        P.r.ids[i] = ids_l[i];
        P.r.p[i] = p_l[i];
        P.perm[i] = perm_l[i];
        P.inv[i] = inv_l[i];
      }
      for (int i = threadIdx.x; i <= E_total; i += kBlock) P.offsets[i] = offs[i];
    }
  }

  // 3. gate/up + SwiGLU -> h
  layer_ffn_phase<0, RC, MFMA>(P.f[0], offs, perm_l, red, stage);
  grid_sync(P.ctr, 1);

  // 4. down -> o
  layer_ffn_phase<1, RC, MFMA>(P.f[1], offs, perm_l, red, stage);
  grid_sync(P.ctr, 2);

  // 5. y[t] = sum_i p[t, i] * o[inv[t, i]] in slot order (moe_combine's sums)
  {
    const int H = P.r.H, H4 = H >> 2;
    const float* o = P.f[1].o;
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < T * H4; i += nb * kBlock) {
      const int t = i / H4, c = i - t * H4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < kt; ++s) {
        const int pos = inv_l[t * kt + s];
        if (pos < 0) continue;
        const float w = p_l[t * kt + s];
        const float* src = o + (size_t)pos * H + 4 * c;
        const float v0 = load_coherent(src), v1 = load_coherent(src + 1);
        const float v2 = load_coherent(src + 2), v3 = load_coherent(src + 3);
        acc.x = fmaf(w, v0, acc.x);
        acc.y = fmaf(w, v1, acc.y);
        acc.z = fmaf(w, v2, acc.z);
        acc.w = fmaf(w, v3, acc.w);
      }
      ((float4*)(P.y + (size_t)t * H))[c] = acc;
    }
  }

  // the last block out (every other block is past every barrier) resets
  // the counters for the next call
  __syncthreads();
  if (threadIdx.x == 0 && sync_arrive(P.ctr, kSyncs - 1)) {
    for (int l = kGrpLine; l < kCtrLines; ++l)
      __hip_atomic_store(ctr_word(P.ctr, l), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);

static size_t route_lds_bytes(int E_total, int A) {
  return round_up256((size_t)(E_total + 1 + 4 * A + 2 * kWaves + 2) * 4);
}

// FFN schedule of one phase, as moe_ffn_tiered chooses it
static void ffn_schedule(FfnParams& P, int phase, int rc, int T, long long A) {
  const int N = phase == 0 ? P.F : P.H, K = phase == 0 ? P.H : P.F;
  const int ranks = (int)(A < P.E ? A : P.E);
  P.G = lanes_per_row(K);
  P.tile_rows = pick_tile_rows(N, P.G, ranks);
  P.ntiles = (N + P.tile_rows - 1) / P.tile_rows;
  P.m_max = T > rc ? rc : 0x7FFFFFFF;
  const long long big_cap = (long long)(rc + 1) * P.ntiles, cols16 = (N + 15) / 16;
  P.ntiles_big = (int)(big_cap < cols16 ? big_cap : cols16);
}

template <int RC, bool MFMA>
static int layer_launch(const LayerParams& P, size_t lds, hipStream_t s) {
  const void* fn = (const void*)&layer_decode_kernel<RC, MFMA>;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, layer_decode_kernel<RC, MFMA>, kBlock,
                                                   lds) != hipSuccess || occ < 1)
    return fail(QMOE_ERR_HIP, "moe_layer_decode: no resident block fits (LDS %zu)", lds);
  int cus = cu_count();
  if (cus <= 0) return fail(QMOE_ERR_HIP, "moe_layer_decode: no device");
  const dim3 grid((unsigned)(occ * cus)), block(kBlock);
  LayerParams arg = P;
  void* args[] = {&arg};
  if (profiling_on()) profile_begin("layer_decode", s);
  const hipError_t e = hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)lds, s);
  if (e != hipSuccess)
    return fail(QMOE_ERR_HIP, "moe_layer_decode: cooperative launch of %u blocks failed: %s",
                grid.x, hipGetErrorString(e));
  const int st = check_launch("layer_decode");
  if (profiling_on()) profile_end("layer_decode", s);
  return st;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

size_t moe_layer_decode_workspace_size(int T, int H, int E, int F, int k, int n_shared) {
  if (T < 0 || H <= 0 || E <= 0 || F <= 0 || k < 0 || n_shared < 0) return 0;
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  const size_t A = (size_t)T * (k + n_shared);
  return kLayerCtrBytes + round_up256((size_t)KS * T * E * sizeof(float)) +
         round_up256(A * F * sizeof(float)) + round_up256(A * H * sizeof(float));
}

int moe_layer_decode(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, const void* x,
                     int x_dtype, int T, const float* Wr, const float* bias, int k, int n_shared,
                     int32_t* ids, float* p, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                     float* y, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || F <= 0 || E <= 0 || k < 1 || k > E || k > 64 || n_shared < 0)
    return fail(QMOE_ERR_INVALID_ARG,
                "moe_layer_decode: bad sizes T=%d H=%d F=%d E=%d k=%d n_shared=%d", T, H, F, E,
                k, n_shared);
  if (T > kLayerRowsMax)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: T=%d > %d rows", T, kLayerRowsMax);
  if (E > 64 * kLayerPer) return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: E=%d > 512", E);
  if (H % 4) return fail(QMOE_ERR_INVALID_ARG, "moe_layer_decode: H %% 4 != 0");
  if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: unknown x_dtype %d", x_dtype);
  const int kt = k + n_shared, E_total = E + n_shared, A = T * kt;
  int st = validate_tiers(tiers, n_tiers, E_total, H, F, false);
  if (st) return st;
  if (!offsets) return fail(QMOE_ERR_INVALID_ARG, "moe_layer_decode: null offsets");
  if (T == 0)  // nothing to route; the empty permutation still zeroes offsets
    return moe_permute(nullptr, 0, kt, E_total, offsets, nullptr, nullptr, stream);
  if (!x || !Wr || !ids || !p || !perm || !inv_perm || !y)
    return fail(QMOE_ERR_INVALID_ARG, "moe_layer_decode: null pointer");
  if (!QMOE_ALIGNED(x, 16) || !QMOE_ALIGNED(Wr, 16) || !QMOE_ALIGNED(y, 16))
    return fail(QMOE_ERR_INVALID_ARG, "moe_layer_decode: misaligned x/Wr/y");
  const size_t need = moe_layer_decode_workspace_size(T, H, E, F, k, n_shared);
  if (!ws || ws_bytes < need || !QMOE_ALIGNED(ws, 256))
    return fail(QMOE_ERR_WORKSPACE, "moe_layer_decode: workspace %zu < %zu (or misaligned)",
                ws_bytes, need);
  // LDS: the routing (offsets, perm, inv, ids, p, schedule scratch), then one
  // staging area shared by the phases
  const size_t route_bytes = route_lds_bytes(E_total, A);
  if (route_bytes >= (size_t)kLdsCap)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: routing of %d rows does not fit LDS", A);
  const size_t budget = (size_t)kLdsCap - route_bytes;
  const int rc1 = pick_rc(T, H, budget), rc2 = pick_rc(T, F, budget);
  const int rc = rc1 < rc2 ? rc1 : rc2;
  if (rc == 0 || stage_bytes(rc, H) > budget || stage_bytes(rc, F) > budget)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: rows of H=%d / F=%d do not fit LDS", H,
                F);
  const bool mfma = T > rc;
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  const int W = permute_waves(A, E_total, (int)(budget / 4), kWaves);
  size_t stage = std::max(stage_bytes(rc, H), stage_bytes(rc, F));
  stage = std::max(stage, (size_t)T * ks_len * sizeof(float));
  stage = std::max(stage, (size_t)W * E_total * sizeof(int));
  if (mfma) stage = std::max(stage, mfma_red_bytes(2));
  if (stage > budget)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: %zu B of LDS staging > %zu", stage,
                budget);
  const size_t lds = route_bytes + stage;

  uint8_t* w = (uint8_t*)ws;
  LayerParams P{};
  P.r = RouteParams{x, x_dtype, T, H, Wr, bias, E, k, n_shared, ids, p, nullptr, nullptr, KS,
                    ks_len};
  P.ctr = (unsigned*)w;
  w += kLayerCtrBytes;
  P.r.part = (float*)w;
  w += round_up256((size_t)KS * T * E * sizeof(float));
  float* h = (float*)w;
  w += round_up256((size_t)A * F * sizeof(float));
  float* o = (float*)w;
  for (int phase = 0; phase < 2; ++phase) {
    FfnParams& f = P.f[phase];
    for (int i = 0; i < n_tiers; ++i) f.tiers[i] = tiers[i];
    f.n_tiers = n_tiers; f.E = E_total; f.H = H; f.F = F; f.T = T; f.k = kt;
    f.x = x; f.x_dtype = x_dtype; f.offsets = nullptr; f.perm = nullptr;
    f.h = h; f.o = o;
    ffn_schedule(f, phase, rc, T, A);
  }
  P.offsets = offsets;
  P.perm = perm;
  P.inv = inv_perm;
  P.y = y;
  P.E_total = E_total;
  P.kt = kt;
  P.A = A;
  P.W = W;
  P.nbits = id_bits(E_total);
  P.eblocks = (E + kWaves - 1) / kWaves;
  P.route_items = P.eblocks * KS;
  P.stage_off = (int)route_bytes;
  hipStream_t s = (hipStream_t)stream;
  if (!mfma) {
    if (rc == 1) return layer_launch<1, false>(P, lds, s);
    if (rc == 2) return layer_launch<2, false>(P, lds, s);
    return layer_launch<4, false>(P, lds, s);
  }
  if (rc == 1) return layer_launch<1, true>(P, lds, s);
  if (rc == 2) return layer_launch<2, true>(P, lds, s);
  return layer_launch<4, true>(P, lds, s);
}

}  // extern "C"
