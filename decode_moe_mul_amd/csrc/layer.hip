// moe_layer_decode: one decode step of the routed-expert layer in a single
// launch -- router, top-k with the renormalised softmax, expert permutation,
// gate/up + SwiGLU, down projection and the weighted combine ([P2] "Three RTX
// 3090 Qwen3.8-Flash-Next guide", section 瓶颈分析: a light router picks 10 of
// 512 experts per token and the layer returns their weighted sum; sections
// 优化策略二/三: experts of three precision tiers in one layer).
//
// At one to a few rows the separate launches of the layer each stream only a
// few MB, so their time goes to dependency latency: every launch waits for
// the previous one to drain, then re-reads its inputs before its first weight
// load.  Here one plain launch holds three kinds of blocks, in block-index
// order, and each block waits only for the data it needs:
//   * router blocks (the first): split-K router partials of 16 experts over
//     one K-slice, written through the L2; the block that completes the last
//     one (an arrival counter decides) takes the top-k of every row, sorts the
//     assignments by expert, publishes ids, p, offsets, perm and inv_perm and
//     raises the routing flag;
//   * gate/up blocks: wait for the flag, take their item of the routed-FFN
//     schedule (moe_ffn_tiered's), write h through and count themselves in on
//     their expert's counter;
//   * down blocks: wait for the flag, take their item, wait until every
//     gate/up block of their expert has counted in, write o through and count
//     themselves in on one counter per (token, 64-row chunk) they covered; the
//     block that completes such a counter (one arrival per valid slot of the
//     token) sums the chunk of y in slot order with moe_combine's arithmetic.
// Blocks only wait for blocks of lower index, which the dispatcher starts
// earlier (every XCD takes its blocks in index order), so the waits end
// whatever the grid size.  No cooperative launch and no grid-wide barrier.
// Every wait is bounded (about a second): a block that gives up sets an
// error word in the workspace and carries on, so a launch always ends.
//
// The arithmetic is that of moe_route_decode, moe_ffn_tiered and
// moe_combine (the same router partials and their order, the same top-k,
// the same unique stable sort, the same FFN items with the same register
// blocking and lanes per row, the same fmaf chain over slots), so the outputs
// equal that sequence of calls bit for bit.
//
// Counters (the first 16 KiB of the workspace, zero between calls): error
// word; 8 group exit counters and a global one (the last block out puts the
// flag and the exit counters back to zero); the router arrival counter (reset
// by the routing block); the routing flag; per expert the gate/up arrivals
// and the down blocks past their wait (the last down block of an expert
// resets both); per (token, chunk) the combine arrivals (reset by the block
// that sums the chunk).  Values handed between blocks are written through
// (agent-scope relaxed atomics), each thread drains its stores before its
// block's arrival is counted, and readers load past the L2.
#include <algorithm>

#include "route.hpp"
#include "decode.hpp"

namespace qmoe {

constexpr int kLayerRowsMax = kGemvRowsMax;  // 16
constexpr int kLayerPer = 8;                 // E <= 64 * 8
constexpr int kLayerAMax = 1024;             // assignments (single-barrier sort)
constexpr unsigned kSpinLimit = 1u << 18;
constexpr int kGroups = 8;
constexpr int kLine = 64;  // uint32 words per 256-byte line
constexpr int kErrW = 0, kGrpW = kLine, kGlbW = 9 * kLine, kRouteW = 10 * kLine,
              kReadyW = 11 * kLine, kArrW = 12 * kLine;
constexpr size_t kLayerCtrBytes = 16384;
constexpr int kLayerCtrWords = (int)(kLayerCtrBytes / 4);
constexpr int kCombRows = 64;  // rows of H per combine counter
constexpr int kRouterExperts = 4 * kWaves;  // experts per router block

struct LayerParams {
  RouteParams r;   // ids and p are the published outputs
  FfnParams f[2];  // gate/up and down schedules (f[1] also: inv, p, y)
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  float* y;
  unsigned* ctr;
  int E_total, kt, A;
  int eblocks;  // router blocks per K-slice
  int nr, ng, nd;  // router, gate/up and down blocks
  int nch;         // combine chunks of H
  uint64_t* sched;  // [ng + nd] schedule entries (write_schedule)
};

QMOE_D unsigned* hcnt_of(const LayerParams& P) { return P.ctr + kArrW; }
QMOE_D unsigned* dcnt_of(const LayerParams& P) { return P.ctr + kArrW + P.E_total; }
QMOE_D unsigned* comb_of(const LayerParams& P) { return P.ctr + kArrW + 2 * P.E_total; }

// Thread 0 waits until the word reaches `target` (bounded); the block then
// goes on together.
QMOE_D void block_wait(const LayerParams& P, const unsigned* w, unsigned target) {
  if (threadIdx.x == 0) {
    for (unsigned n = 0;
         __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++n) {
      if (n == kSpinLimit) {
        __hip_atomic_store(P.ctr + kErrW, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      // a long pause between polls: hundreds of waiting blocks polling one
      // word would otherwise load the memory channel behind it
      __builtin_amdgcn_s_sleep(32);
    }
  }
  __syncthreads();
}

QMOE_D unsigned arrive(unsigned* w) {
  return __hip_atomic_fetch_add(w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The schedule of one FFN phase, as scheduled_expert orders its blocks
// (experts with more than m_max rows first with ntiles_big blocks each, then
// the other non-empty experts with ntiles each, both groups in id order):
// entry vb = {expert | tile << 16 | big << 31, first position | rows << 16}
// as two words of one 64-bit store, expert 0xFFFF past the end.  Written
// through by the routing block, one entry per thread at a time; ord holds E
// ints of LDS.
QMOE_D void write_schedule(const FfnParams& F, const int32_t* offs, int E, int* ord,
                           uint64_t* table, int nblocks) {
  __shared__ int red[2 * kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (E + kBlock - 1) / kBlock;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int nb = 0, ns = 0;  // this thread's big / small experts
  for (int e = lo; e < hi; ++e) {
    const int m = offs[e + 1] - offs[e];
    nb += m > F.m_max;
    ns += m > 0 && m <= F.m_max;
  }
  int sb = nb, ss = ns;
  for (int off = 1; off < 64; off <<= 1) {
    const int ob = __shfl_up(sb, off, 64), os = __shfl_up(ss, off, 64);
    if (lane >= off) { sb += ob; ss += os; }
  }
  if (lane == 63) { red[wave] = sb; red[kWaves + wave] = ss; }
  __syncthreads();
  int bb = 0, bs = 0, tb = 0, ts = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) { bb += red[w]; bs += red[kWaves + w]; }
    tb += red[w];
    ts += red[kWaves + w];
  }
  int ib = bb + sb - nb, is = tb + bs + ss - ns;  // big experts first in ord
  for (int e = lo; e < hi; ++e) {
    const int m = offs[e + 1] - offs[e];
    if (m > F.m_max) ord[ib++] = e;
    else if (m > 0) ord[is++] = e;
  }
  __syncthreads();
  const int big_blocks = tb * F.ntiles_big;
  for (int vb = tid; vb < nblocks; vb += kBlock) {
    int e = 0xFFFF, tile = 0, big = 0;
    if (vb < big_blocks) {
      const int i = vb / F.ntiles_big;
      e = ord[i];
      tile = vb - i * F.ntiles_big;
      big = 1;
    } else {
      const int j = (vb - big_blocks) / F.ntiles;
      if (j < ts) {
        e = ord[tb + j];
        tile = vb - big_blocks - j * F.ntiles;
      }
    }
    uint32_t w1 = 0;
    if (e != 0xFFFF) w1 = (uint32_t)offs[e] | ((uint32_t)(offs[e + 1] - offs[e]) << 16);
    const uint32_t w0 = (uint32_t)e | ((uint32_t)tile << 16) | ((uint32_t)big << 31);
    __hip_atomic_store(table + vb, (uint64_t)w0 | ((uint64_t)w1 << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // red and ord are reused
}

// ------------------------------------------------------------ router ----
QMOE_D void router_block(const LayerParams& P, int b, uint8_t* smem) {
  const int ks = b / P.eblocks, eb = b - ks * P.eblocks;
  float* xsl = (float*)smem;
  router_stage<kBlock>(P.r, xsl, ks);
  __syncthreads();
  constexpr int J = kRouterExperts / kWaves;  // expert rows per wave
  float4 w[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) router_wrow<kBlock>(P.r, eb * J + j, ks, w[j]);
#pragma unroll
  for (int j = 0; j < J; ++j) router_dots<true, kBlock>(P.r, xsl, eb * J + j, ks, w[j]);
  drain_vmem();
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) last = arrive(P.ctr + kRouteW) == (unsigned)P.nr - 1u;
  __syncthreads();
  if (!last) return;
  // the routing of every row (this block alone)
  const int T = P.r.T, A = P.A, E_total = P.E_total;
  int32_t* ids_l = (int32_t*)smem;     // [A]
  float* p_l = (float*)(ids_l + A);    // [A]
  int32_t* offs_l = (int32_t*)(p_l + A);  // [E_total + 1]
  int32_t* perm_l = offs_l + E_total + 1;  // [A]
  int32_t* inv_l = perm_l + A;             // [A]
  int* tmp = inv_l + A;                    // [E_total + 1]
  RouteParams R = P.r;
  R.ids = ids_l;
  R.p = p_l;
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
  permute_small<kBlock>(ids_l, A, E_total, offs_l, perm_l, inv_l, tmp);
  __syncthreads();
  for (int i = threadIdx.x; i < A; i += kBlock) {
    store_coherent(P.r.ids + i, ids_l[i]);
    store_coherent(P.r.p + i, p_l[i]);
    store_coherent(P.perm + i, perm_l[i]);
    store_coherent(P.inv + i, inv_l[i]);
  }
  for (int i = threadIdx.x; i <= E_total; i += kBlock) store_coherent(P.offsets + i, offs_l[i]);
  write_schedule(P.f[0], offs_l, E_total, tmp, P.sched, P.ng);
  write_schedule(P.f[1], offs_l, E_total, tmp, P.sched + P.ng, P.nd);
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(P.ctr + kRouteW, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(P.ctr + kReadyW, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------- combine ----
QMOE_D int valid_slots(const LayerParams& P, int t) {
  int n = 0;
  for (int i = 0; i < P.kt; ++i) n += load_coherent(P.inv + t * P.kt + i) >= 0;
  return n;
}

// y[t, col] in slot order (moe_combine's arithmetic)
QMOE_D float combine_one(const LayerParams& P, int t, int col) {
  const int H = P.r.H;
  const float* o = P.f[1].o;
  float acc = 0.f;
  for (int s = 0; s < P.kt; ++s) {
    const int pos = load_coherent(P.inv + t * P.kt + s);
    if (pos < 0) continue;
    const float w = load_coherent(P.r.p + t * P.kt + s);
    acc = fmaf(w, load_coherent(o + (size_t)pos * H + col), acc);
  }
  return acc;
}

// After a down item's o rows [rb, re) for positions pos0 .. pos0 + m - 1
// are written through: count in on every (token, chunk) covered; sum the
// chunks this block completes.
template <class PermOf>
QMOE_D void combine_arrive(const LayerParams& P, int rb, int re, int pos0, int m, int* list,
                           PermOf perm_of) {
  const int H = P.r.H;
  const int c0 = rb / kCombRows, nc = (re - 1) / kCombRows - c0 + 1;
  unsigned* comb = comb_of(P);
  constexpr int kCap = 1024;
  for (int base = 0; base < m * nc; base += kCap) {
    if (threadIdx.x == 0) list[0] = 0;
    __syncthreads();
    const int end = min(m * nc, base + kCap);
    for (int idx = base + (int)threadIdx.x; idx < end; idx += kBlock) {
      const int r = idx / nc, c = c0 + idx - r * nc;
      const int t = perm_of(pos0 + r) / P.kt;
      const unsigned old = arrive(comb + t * P.nch + c);
      if ((int)old + 1 == valid_slots(P, t)) list[1 + atomicAdd(&list[0], 1)] = t * P.nch + c;
    }
    __syncthreads();
    const int n = list[0];
    for (int idx = threadIdx.x; idx < n * kCombRows; idx += kBlock) {
      const int it = list[1 + idx / kCombRows];
      const int t = it / P.nch, col = (it - t * P.nch) * kCombRows + idx % kCombRows;
      if (col < H) P.y[(size_t)t * H + col] = combine_one(P, t, col);
      if (idx % kCombRows == 0)
        __hip_atomic_store(comb + it, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- FFN blocks ----
template <int PHASE, int RC, bool MFMA>
QMOE_D void ffn_block(const LayerParams& P, int vb, uint8_t* smem) {
  const FfnParams& F = P.f[PHASE];
  block_wait(P, P.ctr + kReadyW, 1u);
  if (PHASE == 1 && vb == 0) {  // y rows of tokens without a valid slot: zero
    for (int t = 0; t < P.r.T; ++t)
      if (valid_slots(P, t) == 0)
        for (int c = threadIdx.x; c < P.r.H; c += kBlock) P.y[(size_t)t * P.r.H + c] = 0.f;
  }
  // this block's entry of the phase's schedule (block-uniform, scalar)
  const uint64_t ent = __hip_atomic_load(P.sched + (PHASE == 0 ? 0 : P.ng) + vb,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t w0 = __builtin_amdgcn_readfirstlane((uint32_t)ent);
  const uint32_t w1 = __builtin_amdgcn_readfirstlane((uint32_t)(ent >> 32));
  const int e = (int)(w0 & 0xFFFFu);
  if (e == 0xFFFF) return;
  const int tile = (int)((w0 >> 16) & 0x7FFFu);
  const bool big = (w0 >> 31) != 0;
  const int pos0 = (int)(w1 & 0xFFFFu), m = (int)(w1 >> 16);
  const int32_t* perm = P.perm;
  auto perm_of = [=](int i) { return load_coherent(perm + i); };
  if (PHASE == 1) {  // every gate/up block of this expert has written its h
    const FfnParams& G = P.f[0];
    const unsigned nb_gu = (unsigned)(m > G.m_max ? G.ntiles_big : G.ntiles);
    block_wait(P, hcnt_of(P) + e, nb_gu);
  }
  ffn_item<PHASE, RC, MFMA, PHASE == 1, true>(F, e, tile, big, pos0, m, smem, perm_of);
  drain_vmem();
  __syncthreads();
  if (PHASE == 0) {
    if (threadIdx.x == 0) arrive(hcnt_of(P) + e);
    return;
  }
  if (threadIdx.x == 0) {  // the last down block of the expert resets its counters
    const unsigned nb_dn = (unsigned)(m > F.m_max ? F.ntiles_big : F.ntiles);
    if (arrive(dcnt_of(P) + e) + 1u == nb_dn) {
      __hip_atomic_store(hcnt_of(P) + e, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dcnt_of(P) + e, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  int rb, re;
  item_rows<1>(F, tile, big, rb, re);
  if (rb >= re) return;
  qmoe_tier t;
  if (!tier_of(F.tiers, F.n_tiers, e, t)) return;
  combine_arrive(P, rb, re, pos0, m, (int*)smem, perm_of);
}

// Every block counts out at the end (in kGroups groups, so that arrivals on
// one word do not serialise); the last one puts the flag and the exit
// counters back to zero.
QMOE_D void exit_arrive(const LayerParams& P) {
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int g = blockIdx.x % kGroups;
  const unsigned nb = gridDim.x;
  const unsigned gsize = nb / kGroups + ((unsigned)g < nb % kGroups ? 1u : 0u);
  const unsigned ngroups = nb < (unsigned)kGroups ? nb : (unsigned)kGroups;
  if (arrive(P.ctr + kGrpW + g * kLine) != gsize - 1) return;
  if (arrive(P.ctr + kGlbW) != ngroups - 1) return;
  for (int i = 0; i < kGroups; ++i)
    __hip_atomic_store(P.ctr + kGrpW + i * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(P.ctr + kGlbW, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(P.ctr + kReadyW, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int RC, bool MFMA>
__global__ __launch_bounds__(kBlock, 2) void layer_decode_kernel(LayerParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  if (b < P.nr)
    router_block(P, b, smem);
  else if (b < P.nr + P.ng)
    ffn_block<0, RC, MFMA>(P, b - P.nr, smem);
  else
    ffn_block<1, RC, MFMA>(P, b - P.nr - P.ng, smem);
  exit_arrive(P);
}

int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill);
int ffn_blocks_per_cu(const qmoe_tier* tiers, int n_tiers, int H, int F, int phase, int ranks);

// FFN schedule of one phase, as moe_ffn_tiered chooses it (the down phase's
// row tiles rounded up to whole combine chunks); returns its block count
static long long ffn_schedule(FfnParams& P, const qmoe_tier* tiers, int n_tiers, int phase,
                              int rc, int T, long long A) {
  const int N = phase == 0 ? P.F : P.H, K = phase == 0 ? P.H : P.F;
  const int ranks = (int)(A < P.E ? A : P.E);
  P.G = lanes_per_row(K);
  P.tile_rows =
      pick_tile_rows(N, P.G, ranks, ffn_blocks_per_cu(tiers, n_tiers, P.H, P.F, phase, ranks));
  if (phase == 1) P.tile_rows = (P.tile_rows + kCombRows - 1) / kCombRows * kCombRows;
  P.ntiles = (N + P.tile_rows - 1) / P.tile_rows;
  P.m_max = rc == 0 ? 0 : T > rc ? rc : 0x7FFFFFFF;
  const long long big_cap = (long long)(rc + 1) * P.ntiles, cols16 = (N + 15) / 16;
  P.ntiles_big = (int)(big_cap < cols16 ? big_cap : cols16);
  const long long need_a = A * P.ntiles;
  const long long need_e = (long long)P.E * std::max(P.ntiles, P.ntiles_big);
  return std::min(need_a, need_e);
}

// schedule table entries: a phase never schedules more than min(A, experts)
// non-empty experts times ceil(N / 16) blocks each
static size_t sched_entries(int T, int H, int E, int F, int k, int n_shared) {
  const size_t A = (size_t)T * (k + n_shared), Et = (size_t)E + n_shared;
  return std::min(A, Et) * (size_t)((F + 15) / 16 + (H + 15) / 16);
}

template <int RC, bool MFMA>
static int layer_launch(const LayerParams& P, unsigned blocks, size_t lds, hipStream_t s) {
  allow_lds(layer_decode_kernel<RC, MFMA>, lds);
  return QMOE_LAUNCH("layer_decode", (layer_decode_kernel<RC, MFMA>), dim3(blocks), kBlock, lds,
                     s, P);
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
         round_up256(A * F * sizeof(float)) + round_up256(A * H * sizeof(float)) +
         round_up256(sched_entries(T, H, E, F, k, n_shared) * sizeof(uint64_t));
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
  const int nch = (H + kCombRows - 1) / kCombRows;
  if (A > kLayerAMax || kArrW + 2 * E_total + T * nch > kLayerCtrWords)
    return fail(QMOE_ERR_UNSUPPORTED,
                "moe_layer_decode: %d assignments / %d experts / %d rows of %d do not fit the "
                "counters", A, E_total, T, H);
  int KS, ks_len;
  route_split(T, H, KS, ks_len);
  // the FFN's register blocking exactly as moe_ffn_tiered picks it
  const int rc1 = pick_rc(T, H, kFfnStageBudget), rc2 = pick_rc(T, F, kFfnStageBudget);
  const bool mfma = T > rc1 || T > rc2 || rc1 == 0 || rc2 == 0;
  const int rc_max = std::max(rc1, rc2);
  // LDS: the largest of the roles' needs
  size_t lds = (size_t)T * ks_len * sizeof(float);                                 // router
  lds = std::max(lds, (size_t)(4 * A + 2 * (E_total + 1)) * sizeof(int));          // routing
  lds = std::max(lds, (size_t)(E_total + 1 + 2 * kWaves + 2) * sizeof(int));       // schedule
  lds = std::max(lds, (size_t)(1024 + 1) * sizeof(int));                           // combine
  if (rc1) lds = std::max(lds, stage_bytes(rc1, H));
  if (rc2) lds = std::max(lds, stage_bytes(rc2, F));
  if (mfma) lds = std::max(lds, mfma_red_bytes(2));
  if (lds > kFfnStageBudget)
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: rows of H=%d / F=%d do not fit LDS", H,
                F);

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
  w += round_up256((size_t)A * H * sizeof(float));
  P.sched = (uint64_t*)w;
  long long nblk[2];
  for (int phase = 0; phase < 2; ++phase) {
    FfnParams& f = P.f[phase];
    for (int i = 0; i < n_tiers; ++i) f.tiers[i] = tiers[i];
    f.n_tiers = n_tiers; f.E = E_total; f.H = H; f.F = F; f.T = T; f.k = kt;
    f.x = x; f.x_dtype = x_dtype; f.offsets = offsets; f.perm = perm;
    f.h = h; f.o = o;
    nblk[phase] = ffn_schedule(f, tiers, n_tiers, phase, phase == 0 ? rc1 : rc2, T, A);
    f.chunk = phase == 0 ? rc1 : rc2;
  }
  P.offsets = offsets;
  P.perm = perm;
  P.inv = inv_perm;
  P.y = y;
  P.E_total = E_total;
  P.kt = kt;
  P.A = A;
  P.eblocks = (E + kRouterExperts - 1) / kRouterExperts;
  P.nr = P.eblocks * KS;
  P.ng = (int)nblk[0];
  P.nd = (int)nblk[1];
  P.nch = nch;
  if ((size_t)(nblk[0] + nblk[1]) > sched_entries(T, H, E, F, k, n_shared))
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: schedule larger than its table");
  const long long blocks = (long long)P.nr + nblk[0] + nblk[1];
  if (blocks >= (1LL << 31))
    return fail(QMOE_ERR_UNSUPPORTED, "moe_layer_decode: grid too large");
  hipStream_t s = (hipStream_t)stream;
  const unsigned nb = (unsigned)blocks;
  // one register blocking for both phases: the larger (a chunk's blocking
  // follows its row count, so a smaller phase loses nothing)
  if (!mfma) {
    if (rc_max == 1) return layer_launch<1, false>(P, nb, lds, s);
    if (rc_max == 2) return layer_launch<2, false>(P, nb, lds, s);
    return layer_launch<4, false>(P, nb, lds, s);
  }
  if (rc_max <= 1) return layer_launch<1, true>(P, nb, lds, s);
  if (rc_max == 2) return layer_launch<2, true>(P, nb, lds, s);
  return layer_launch<4, true>(P, nb, lds, s);
}

}  // extern "C"
