// moe_permute: stable counting sort of the flat routing assignments by expert
// id.  The routed matmul of [P2] "Three RTX 3090 Qwen3.8-Flash-Next guide"
// (section 优化策略三) works per expert on the tokens routed to it; its bug
// item 1 is a grouping that broke on duplicate ids, and item 3 a -1 sentinel
// turned into a huge unsigned index.  Here ids are signed and anything outside
// [0, E) gets no position at all.
//
// One workgroup of W waves.  Wave w owns the contiguous assignment range
// [w*A/W, (w+1)*A/W):
//   pass 1: per-wave histogram hist[w][e] in LDS (lanes with the same id are
//           found with ballots over the id bits; their leader adds the count);
//   scan:   offsets[e] = sum over e' < e, then per-wave cursors
//           cursor[w][e] = offsets[e] + sum over w' < w of hist[w'][e];
//   pass 2: each wave walks its range in order and places assignment a at
//           cursor[w][e] + (rank of a among equal ids in this 64-chunk).
// Ascending a within an expert follows from the range order, the chunk order
// and the lane order, so the result is the unique stable order.
#include "common.hpp"

namespace qmoe {

constexpr int kPermBlock = 1024;
constexpr int kPermLds = 15872;  // ints of LDS for hist/cursors (62 KiB)

QMOE_D uint64_t lanes_below(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

// Lanes of this wave whose id equals mine (only among `active` lanes).
QMOE_D uint64_t peers_of(int id, int nbits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < nbits; ++b) {
    const uint64_t on = __ballot((id >> b) & 1);
    m &= ((id >> b) & 1) ? on : ~on;
  }
  return m;
}

__global__ __launch_bounds__(kPermBlock) void permute_kernel(const int32_t* ids, int A, int E,
                                                             int W, int nbits,
                                                             int32_t* offsets, int32_t* perm,
                                                             int32_t* inv) {
  __shared__ int hist[kPermLds];  // [W][E]
  __shared__ int wsum[kPermBlock / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < W * E; i += kPermBlock) hist[i] = 0;
  __syncthreads();
  const long long a_begin = (long long)wave * A / W, a_end = (long long)(wave + 1) * A / W;
  // pass 1: per-wave histogram
  if (wave < W) {
    for (long long c = a_begin; c < a_end; c += 64) {
      const long long a = c + lane;
      const bool in = a < a_end;
      const int id = in ? ids[a] : -1;
      const bool valid = in && id >= 0 && id < E;
      const uint64_t active = __ballot(valid);
      const uint64_t peers = peers_of(valid ? id : 0, nbits, active);
      if (valid && (peers & lanes_below(lane)) == 0)
        hist[wave * E + id] += __popcll(peers);
    }
  }
  __syncthreads();
  // scan over experts of the per-expert totals (thread i owns a slice)
  const int per = (E + kPermBlock - 1) / kPermBlock;
  const int e_lo = min(E, threadIdx.x * per), e_hi = min(E, e_lo + per);
  int local = 0;
  for (int e = e_lo; e < e_hi; ++e)
    for (int w = 0; w < W; ++w) local += hist[w * E + e];
  // inclusive scan of `local` across the block
  int v = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += wsum[w];
  int run = wave_base + v - local;  // exclusive prefix for this thread's slice
  for (int e = e_lo; e < e_hi; ++e) {
    offsets[e] = run;
    for (int w = 0; w < W; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;  // becomes the cursor of wave w for expert e
      run += c;
    }
  }
  int total = 0;
  for (int w = 0; w < kPermBlock / 64; ++w) total += wsum[w];
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  // pass 2: stable scatter within each wave's range
  if (wave < W) {
    for (long long c = a_begin; c < a_end; c += 64) {
      const long long a = c + lane;
      const bool in = a < a_end;
      const int id = in ? ids[a] : -1;
      const bool valid = in && id >= 0 && id < E;
      const uint64_t active = __ballot(valid);
      const uint64_t peers = peers_of(valid ? id : 0, nbits, active);
      if (valid) {
        const int pos = hist[wave * E + id] + __popcll(peers & lanes_below(lane));
        perm[pos] = (int32_t)a;
        inv[a] = pos;
      } else if (in) {
        inv[a] = -1;
      }
      // all lanes have read their cursor; now the leaders advance it
      __builtin_amdgcn_wave_barrier();
      if (valid && (peers & lanes_below(lane)) == 0) hist[wave * E + id] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
    }
  }
  // positions past the valid ones hold -1
  for (long long i = (long long)total + threadIdx.x; i < A; i += kPermBlock) perm[i] = -1;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" int moe_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                           int32_t* perm, int32_t* inv_perm, void* stream) {
  if (T < 0 || k < 0 || E <= 0)
    return fail(QMOE_ERR_INVALID_ARG, "moe_permute: bad sizes T=%d k=%d E=%d", T, k, E);
  if (E > 8192) return fail(QMOE_ERR_UNSUPPORTED, "moe_permute: E=%d > 8192", E);
  const long long A = (long long)T * k;
  if (A > (1 << 24)) return fail(QMOE_ERR_UNSUPPORTED, "moe_permute: T*k too large");
  if (!offsets) return fail(QMOE_ERR_INVALID_ARG, "moe_permute: null offsets");
  if (A > 0 && (!ids || !perm || !inv_perm))
    return fail(QMOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  // waves: as many as the LDS table [W][E] allows, up to 16
  int W = kPermLds / E;
  if (W > kPermBlock / 64) W = kPermBlock / 64;
  if (W < 1) W = 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return QMOE_LAUNCH("permute", permute_kernel, dim3(1), kPermBlock, 0, (hipStream_t)stream,
                     ids, (int)A, E, W, nbits, offsets, perm, inv_perm);
}
