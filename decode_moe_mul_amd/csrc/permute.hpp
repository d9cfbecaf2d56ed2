// Stable counting sort of routing assignments by expert id, as one
// workgroup: shared by moe_permute and the fused decode routing kernel.
// Wave w of the first W waves owns the contiguous assignment range
// [w*A/W, (w+1)*A/W):
//   pass 1: per-wave histogram hist[w][e] in LDS (LDS atomic adds);
//   scan:   offsets[e] = sum over e' < e, then per-wave cursors
//           cursor[w][e] = offsets[e] + sum over w' < w of hist[w'][e];
//   pass 2: each wave walks its range in order and places assignment a at
//           cursor[w][e] + (rank of a among equal ids in this 64-chunk).
// Ascending a within an expert follows from the range order, the chunk order
// and the lane order, so the result is the unique stable order.  Ids outside
// [0, E) get no position (inv = -1); perm past the valid count is -1.
#pragma once
#include "common.hpp"

namespace qmoe {

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

// NT threads; hist holds W*E ints and wsum NT/64 ints of LDS.  ids may live
// in global memory or LDS.  Called by every thread of the block.  The ids of
// kIdBatch 64-chunks are loaded together (every lane loads; past the range it
// re-reads the range's last id), so a pass waits for memory once per batch
// rather than once per chunk; a wave whose range fits one batch loads it once
// for both passes.
template <int NT, int kIdBatch = 8>
QMOE_D void permute_block(const int32_t* ids, int A, int E, int W, int nbits, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int* hist, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < W * E; i += NT) hist[i] = 0;
  __syncthreads();
  const long long a_begin = (long long)wave * A / W, a_end = (long long)(wave + 1) * A / W;
  auto load_batch = [&](long long c0, int (&idb)[kIdBatch]) {
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) {
      const long long a = c0 + 64 * j + lane;
      idb[j] = ids[a < a_end ? a : a_end - 1];
    }
  };
  const bool once = a_end - a_begin <= 64 * kIdBatch;  // wave-uniform
  int idk[kIdBatch];
  if (wave < W && a_begin < a_end && once) load_batch(a_begin, idk);
  // pass 1: per-wave histogram
  if (wave < W && a_begin < a_end) {
    for (long long c0 = a_begin; c0 < a_end; c0 += 64 * kIdBatch) {
      int idb[kIdBatch];
      if (once) {
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) idb[j] = idk[j];
      } else {
        load_batch(c0, idb);
      }
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j) {
        const long long c = c0 + 64 * j;
        if (c >= a_end) break;  // wave-uniform
        const long long a = c + lane;
        const int id = idb[j];
        // counts need no order: one LDS atomic per assignment
        if (a < a_end && id >= 0 && id < E) atomicAdd(&hist[wave * E + id], 1);
      }
    }
  }
  __syncthreads();
  // scan over experts of the per-expert totals (thread i owns a slice)
  const int per = (E + NT - 1) / NT;
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
  for (int w = 0; w < NT / 64; ++w) total += wsum[w];
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  // pass 2: stable scatter within each wave's range
  if (wave < W && a_begin < a_end) {
    for (long long c0 = a_begin; c0 < a_end; c0 += 64 * kIdBatch) {
      int idb[kIdBatch];
      if (once) {
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) idb[j] = idk[j];
      } else {
        load_batch(c0, idb);
      }
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j) {
        const long long c = c0 + 64 * j;
        if (c >= a_end) break;  // wave-uniform
        const long long a = c + lane;
        const bool in = a < a_end;
        const int id = idb[j];
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
  }
  // positions past the valid ones hold -1
  for (long long i = (long long)total + threadIdx.x; i < A; i += NT) perm[i] = -1;
}

// The same stable counting sort for the few assignments of decode rows (A
// <= NT, ids in LDS), with one block-wide barrier instead of the histogram
// passes: offsets[e] = number of valid ids below e (thread e counts them);
// assignment a goes to offsets[ids[a]] plus the number of earlier
// assignments with the same id.  The result is the unique stable order, so
// it equals permute_block's.  offs holds E + 1 ints of LDS.
template <int NT>
QMOE_D void permute_small(const int32_t* ids, int A, int E, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int* offs) {
  for (int e = threadIdx.x; e <= E; e += NT) {
    int c = 0;
    for (int b = 0; b < A; ++b) {
      const int id = ids[b];
      c += id >= 0 && id < e;
    }
    offs[e] = c;
    offsets[e] = c;
  }
  __syncthreads();
  const int total = offs[E];
  for (int a = threadIdx.x; a < A; a += NT) {
    const int id = ids[a];
    if (id >= 0 && id < E) {
      int r = 0;
      for (int b = 0; b < a; ++b) r += ids[b] == id;
      const int pos = offs[id] + r;
      perm[pos] = (int32_t)a;
      inv[a] = pos;
    } else {
      inv[a] = -1;
    }
  }
  for (int i = total + threadIdx.x; i < A; i += NT) perm[i] = -1;
}

// Inclusive prefix sum over the wave (DPP row shifts, then row broadcasts;
// lanes whose source is out of range add 0).
QMOE_D int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The same stable order for decode routing output: assignment a = t * kt + j
// of row t < T <= 32, where a row never names an expert twice (a top-k
// followed by distinct shared experts).  Each expert records the set of rows
// that chose it as a bit mask (LDS atomic or); offsets are the block's prefix
// sum of the masks' popcounts, and a row's rank within its expert is the
// number of earlier rows in the mask, which is the number of earlier equal
// ids.  lds holds 2 E + 1 + NT/64 ints.  Called by every thread of the block.
template <int NT>
QMOE_D void permute_rows(const int32_t* ids, int T, int kt, int E, int32_t* offsets,
                         int32_t* perm, int32_t* inv, int* lds) {
  uint32_t* rows = (uint32_t*)lds;  // [E]
  int* offs = lds + E;              // [E + 1]
  int* wsum = offs + E + 1;         // [NT / 64]
  const int A = T * kt, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += NT) rows[e] = 0u;
  __syncthreads();
  for (int a = threadIdx.x; a < A; a += NT) {
    const int id = ids[a];
    if (id >= 0 && id < E) atomicOr(&rows[id], 1u << (a / kt));
  }
  __syncthreads();
  int carry = 0;  // total of the earlier chunks of experts
  for (int e0 = 0; e0 <= E; e0 += NT) {
    const int e = e0 + threadIdx.x;
    const int c = e < E ? __builtin_popcount(rows[e]) : 0;
    const int incl = wave_prefix_sum(c);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = carry, chunk = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const int v = wsum[w];
      before += w < wave ? v : 0;
      chunk += v;
    }
    if (e <= E) {
      offs[e] = before + incl - c;
      offsets[e] = before + incl - c;
    }
    carry += chunk;
    __syncthreads();  // offs complete; wsum free for the next chunk
  }
  for (int a = threadIdx.x; a < A; a += NT) {
    const int id = ids[a];
    if (id >= 0 && id < E) {
      const int pos = offs[id] + __builtin_popcount(rows[id] & ((1u << (a / kt)) - 1u));
      perm[pos] = (int32_t)a;
      inv[a] = pos;
    } else {
      inv[a] = -1;
    }
  }
  for (int i = offs[E] + threadIdx.x; i < A; i += NT) perm[i] = -1;
}

// waves of a permute_block over A assignments and E experts with `lds_ints`
// ints of LDS for hist: one per 64 assignments (more would only add empty
// histograms to clear and scan), at most max_waves and what the LDS holds
QMOE_HD int permute_waves(long long A, int E, int lds_ints, int max_waves) {
  int W = lds_ints / E;
  if (W > max_waves) W = max_waves;
  const long long by_a = (A + 63) / 64;
  if (W > by_a) W = (int)by_a;
  return W < 1 ? 1 : W;
}
QMOE_HD int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

}  // namespace qmoe
