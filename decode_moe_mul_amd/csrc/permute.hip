// moe_permute: stable counting sort of the flat routing assignments by expert
// id.  The routed matmul of [P2] "Three RTX 3090 Qwen3.8-Flash-Next guide"
// (section 优化策略三) works per expert on the tokens routed to it; its bug
// item 1 is a grouping that broke on duplicate ids, and item 3 a -1 sentinel
// turned into a huge unsigned index.  Here ids are signed and anything outside
// [0, E) gets no position at all.  The sort itself is permute_block
// (permute.hpp), run by one 1024-thread workgroup.
#include "permute.hpp"

namespace qmoe {

constexpr int kPermBlock = 1024;
constexpr int kPermLds = 15872;  // ints of LDS for hist/cursors (62 KiB)
// 64-chunks of ids a wave loads at once: 24 cover a 2048-row chunk's 20480
// top-10 assignments over 16 waves, so each wave reads its ids once.
constexpr int kPermIdBatch = 24;

__global__ __launch_bounds__(kPermBlock) void permute_kernel(const int32_t* ids, int A, int E,
                                                             int W, int nbits,
                                                             int32_t* offsets, int32_t* perm,
                                                             int32_t* inv) {
  __shared__ int hist[kPermLds];  // [W][E]
  __shared__ int wsum[kPermBlock / 64];
  permute_block<kPermBlock, kPermIdBatch>(ids, A, E, W, nbits, offsets, perm, inv, hist, wsum);
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
  const int W = permute_waves(A, E, kPermLds, kPermBlock / 64);
  return QMOE_LAUNCH("permute", permute_kernel, dim3(1), kPermBlock, 0, (hipStream_t)stream,
                     ids, (int)A, E, W, id_bits(E), offsets, perm, inv_perm);
}
