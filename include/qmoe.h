/*
 * qmoe.h -- C ABI of libqmoe.so: quantized-weight decode and routed-expert
 * (mixture-of-experts) layer kernels for AMD MI355X (gfx950), in HIP.
 *
 * What the path computes comes from these pages (cited by title + section):
 *  [P2] "三张 RTX 3090 显卡实现 Qwen3.8-Flash-Next 80 Token 每秒的高效推理优化指南"
 *       (n1n.ai): a 512-expert, top-10 MoE layer ("瓶颈分析"); experts re-indexed
 *       by selection frequency so a precision tier is a contiguous id range
 *       ("优化策略一"); per-tier formats Q6_K/Q8_0, 4-bit, MXFP4 ("优化策略二");
 *       the routed matmul skips ids outside a tier's [min, max) range
 *       ("优化策略三", kernel k_mul_mat_id_tiered); -1 skip sentinels must never
 *       be dereferenced and gate/up/activation are fused in decode
 *       ("关键 Bug 修复与调试踩坑记录", items 1, 3, 4).
 *  [P3] "一张 RTX 3090 跑 Llama 70B：三层流式缓存 + NVMe 直连，速度干到 83 倍":
 *       GGUF formats Q4_0, Q8_0, Q4_K, Q6_K (section 一); hand-written GEMV for
 *       single-token decode and SwiGLU fused with the FC (section 4.4).
 *  [P4] "多卡 CUDA 张量并行DwarfStar 如何在 8 张 L40S 上跑出 120 t/s": one kernel
 *       launch serves 16 sessions' decode rows over Q4_K routed experts, with
 *       a Q8 shared expert; prefill in 2048-token chunks
 *       ("120 t/s 的秘密微批次分组解码", "快速上手").
 *  [P1] "RTX 4080 SUPER 原生 Windows 跑 27B:NInfer 80 SM 移植实录": launch
 *       geometry must follow the device's compute-unit count (sections 三, 四);
 *       a bad memory plan must fail up front, not mid-run (section 五).
 *
 * Conventions (every entry point):
 *  - All tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps caller memory.  Scratch space is a
 *    caller-provided device workspace of at least *_workspace_size() bytes.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    only enqueue work: no host synchronisation, no allocation, no memset, so
 *    they may be captured in a HIP graph.
 *  - Return 0 (QMOE_OK) or a negative qmoe_status.  All argument checks run on
 *    the host before anything is launched; a failed call launches nothing.
 *    qmoe_last_error() gives the detail text of the calling thread's last
 *    failure.
 *  - Sizes are int; a row count of 0 is a valid no-op.  Matrices are
 *    row-major.  Activations are fp32 (QMOE_F32) or bf16 (QMOE_BF16, raw
 *    uint16 storage); outputs are fp32.
 *  - Quantized weight tensors use the plane layout below.  Weight and
 *    workspace pointers must be 256-byte aligned; activation/output pointers
 *    16-byte aligned.
 *  - Device-side routing ids outside [0, E) (including the -1 sentinel) are
 *    skipped: they contribute nothing and index nothing.
 *  - Determinism: no floating-point atomics; repeated calls on the same
 *    inputs give bit-identical results.
 *
 * Weight layout ("planes").  W[N, K] is quantized along K in blocks of B
 * values (nb = K / B per row).  Each per-block field is a plane, row-major
 * [N][nb][field bytes]; planes follow in the order listed, each starting at a
 * 256-byte aligned offset; qmoe_tensor_bytes() gives the total.
 *   Q8_0  B=32  : q int8[32]; d fp16.                      value d*q
 *   Q4_0  B=32  : q 4-bit[32]; d fp16.                     value d*(q-8)
 *   MXFP4 B=32  : q E2M1[32]; e uint8 (E8M0).              value 2^(e-127)*E2M1(q)
 *   Q4_K  B=256 : q 4-bit[256]; meta 16 B = fp16 d, fp16 dmin, 96-bit LE field
 *                 with sc_j at bits 6j.., m_j at bits 48+6j.. (j=0..7, 32-value
 *                 sub-blocks).                             value d*sc_j*q - dmin*m_j
 *   Q6_K  B=256 : ql 4-bit[256]; qh 2-bit[256]; sc int8[16]; d fp16 (16-value
 *                 sub-blocks).                             value d*sc_j*(q-32)
 *   T5    B=128 : one plane of 28-byte groups: 26 base-3 code bytes, then
 *                 fp16 d.  Weight i of a group is digit i mod 5 (least
 *                 significant first) of code byte i div 5, holding t + 1;
 *                 byte 25 holds weights 125..127 (digits 3, 4 are t = 0).
 *                 1.75 bits per weight.                    value d*t, t in {-1,0,1}
 *                 ("t5_g128_fp16" of [P1] section 九.2: base-3, five weights
 *                 per byte, one FP16 scale per 128 weights.)
 *   4-bit element i of a row: byte i>>1, low nibble for even i.  Q6_K high
 *   bits of element i: byte i>>2, bits 2*(i&3).  E2M1: bit3 sign, bits 2-1
 *   exponent, bit 0 mantissa, magnitudes {0,.5,1,1.5,2,3,4,6} (OCP MX v1.0).
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 1
#define QMOE_MAX_TIERS 8

typedef enum {
  QMOE_OK = 0,
  QMOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, k > E ... */
  QMOE_ERR_UNSUPPORTED = -2, /* unknown format or dtype, size beyond a limit  */
  QMOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required    */
  QMOE_ERR_HIP = -4          /* the HIP runtime reported an error             */
} qmoe_status;

typedef enum {
  QMOE_Q8_0 = 0,
  QMOE_Q4_0 = 1,
  QMOE_MXFP4 = 2,
  QMOE_Q4_K = 3,
  QMOE_Q6_K = 4,
  QMOE_T5 = 5 /* ternary, dense GEMV only (not a tier format) */
} qmoe_format;

typedef enum { QMOE_F32 = 0, QMOE_BF16 = 1 } qmoe_dtype;

/* ---------------------------------------------------------------- meta -- */
int qmoe_abi_version(void);
const char *qmoe_status_string(int status);
/* Detail text of the calling thread's most recent failing call ("" if none). */
const char *qmoe_last_error(void);
/* Block size B of a format (32 or 256), or 0 for an unknown format. */
int qmoe_block_size(int fmt);  /* 128 for QMOE_T5 */
/* Bytes of a packed [N, K] tensor; 0 if fmt is unknown or K % B != 0. */
size_t qmoe_tensor_bytes(int fmt, int N, int K);
/* Byte offset of each plane of a packed [N, K] tensor (up to 4 planes).
 * Returns the number of planes, or a negative status. */
int qmoe_plane_offsets(int fmt, int N, int K, size_t offsets[4]);
/* Compute units of the current device (the launch geometry is sized from it). */
int qmoe_device_cu_count(void);

/* ---------------------------------------------------- block formats ----
 * qquantize_<fmt>: w [N, K] fp32 -> packed tensor `out` (qmoe_tensor_bytes
 *   bytes).  Quantization rule per block (float64 arithmetic on the fp32
 *   inputs; scales rounded to fp16 nearest-even; codes against the stored
 *   scale; code rounding half away from zero, then clamped; zero divisor ->
 *   code offset only):
 *     Q8_0 : d = fp16(max|w|/127); q = clamp(round(w/d), -127, 127)
 *     Q4_0 : d = fp16(max|w|/7);   q = clamp(round(w/d) + 8, 0, 15)
 *     MXFP4: e = clamp(127 + floor(log2 max|w|) - 2, 0, 254) (0 for an
 *            all-zero block); codes = E2M1 round-to-nearest-even of
 *            w / 2^(e-127), saturating at 6; sign bit = (w < 0)
 *     Q4_K : per 32-sub-block lo = min(0, min w), s = (max w - lo)/15,
 *            m' = 0 - lo; d = fp16(max s/63), dmin = fp16(max m'/63),
 *            sc = clamp(round(s/d),0,63), m = clamp(round(m'/dmin),0,63),
 *            q = clamp(round((w + dmin*m)/(d*sc)), 0, 15)
 *     Q6_K : per 16-sub-block s = max|w|/31; d = fp16(max s/127),
 *            sc = clamp(round(s/d),-128,127), q = clamp(round(w/(d*sc))+32,0,63)
 *     T5   : per 128-group d = fp16(mean|w|), t = clamp(round(w/d), -1, 1)
 *   (the offline per-tier packing of [P2] "优化策略二", done on the device).
 * qdequant_<fmt>: packed [N, K] -> out [N, K] fp32, each value the exact
 *   format value rounded to nearest-even fp32 (bit-exact reference decoder).
 * qgemv_<fmt>: y[r, n] = sum_k deq(W)[n, k] * x[r, k] for r < R, n < N
 *   ([P3] section 4.4 GEMV operator).  x is [R, K] of x_dtype, y is [R, N]
 *   fp32.  R >= 0 (R rows share one pass over W).  Activations are rounded to
 *   fp16 inside the dot product: |x| must stay below 65504.  Up to 4 rows
 *   (fewer for long K) run as fp16 dot products against the exact codes; more
 *   rows, or K > 27456, run on the matrix cores, also against the exact codes
 *   (the unit scale multiplies the fp32 result), so only the activations are
 *   rounded.
 * Errors: INVALID_ARG for null pointers, N or K < 0, K % B != 0, K > 65536,
 *   misalignment; UNSUPPORTED for an unknown x_dtype.                      */
#define QMOE_DECLARE_FORMAT(F)                                                 \
  int qquantize_##F(const float *w, int N, int K, void *out, void *stream);    \
  int qdequant_##F(const void *W, int N, int K, float *out, void *stream);     \
  int qgemv_##F(const void *W, int N, int K, const void *x, int x_dtype, int R, \
                float *y, void *stream);
QMOE_DECLARE_FORMAT(q8_0)
QMOE_DECLARE_FORMAT(q4_0)
QMOE_DECLARE_FORMAT(mxfp4)
QMOE_DECLARE_FORMAT(q4_k)
QMOE_DECLARE_FORMAT(q6_k)
#undef QMOE_DECLARE_FORMAT
/* T5 (ternary): qquantize_t5, qdequant_t5 as above.  qgemv_t5 as qgemv_<fmt>
 *   with 1 <= R <= 16: code bytes are decoded to ternary fp16 pairs in
 *   registers and dotted with fp16-rounded activations (|x| < 65504), so the
 *   products are exact and only the activations are rounded.  Code bytes
 *   above 242 are not produced by qquantize_t5 and give unspecified values.
 *   ([P1] section 九.2: ternary decode is memory-bound.)
 * Limits: K <= 20096 (one staged activation row fits in LDS; UNSUPPORTED
 *   beyond).
 * Errors: as qgemv_<fmt>; INVALID_ARG for K % 128 != 0 or R > 16.          */
int qquantize_t5(const float *w, int N, int K, void *out, void *stream);
int qdequant_t5(const void *W, int N, int K, float *out, void *stream);
int qgemv_t5(const void *W, int N, int K, const void *x, int x_dtype, int R,
             float *y, void *stream);

/* qgemv_batch: y_i = deq(W_i) x_i for n independent matrices in one launch
 *   (the dense layer's matrices of [P3] section 4.4 streamed back to back
 *   instead of one launch each).  descs[i] holds what qgemv_<fmt> takes for
 *   matrix i (fmt one of QMOE_Q8_0 .. QMOE_Q6_K); every y_i equals that
 *   qgemv call's result bit for bit.  No y_i may overlap any W_j, x_j or y_j.
 *   descs is host memory, read during the call only.  A matrix with N == 0
 *   or R == 0 is skipped (its pointers may be NULL).
 * Limits: 0 <= n <= QMOE_MAX_BATCH; per matrix as qgemv, and R <= 16.
 * Errors: as qgemv, for the first offending matrix; INVALID_ARG for n out of
 *   range or null descs (n > 0).                                           */
#define QMOE_MAX_BATCH 16
typedef struct qmoe_gemv_desc {
  int32_t fmt, N, K, x_dtype, R, reserved;
  const void *W; /* device, 256-byte aligned, qmoe_tensor_bytes(fmt, N, K) */
  const void *x; /* device [R, K] of x_dtype, 16-byte aligned */
  float *y;      /* device [R, N] fp32 */
} qmoe_gemv_desc;
int qgemv_batch(const qmoe_gemv_desc *descs, int n, void *stream);

/* ----------------------------------------------------------- routing ----
 * moe_route ([P2] "瓶颈分析": a light router picks the top-k of E experts per
 * token):
 *   logits[t, e] = sum_h x[t, h] * Wr[e, h] + bias[e]   (fp32 accumulation)
 *   ids[t, 0..k-1] = the k largest logits, descending, ties to the lower id
 *                    (NaN ranks below every number)
 *   p[t, i] = exp(l_i - l_0) / sum_j exp(l_j - l_0) over the kept k
 *   ids[t, k+s] = E + s and p[t, k+s] = 1 for s < n_shared (always-on shared
 *   experts, [P4] "快速上手": Q8 shared expert)
 * x [T, H] (x_dtype), Wr [E, H] fp32, bias [E] fp32 or NULL, ids/p
 * [T, k+n_shared] int32/fp32, logits [T, E] fp32 or NULL (written when given).
 * Limits: 1 <= k <= min(E, 64), E <= 4096, n_shared >= 0.
 * Workspace: moe_route_workspace_size(T, H, E) bytes.                       */
size_t moe_route_workspace_size(int T, int H, int E);
int moe_route(const void *x, int x_dtype, int T, int H, const float *Wr,
              const float *bias, int E, int k, int n_shared, int32_t *ids,
              float *p, float *logits, void *ws, size_t ws_bytes, void *stream);

/* moe_route_decode: moe_route followed by moe_permute(ids, T, k + n_shared,
 * E + n_shared, offsets, perm, inv_perm) in a single launch, for decode rows.
 * Outputs (ids, p, logits when not NULL, offsets, perm, inv_perm) are
 * identical to those two calls, bit for bit.  Inside the launch the block that
 * finishes last (a device-scope counter in the workspace decides) sums the
 * split-K router partials, takes the top-k of every row and sorts the
 * assignments, so the routing of a decode step is one launch instead of three.
 * Limits: as moe_route, plus T <= 16, E <= 512 and
 * round_up(T*(k+n_shared), 64) + E + n_shared <= 8176 (UNSUPPORTED beyond).
 * T == 0 writes zero offsets and nothing else.
 * Workspace: moe_route_decode_workspace_size(T, H, E) bytes, 256-byte
 * aligned, whose first 256 bytes must be zero before the first call that uses
 * it; every call leaves them zero again.  Calls sharing one workspace must not
 * run concurrently.  */
size_t moe_route_decode_workspace_size(int T, int H, int E);
int moe_route_decode(const void *x, int x_dtype, int T, int H, const float *Wr,
                     const float *bias, int E, int k, int n_shared, int32_t *ids,
                     float *p, float *logits, int32_t *offsets, int32_t *perm,
                     int32_t *inv_perm, void *ws, size_t ws_bytes, void *stream);

/* moe_route_decode_noalloc: moe_route_decode without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments and outputs as moe_route_decode, bit for bit, minus ws and
 * ws_bytes: the split-K partials and the block counter live in a
 * library-owned device array of moe_route_decode_noalloc_max_bytes() bytes
 * (1 MiB) per GPU, held until the process ends.  The call allocates nothing
 * (no hipMalloc, no memset); the first successful call on a GPU clears the
 * counter with one small kernel, and every call leaves it at zero.  All calls
 * on one GPU share that array: calls that overlap on one GPU (other streams,
 * other threads) race and must not be issued.
 * Errors: as moe_route_decode; UNSUPPORTED when
 * moe_route_decode_workspace_size(T, H, E) exceeds the array.               */
size_t moe_route_decode_noalloc_max_bytes(void);
int moe_route_decode_noalloc(const void *x, int x_dtype, int T, int H,
                             const float *Wr, const float *bias, int E, int k,
                             int n_shared, int32_t *ids, float *p, float *logits,
                             int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                             void *stream);

/* moe_permute: stable counting sort of the flat assignments a = t*k + i by
 * expert id ([P2] "优化策略三" groups a layer's routed tokens by expert; bug
 * item 1 shows grouping must survive duplicate ids).
 *   offsets[e] = number of valid assignments with id < e, e = 0..E
 *   perm[pos]  = a, in ascending a within each expert, for pos < offsets[E];
 *                -1 for pos >= offsets[E]
 *   inv_perm[a] = pos, or -1 when ids[a] is outside [0, E)
 * ids [T*k] int32 (any values); offsets [E+1], perm [T*k], inv_perm [T*k].
 * Limits: E <= 8192, T*k <= 1<<24.  No workspace.                           */
int moe_permute(const int32_t *ids, int T, int k, int E, int32_t *offsets,
                int32_t *perm, int32_t *inv_perm, void *stream);

/* ------------------------------------------------------- expert FFN ----
 * A tier is a contiguous expert-id range with one format for gate/up and one
 * for down ([P2] "优化策略二", "优化策略三").  Its experts are stored back to
 * back: expert e's gate tensor [F, H] starts at
 *   gate + (e - e_begin) * qmoe_tensor_bytes(fmt_gate_up, F, H),
 * and likewise up [F, H] and down [H, F] (stride qmoe_tensor_bytes(fmt_down,
 * H, F)).  Tiers must be disjoint; together they cover [0, E).               */
typedef struct qmoe_tier {
  int32_t e_begin, e_end; /* expert ids [e_begin, e_end)        */
  int32_t fmt_gate_up;    /* qmoe_format of gate and up [F, H]  */
  int32_t fmt_down;       /* qmoe_format of down [H, F]         */
  const void *gate, *up, *down;
} qmoe_tier;

/* moe_ffn_tiered (decode rows): for every valid permuted position pos
 * (pos < offsets[E]) with expert e and token t = perm[pos] / k:
 *   g = deq(Wg_e) x_t,  u = deq(Wu_e) x_t,  h = g / (1 + exp(-g)) * u,
 *   o[pos, :] = deq(Wd_e) h                                (fp32 [T*k, H])
 * ([P2] bug item 4: gate, up and activation fused; [P3] 4.4: SwiGLU fused).
 * All tiers run in the same launches; rows o[pos] for pos >= offsets[E] are
 * not written.  offsets/perm are moe_permute's.  x as in moe_route; |x| and
 * |h| must stay below 65504 (fp16 inside the dot products).  An expert with
 * more rows than the dot-product blocking (1, 2 or 4 rows, set by T and by
 * how many staged rows of length H or F fit in 96 KB of LDS) runs on the
 * matrix cores against the exact weight codes (the unit scale multiplies
 * the fp32 result), so only the activations are rounded, as in qgemv.
 * Limits: n_tiers <= QMOE_MAX_TIERS; H, F <= 65536.
 * Workspace: moe_ffn_workspace_size(T, k, F) bytes.                         */
size_t moe_ffn_workspace_size(int T, int k, int F);
int moe_ffn_tiered(const qmoe_tier *tiers, int n_tiers, int E, int H, int F,
                   const void *x, int x_dtype, int T, int k,
                   const int32_t *offsets, const int32_t *perm, float *o,
                   void *ws, size_t ws_bytes, void *stream);

/* qgemm_grouped_prefill: the same result as moe_ffn_tiered for long chunks
 * (a 2048-token prefill chunk, [P4] "120 t/s 的秘密微批次分组解码"): per
 * expert, rows are cut into tiles of 128; each tile's weights are
 * dequantized to fp16 in registers (the exact code times its block scale,
 * rounded once) and multiplied on the matrix cores against the tile's
 * activations with fp32 accumulation ([P1] section 九.3).  x is rounded to
 * fp16 once (|x| must stay below 65504) and h = SiLU(g) * u is stored as
 * fp16 between the gate/up pass and the down pass.  Same arguments as
 * moe_ffn_tiered; H and F must be multiples of 64.
 * Workspace: qgemm_grouped_prefill_workspace_size(T, k, E, H, F) bytes:
 * h [T*k, F] fp16, x [T, H] fp16, the tile table, and the MXFP8 copies of x
 * and h used by qgemm_grouped_prefill_mx.                                   */
size_t qgemm_grouped_prefill_workspace_size(int T, int k, int E, int H, int F);
int qgemm_grouped_prefill(const qmoe_tier *tiers, int n_tiers, int E, int H,
                          int F, const void *x, int x_dtype, int T, int k,
                          const int32_t *offsets, const int32_t *perm, float *o,
                          void *ws, size_t ws_bytes, void *stream);

/* qgemm_grouped_prefill_mx: qgemm_grouped_prefill, except that every tier
 * whose gate/up and down are both MXFP4 runs on the gfx950 block-scaled matrix
 * cores ([P1] "NInfer 80 SM port", list of hardware limits): its weights are
 * used as stored, x is quantized to MXFP8 as qquantize_act_mxfp8 does, and
 * h = SiLU(g) * u (fp32 from the matrix cores) is quantized the same way
 * along F before the down projection.  Other tiers give the same o as
 * qgemm_grouped_prefill, bit for bit.  Same arguments and workspace.        */
int qgemm_grouped_prefill_mx(const qmoe_tier *tiers, int n_tiers, int E, int H,
                             int F, const void *x, int x_dtype, int T, int k,
                             const int32_t *offsets, const int32_t *perm,
                             float *o, void *ws, size_t ws_bytes, void *stream);

/* moe_combine: y[t, :] = sum_{i<k} p[t, i] * o[inv_perm[t*k + i], :]
 *                        + shared[t, :]
 * summed in slot order i = 0..k-1 (slots with inv_perm < 0 skipped), shared
 * added last when not NULL ([P2] "瓶颈分析": weighted sum of the selected
 * experts).  o [*, H] fp32 (permuted rows), p [T, k] fp32, y [T, H] fp32.
 * Limit: H % 4 == 0.                                                         */
int moe_combine(const float *o, const int32_t *inv_perm, const float *p, int T,
                int k, int H, const float *shared, float *y, void *stream);

/* ---------------------------------------------- block-scaled MX GEMM ----
 * MXFP4 weights multiplied on the gfx950 block-scaled matrix cores, without
 * dequantization ([P1] "NInfer 80 SM port", list of hardware limits: 4-bit
 * weight x low-precision activation matrix ops are what its GPU lacks).  The
 * activations are quantized once to MXFP8 (OCP Microscaling v1.0, E4M3
 * elements, one E8M0 scale per 32 values along K):
 *   E = floor(log2 max|x|) - 8 per block, stored as E + 127 clamped to
 *   [0, 254] (0 for an all-zero block); code = nearest E4M3 value to
 *   |x| / 2^E, ties to even, saturating at 448, sign of x.
 * qquantize_act_mxfp8: x [R, K] (x_dtype) -> codes [R, K] (E4M3 bytes) and
 * scales [R, K/32] (E8M0 bytes).  K % 32 == 0; x and codes 16-byte aligned.
 * qgemm_mxfp4_mxfp8: y [R, N] fp32 = sum_k w[n, k] * xq[r, k] for MXFP4
 * weights W [N, K] (qmoe layout, 256-byte aligned) and MXFP8 activations as
 * qquantize_act_mxfp8 writes them; every product is exact, sums are fp32 in
 * the matrix cores.  K % 128 == 0; N*K and R*K < 2^32; codes 16-byte and
 * scales 4-byte aligned.                                                    */
int qquantize_act_mxfp8(const void *x, int x_dtype, int R, int K,
                        uint8_t *codes, uint8_t *scales, void *stream);
int qgemm_mxfp4_mxfp8(const void *W, int N, int K, const uint8_t *codes,
                      const uint8_t *scales, int R, float *y, void *stream);

/* ------------------------------------------- int8 activations, decode ----
 * Q8_0 weights against int8 activations with integer dot products ([P1]
 * "NInfer 80 SM port", its int8 artifact and section 八.2: decode quantizes
 * the activations to int8 and takes dp4a-class dot products).
 * qquantize_act_q8: x [R, K] (x_dtype) -> q [R, K] int8 and d [R, K/32] fp32:
 *   per 32 values d = max|x| / 127, q = round-half-away(x / d) clamped to
 *   [-127, 127] (fp32 divisions, correctly rounded; zero block: d = 0, q = 0).
 *   K % 32 == 0; x and q 16-byte aligned.
 * qgemv_q8_0_i8: y [R, N] fp32 = sum_b d_w[n, b] d[r, b] sum_{k in b} q_w q
 *   (exact int32 per 32-value block, then fp32) for Q8_0 W [N, K] (256-byte
 *   aligned).  R <= 16, K % 32 == 0.                                        */
int qquantize_act_q8(const void *x, int x_dtype, int R, int K, int8_t *q,
                     float *d, void *stream);
int qgemv_q8_0_i8(const void *W, int N, int K, const int8_t *q, const float *d,
                  int R, float *y, void *stream);

/* qgemm_q8_0_i8: the same product for prefill-sized R on the int8 matrix
 * cores ([P1] "NInfer 80 SM port", its int8 artifact: prefill on the int8
 * tensor cores with int8 activations, section 九 items 2-3):
 *   y [R, N] fp32 = sum_b (d_w[n, b] d[r, b]) * sum_{k in b} q_w q
 * with each block's integer sum exact (one v_mfma_i32_16x16x32_i8 per 16 x 16
 * tile and 32-value block) and the scaling and the sum over blocks in fp32.
 * W Q8_0 [N, K] (256-byte aligned), q [R, K] int8 (16-byte aligned), d
 * [R, K/32] fp32 as qquantize_act_q8 writes them.  K % 32 == 0; N*K and R*K
 * < 2^32.  Any R >= 0 (rows are tiled by 128).                            */
int qgemm_q8_0_i8(const void *W, int N, int K, const int8_t *q, const float *d,
                  int R, float *y, void *stream);

/* moe_layer_decode: the whole routed-expert layer of a decode step in one
 * launch ([P2] "瓶颈分析": router top-k over the experts, the selected
 * experts' SwiGLU FFNs, their weighted sum; "优化策略二/三": tiers of mixed
 * precision in one layer).  Computes what
 *   moe_route_decode(x, Wr, bias, E, k, n_shared) -> ids, p, offsets, perm,
 *   inv_perm;  moe_ffn_tiered(tiers, E + n_shared, H, F, x, T, k + n_shared)
 *   -> o;  moe_combine(o, inv_perm, p, T, k + n_shared, H, NULL) -> y
 * computes, with the same arithmetic: the outputs are equal bit for bit.  One
 * plain launch holds, in block-index order, the router blocks (the last of
 * them routes every row and publishes the routing), the gate/up blocks and
 * the down blocks of moe_ffn_tiered's schedule; each block waits only for the
 * data it reads (the routing, its expert's h), through counters in the
 * workspace, and the block that writes the last piece of a (token, 64-row
 * chunk) of y sums that chunk.  Blocks wait only on blocks of lower index.
 * Arguments: tiers cover ids [0, E + n_shared) (shared experts are ids E..,
 * always selected with weight 1); x [T, H] (x_dtype), Wr [E, H] fp32, bias [E]
 * fp32 or NULL; outputs ids/p [T, k+n_shared], offsets [E+n_shared+1], perm
 * and inv_perm [T*(k+n_shared)], y [T, H] fp32.  x, Wr and y 16-byte aligned.
 * Limits: T <= 16, 1 <= k <= min(E, 64), E <= 512, H % 4 == 0,
 * T*(k+n_shared) <= 1024 and 768 + 2*(E+n_shared) + T*ceil(H/64) <= 4096
 * (the counters), plus moe_ffn_tiered's (UNSUPPORTED beyond).  T == 0 writes
 * zero offsets and nothing else.
 * Workspace: moe_layer_decode_workspace_size(T, H, E, F, k, n_shared) bytes,
 * 256-byte aligned, whose first 16384 bytes (the counters) must be zero
 * before the first call that uses it; every call leaves them zero again.
 * A nonzero first word (uint32 at byte 0) after a call means a wait ran out
 * (about a second) and the outputs are invalid; the workspace must then be
 * zeroed again.  Calls sharing one workspace must not run concurrently. */
size_t moe_layer_decode_workspace_size(int T, int H, int E, int F, int k,
                                       int n_shared);
int moe_layer_decode(const qmoe_tier *tiers, int n_tiers, int E, int H, int F,
                     const void *x, int x_dtype, int T, const float *Wr,
                     const float *bias, int k, int n_shared, int32_t *ids,
                     float *p, int32_t *offsets, int32_t *perm,
                     int32_t *inv_perm, float *y, void *ws, size_t ws_bytes,
                     void *stream);

/* ------------------------------------------------------- measurement --
 * qmoe_stream_read: reads `bytes` of device memory at buf once
 * (blocks_per_cu * CUs blocks of 256 threads, each block on a contiguous
 * chunk of its own, 16-byte nontemporal vector loads, consecutive lanes on
 * consecutive pieces, eight loads in flight per lane; the remainder past the
 * equal chunks read grid-stride), and writes at most one word to
 * sink[0].  For measuring the HBM read rate the part sustains, the practical
 * ceiling of a weight stream ([P3] section 4.4: decode reads every weight
 * once per token).  buf 16-byte aligned, bytes % 16 == 0, 1 <= blocks_per_cu
 * <= 64; sink a device word.                                              */
int qmoe_stream_read(const void *buf, size_t bytes, int blocks_per_cu,
                     uint32_t *sink, void *stream);

/* qmoe_wave_latency: runs one 64-lane wave that times, with the shader clock,
 * the dependent steps a single wave per routed row works through in the decode
 * routing's tail (the top-k of [P2] "瓶颈分析": 10 of 512 experts per token):
 *   out[0] cycles per dependent vector op, out[1] per DPP wave max with its
 *   read-back to a scalar, out[2] per ballot round trip (compare, ballot,
 *   first set lane, read-lane), out[3] per top-k of 512 keys with k = 10 (the
 *   library's own wave top-k), out[4] per sort of a lane's 8 keys, out[5] the
 *   shader clock in MHz over the run, out[6] a value without meaning.
 * out: 8 device words (uint64), written by one thread.  For measurement only. */
int qmoe_wave_latency(uint64_t *out, void *stream);

/* ----------------------------------------------------------- profiling --
 * Optional per-kernel timing with HIP events recorded around every launch the
 * library makes while enabled (on the launch stream).  qmoe_profile_read
 * waits for the recorded events and returns, for the kernel named `name`,
 * the number of launches and their summed duration in milliseconds.
 * qmoe_profile_only(name) restricts recording to launches of that kernel
 * (NULL: all kernels); each recorded launch adds two event records to its
 * stream, so timing one kernel perturbs the others least.                   */
int qmoe_profile_enable(int on);
int qmoe_profile_only(const char *name);
int qmoe_profile_reset(void);
int qmoe_profile_read(const char *name, int *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
