"""MXFP8 activations for the block-scaled matrix-core GEMM of MXFP4 weights.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Reading.  The "RTX 4080 SUPER native Windows 27B: NInfer 80 SM port" page
(its list of hardware limits) names 4-bit weight and activation matrix ops
(NVFP4, W4A4) as a tensor-core feature the sm_89 line lacks, so the 4-bit
tier there dequantizes on chip instead.  CDNA4's scaled matrix-core ops take
block-scaled FP8/FP6/FP4 operands with one E8M0 scale per 32 values along K
(OCP Microscaling Formats specification v1.0), and the two operands may use
different element types.  This build keeps MXFP4 weights as stored and
quantizes the activations to MXFP8 with E4M3 elements, the least lossy
element type that instruction takes; the product is then the exact sum of
(weight) x (quantized activation) terms.

E4M3 (OCP MX v1.0, FP8 E4M3): bit 7 sign, bits 6..3 exponent (bias 7),
bits 2..0 mantissa; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111
is NaN; there are no infinities; the largest magnitude is 448 (code 0x7E).

Quantizer, per 32 consecutive values along K:
  * amax = max |x|; shared exponent E = floor(log2 amax) - 8 (8 is E4M3's
    largest exponent), stored as the E8M0 byte E + 127 clamped to [0, 254];
    an all-zero block stores 0;
  * element code = the E4M3 value nearest to |x| / 2^E, ties to the even
    code, saturating at 448 (the OCP saturating conversion), sign bit set
    for x < 0.
|x| / 2^E lies in [256, 512) for the block's largest value, so values above
448 * 2^E clip to it (at most 12.5 % low); smaller values keep 4 significant
bits, so every value is within 2^-4 of itself relative, down to the E4M3
subnormal step 2^(E - 9).
"""
import numpy as np

from . import formats as fm

E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e4m3_value(code):
    """float64 value of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes in increasing order of value
_GRID = e4m3_value(np.arange(E4M3_MAX_CODE + 1))


def e4m3_code_of_magnitude(m):
    """Nearest non-negative E4M3 code for m >= 0, ties to the even code,
    saturating at 448."""
    m = np.asarray(m, dtype=np.float64)
    hi = np.clip(np.searchsorted(_GRID, m, side="left"), 1, E4M3_MAX_CODE)
    lo = hi - 1
    dl, dh = m - _GRID[lo], _GRID[hi] - m
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(m >= E4M3_MAX, E4M3_MAX_CODE, code)
    return code.astype(np.uint8)


def quantize_mxfp8(X):
    """X [R, K] (K % 32 == 0) -> (codes [R, K] uint8, scales [R, K/32] uint8)."""
    X = np.asarray(X, dtype=np.float64)
    R, K = X.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    x = X.reshape(R, K // 32, 32)
    amax = np.abs(x).max(axis=-1)
    _, ex = np.frexp(amax)                      # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, np.clip(127 + (ex - 1) - 8, 0, 254), 0).astype(np.int64)
    scaled = np.abs(x) / np.ldexp(1.0, e - 127)[..., None]
    code = e4m3_code_of_magnitude(scaled) | np.where(x < 0, 0x80, 0).astype(np.uint8)
    return code.reshape(R, K).astype(np.uint8), e.astype(np.uint8)


def dequantize_mxfp8(codes, scales):
    codes = np.asarray(codes)
    R, K = codes.shape
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return e4m3_value(codes) * np.repeat(s, 32, axis=1)


def mx_gemm(W, N, K, X):
    """y [R, N] = deq(W) deq(q(X))^T for MXFP4 weights W (packed bytes) and
    activations X [R, K] quantized to MXFP8, in float64 (every product is
    exact), with the parity bound sum_k |w x_q| per output."""
    xq = dequantize_mxfp8(*quantize_mxfp8(X))
    w = fm.dequantize("mxfp4", W, N, K)
    return xq @ w.T, np.abs(xq) @ np.abs(w).T


def mx_expert_ffn(gbuf, ubuf, dbuf, H, F, X):
    """One MXFP4/MXFP4 expert on the block-scaled path: g = W_g q(x),
    u = W_u q(x), h = SiLU(g) u, o = W_d q(h), q = quantize_mxfp8 along the
    inner dimension; returns o [R, H] and the bound sum_j |w_d[n, j] q(h)_j|.
    Composed of mx_gemm and quantize_mxfp8 (pinned above) and SiLU."""
    g, _ = mx_gemm(gbuf, F, H, X)
    u, _ = mx_gemm(ubuf, F, H, X)
    h = g / (1.0 + np.exp(-g)) * u
    return mx_gemm(dbuf, H, F, h)
