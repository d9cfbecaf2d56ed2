"""Int8 activations for integer dot products against Q8_0 weights.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The "RTX 4080 SUPER native Windows 27B: NInfer 80 SM port" page (its note on
the int8 artifact and section 八.2-3) quantizes the activations to int8 so
that both GEMM operands are integers: decode takes dp4a-class dot products,
prefill the int8 tensor cores; it gives no block size or rounding rule.
Reading (the plainest one the Q8_0 weights suggest, and the 32-value
activation blocks of the same GGUF family): per 32 consecutive values along
K,
  * d = max|x| / 127, an fp32 division of the fp32 values;
  * q = round-half-away-from-zero(x / d) (fp32 division), clamped to
    [-127, 127]; an all-zero block has d = 0 and q = 0.
Both divisions are taken in fp32 (IEEE, correctly rounded), as the kernel
takes them, so the integer codes are one decision on both sides.

The product with a Q8_0 row is then exact block by block:
  y[r, n] = sum_b  d_w[n, b] * d[r, b] * sum_{k in b} q_w[n, k] q[r, k]
(the integer sums are exact; float64 here).
"""
import numpy as np

from . import formats as fm


def quantize_act_q8(X):
    """X [R, K] (K % 32 == 0), float32 values -> (q [R, K] int8, d [R, K/32] float32)."""
    X = np.asarray(X, dtype=np.float32)
    R, K = X.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    x = X.reshape(R, K // 32, 32)
    amax = np.abs(x).max(axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d[..., None] > 0, x / d[..., None], np.float32(0)).astype(np.float32)
    q = np.clip(fm.round_half_away(r.astype(np.float64)), -127, 127)
    return q.reshape(R, K).astype(np.int8), d


def dequantize_act_q8(q, d):
    return np.asarray(q, np.float64) * np.repeat(np.asarray(d, np.float64), 32, axis=1)


def gemv_q8_0_i8(W, N, K, X):
    """y [R, N] for Q8_0 weights W (packed bytes) against the int8-quantized
    activations of X [R, K], with the parity bound sum_k |w x_q|."""
    q, d = quantize_act_q8(X)
    f = fm.unpack("q8_0", W, N, K)
    qw = np.asarray(f["q"], np.int64).reshape(N, K // 32, 32)
    dw = np.asarray(f["d"], np.float64).reshape(N, K // 32)
    qx = np.asarray(q, np.int64).reshape(-1, K // 32, 32)
    isum = np.einsum("nbk,rbk->rnb", qw, qx)            # exact integers
    y = np.einsum("rnb,nb,rb->rn", isum.astype(np.float64), dw, d.astype(np.float64))
    xq = dequantize_act_q8(q, d)
    w = fm.dequantize("q8_0", W, N, K)
    return y, np.abs(xq) @ np.abs(w).T
