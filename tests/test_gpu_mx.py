"""MXFP8 activation quantizer (bit-exact) and the block-scaled MXFP4 x MXFP8
GEMM (exact-grid bit-exact; random data within the parity bound) against the
oracle."""
import numpy as np
import pytest

from gpu_util import requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound, torch
from oracle import formats as fm
from oracle import mx
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _cases():
    rng = np.random.default_rng(0)
    yield "normal", rng.normal(0, 1, (7, 2048)).astype(np.float32)
    yield "scaled rows", (rng.normal(0, 1, (9, 96)) * np.exp2(rng.integers(-40, 40, (9, 1)))).astype(np.float32)
    x = np.zeros((6, 64), np.float32)
    x[0, :32] = 1.0                                  # exact powers of two
    x[1, 0] = 1.99                                   # saturates at 448 * 2^-8
    x[1, 1:32] = rng.uniform(-1, 1, 31)
    x[2, 0], x[2, 1] = 256.0, 1.0625                 # tie: 1.0625 * 2^0 -> even code
    x[2, 2], x[2, 3] = 1.1875, -1.1875
    x[3, 0], x[3, 1:8] = 1.0, np.float32(2.0 ** -15) * np.arange(1, 8)   # E4M3 subnormals
    x[4, 32:] = -0.0                                 # zero block of negative zeros
    x[5] = rng.uniform(-3e-38, 3e-38, 64)            # amax near the fp32 normal floor
    yield "special", x
    # every E4M3 value times its block scale, plus the midpoints between them
    grid = mx.e4m3_value(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids, -mids])
    pad = (-len(vals)) % 31
    vals = np.concatenate([vals, np.zeros(pad)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((vals.shape[0], 1), 448.0), vals], axis=1)  # pin E = 0
    yield "grid and midpoints", (blocks.reshape(1, -1) * 2.0 ** -3).astype(np.float32)


@pytest.mark.parametrize("name,x", list(_cases()), ids=[c[0] for c in _cases()])
def test_activation_quantizer_bitexact(name, x):
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    rc, rs = mx.quantize_mxfp8(x.astype(np.float64))
    assert (to_np(scales) == rs).all(), name
    got = to_np(codes)
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{name}: {len(bad)} codes differ, first {tuple(bad[0])}: {got[tuple(bad[0])]:#x} vs {rc[tuple(bad[0])]:#x}"


def test_activation_quantizer_bf16_input():
    x = synth.bf16_round(synth.normal((5, 256), 1.0, 3, synth.ACT, 5))
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x).to(torch.bfloat16))
    rc, rs = mx.quantize_mxfp8(x.astype(np.float64))
    assert (to_np(codes) == rc).all() and (to_np(scales) == rs).all()


def _w(N, K, seed, sigma=0.02):
    return synth.normal((N, K), sigma, seed, synth.GATE, 0)


@pytest.mark.parametrize("N,K,R", [(16, 128, 16), (48, 256, 33), (130, 384, 70)])
def test_gemm_exact_grid_bitexact(N, K, R):
    """Weights with E8M0 = 127 (unit scale) and activation codes on a coarse
    grid with unit scales: every product and every partial sum is exact in
    fp32, so any summation order gives the oracle's value exactly (this also
    pins the operand layout: a wrong pairing of K positions changes sums)."""
    rng = np.random.default_rng(N + K + R)
    wcodes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    buf = fm.pack("mxfp4", {"q": wcodes, "e": np.full((N, K // 32), 127, np.uint8)}, N, K)
    # zero or E4M3 values 1 .. 3.75 (steps of 1/8), both signs: products are
    # multiples of 1/16 below 23, sums stay below 2^14
    acodes = np.where(rng.random((R, K)) < 0.2, 0, rng.integers(0x38, 0x48, (R, K)))
    acodes = (acodes | (rng.integers(0, 2, (R, K)) << 7)).astype(np.uint8)
    ascales = np.full((R, K // 32), 127, np.uint8)
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, to_gpu(acodes), to_gpu(ascales)))
    ref = mx.dequantize_mxfp8(acodes, ascales) @ fm.dequantize("mxfp4", buf, N, K).T
    assert_bitexact(y, ref, f"exact grid {N}x{K} R={R}")


@pytest.mark.parametrize("N,K,R", [(640, 2048, 40), (2048, 640, 33), (130, 384, 70), (16, 128, 1),
                                   (256, 1024, 129)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_gemm_within_bound(N, K, R, x_dtype):
    x = synth.normal((R, K), 1.0, 7, synth.ACT, R)
    if x_dtype == "bf16":
        x = synth.bf16_round(x)
    W = _w(N, K, 11)
    buf = fm.quantize("mxfp4", W)
    xg = to_gpu(x) if x_dtype == "f32" else to_gpu(x).to(torch.bfloat16)
    codes, scales = qmoe.quantize_act_mxfp8(xg)
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, codes, scales))
    ref, bound = mx.mx_gemm(buf, N, K, x.astype(np.float64))
    assert_within_bound(y, ref, bound, what=f"mx gemm {N}x{K} R={R}")


def test_gemm_full_size_sampled_columns():
    """A Llama-size MXFP4 matrix [14336, 4096] against 256 rows: the oracle
    checks 48 sampled output columns (MXFP4 quantizes each weight row on its
    own, so the sampled rows' bytes are the full matrix's)."""
    N, K, R = 14336, 4096, 256
    W = synth.normal_device((N, K), 0.02, 3, synth.UP, 0, "cuda")
    buf = qmoe.quantize("mxfp4", W)
    x = synth.normal((R, K), 1.0, 9, synth.ACT, 1)
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    y = to_np(qmoe.gemm_mxfp4_mxfp8(buf, N, K, codes, scales))
    cols = np.sort(np.random.default_rng(4).choice(N, 48, replace=False))
    Wc = to_np(W[torch.from_numpy(cols).cuda()])
    ref, bound = mx.mx_gemm(fm.quantize("mxfp4", Wc), len(cols), K, x.astype(np.float64))
    assert_within_bound(y[:, cols], ref, bound, what="mx gemm 14336x4096 sampled")


def test_quantized_activation_error_against_fp_activations():
    """Context, not parity: the MXFP8 activations move each output by a few
    parts in a thousand of sum |w x| against the unquantized product."""
    N, K, R = 640, 2048, 64
    x = synth.normal((R, K), 1.0, 5, synth.ACT, 2)
    buf = fm.quantize("mxfp4", _w(N, K, 12))
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, codes, scales))
    w = fm.dequantize("mxfp4", buf, N, K)
    exact = x.astype(np.float64) @ w.T
    rel = np.abs(y - exact) / (np.abs(x) @ np.abs(w).T)
    assert rel.max() < 2e-2 and np.median(rel) < 2e-3
