"""Int8 activation quantizer (bit-exact) and the Q8_0 x int8 GEMV (exact-grid
bit-exact; random data within the parity bound) against the oracle."""
import numpy as np
import pytest

from gpu_util import requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound, torch
from oracle import formats as fm
from oracle import int8
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs():
    rng = np.random.default_rng(0)
    yield "normal", rng.normal(0, 1, (9, 4096)).astype(np.float32)
    yield "scaled rows", (rng.normal(0, 1, (5, 96)) * np.exp2(rng.integers(-60, 60, (5, 1)))).astype(np.float32)
    x = np.zeros((3, 64), np.float32)
    x[0, :6] = [127.0, -63.5, 0.5, -0.5, 1.49, 126.6]   # d = 1: halves go away from zero
    x[1, 32] = -2.54
    x[2, :32] = np.float32(1e-40) * np.arange(32)         # fp32 subnormals
    yield "special", x


@pytest.mark.parametrize("name,x", list(_inputs()), ids=[c[0] for c in _inputs()])
def test_act_quantizer_bitexact(name, x):
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    rq, rd = int8.quantize_act_q8(x)
    assert_bitexact(to_np(d), rd, f"{name} scales")
    assert (to_np(q) == rq).all(), name


def test_act_quantizer_bf16_input():
    x = synth.bf16_round(synth.normal((4, 512), 1.0, 2, synth.ACT, 3))
    q, d = qmoe.quantize_act_q8(to_gpu(x).to(torch.bfloat16))
    rq, rd = int8.quantize_act_q8(x)
    assert (to_np(q) == rq).all() and np.array_equal(to_np(d), rd)


@pytest.mark.parametrize("N,K,R", [(16, 128, 1), (70, 256, 5), (33, 1024, 16)])
def test_gemv_exact_grid_bitexact(N, K, R):
    """Weight scales 1 and activation rows whose block maximum is 127 (d = 1):
    every product and partial sum is an integer far below 2^24."""
    rng = np.random.default_rng(N + K)
    W = rng.integers(-127, 128, (N, K)).astype(np.float64)
    W[:, ::32] = 127.0                                     # d_w = 127 / 127 = 1
    buf = fm.quantize("q8_0", W)
    x = rng.integers(-20, 21, (R, K)).astype(np.float32)
    x[:, ::32] = 127.0                                     # d_x = 1
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    y = to_np(qmoe.gemv_q8_0_i8(to_gpu(buf), N, K, q, d))
    ref, _ = int8.gemv_q8_0_i8(buf, N, K, x)
    assert_bitexact(y, ref, f"exact grid {N}x{K} R={R}")


@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (4096, 14336), (130, 384), (64, 32)])
@pytest.mark.parametrize("R", [1, 2, 6, 16])
def test_gemv_within_bound(N, K, R):
    W = synth.normal((N, K), 0.02, 5, synth.GATE, N)
    buf = fm.quantize("q8_0", W)
    x = synth.normal((R, K), 1.0, 6, synth.ACT, R)
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    y = to_np(qmoe.gemv_q8_0_i8(to_gpu(buf), N, K, q, d))
    ref, bound = int8.gemv_q8_0_i8(buf, N, K, x)
    assert_within_bound(y, ref, bound, what=f"int8 gemv {N}x{K} R={R}")


def test_int8_activation_error_against_fp_activations():
    """Context, not parity: int8 activations move each output by a few parts
    in a thousand of sum |w x| against the unquantized product."""
    N, K, R = 1024, 4096, 8
    buf = fm.quantize("q8_0", synth.normal((N, K), 0.02, 7, synth.UP, 0))
    x = synth.normal((R, K), 1.0, 8, synth.ACT, 1)
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    y = to_np(qmoe.gemv_q8_0_i8(to_gpu(buf), N, K, q, d))
    w = fm.dequantize("q8_0", buf, N, K)
    rel = np.abs(y - x.astype(np.float64) @ w.T) / (np.abs(x) @ np.abs(w).T)
    assert rel.max() < 2e-2 and np.median(rel) < 2e-3


# ------------------------------------ int8 matrix cores (prefill rows) ----

@pytest.mark.parametrize("N,K,R", [(16, 32, 1), (70, 96, 33), (130, 384, 130), (257, 1024, 300)])
def test_gemm_exact_grid_bitexact(N, K, R):
    """qgemm_q8_0_i8 on the exact grid (weight and activation scales 1,
    integer codes): every block sum and every partial sum over blocks is an
    integer far below 2^24, so the result is exact; ragged row and column
    tiles, an odd block count (K = 96)."""
    rng = np.random.default_rng(N + K + R)
    W = rng.integers(-127, 128, (N, K)).astype(np.float64)
    W[:, ::32] = 127.0
    buf = fm.quantize("q8_0", W)
    x = rng.integers(-20, 21, (R, K)).astype(np.float32)
    x[:, ::32] = 127.0
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    y = to_np(qmoe.gemm_q8_0_i8(to_gpu(buf), N, K, q, d))
    ref, _ = int8.gemv_q8_0_i8(buf, N, K, x)
    assert_bitexact(y, ref, f"int8 gemm exact grid {N}x{K} R={R}")


@pytest.mark.parametrize("N,K,R", [(640, 2048, 2048), (2048, 640, 300), (4096, 14336, 200),
                                   (14336, 4096, 2048), (130, 384, 17)])
def test_gemm_within_bound(N, K, R):
    """Realistic Q8_0 weights and activations at prefill row counts; up to 64
    sampled output columns of the large shapes (rows of W quantize
    independently, so a subset of rows is the same tensor's rows)."""
    Wd = synth.normal_device((N, K), 0.02, 11, synth.GATE, N, "cuda")
    buf = qmoe.quantize("q8_0", Wd)
    x = synth.normal((R, K), 1.0, 12, synth.ACT, R)
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    y = to_np(qmoe.gemm_q8_0_i8(buf, N, K, q, d))
    cols = np.arange(N) if N <= 130 else np.sort(
        np.random.default_rng(N).choice(N, 64, replace=False))
    Wc = to_np(Wd[torch.from_numpy(cols).cuda()])
    ref, bound = int8.gemv_q8_0_i8(fm.quantize("q8_0", Wc), len(cols), K, x)
    assert_within_bound(y[:, cols], ref, bound, what=f"int8 gemm {N}x{K} R={R}")


def test_gemm_equals_gemv_on_few_rows():
    """The matrix-core GEMM and the v_dot4 GEMV take the same integer block
    sums; their fp32 sums over blocks differ at most by rounding order."""
    N, K, R = 512, 2048, 16
    buf = fm.quantize("q8_0", synth.normal((N, K), 0.02, 13, synth.UP, 0))
    x = synth.normal((R, K), 1.0, 14, synth.ACT, 2)
    q, d = qmoe.quantize_act_q8(to_gpu(x))
    a = to_np(qmoe.gemm_q8_0_i8(to_gpu(buf), N, K, q, d))
    b = to_np(qmoe.gemv_q8_0_i8(to_gpu(buf), N, K, q, d))
    _, bound = int8.gemv_q8_0_i8(buf, N, K, x)
    assert np.all(np.abs(a - b) <= 1e-5 * bound)
