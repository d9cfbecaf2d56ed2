"""GPU parity of the ternary format T5 ("t5_g128_fp16", the "RTX 4080 SUPER
native Windows 27B: NInfer 80 SM port" page, section 九.2): device quantizer
bytes == oracle bytes, device dequantizer bit-exact, qgemv_t5 bit-exact on
grid values and within 1e-3 * sum |w x| on synthetic layers."""
import numpy as np
import pytest

from gpu_util import (requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound,
                      torch)
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import configs, qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _weights(kind, N, K, seed):
    W = synth.normal((N, K), 0.02, seed, synth.DENSE, 11)
    if kind == "outlier":
        W[:, ::97] *= 40
    elif kind == "zeros":
        W[:, :128] = 0
    elif kind == "heavy":
        rng = np.random.default_rng(seed)
        W = (W * rng.standard_t(2, W.shape).astype(np.float32)).astype(np.float32)
    return W


@pytest.mark.parametrize("kind", ["normal", "outlier", "zeros", "heavy"])
@pytest.mark.parametrize("N,K", [(3, 128), (37, 2048), (2, 14336), (2049, 384)])
def test_t5_device_quantizer_matches_oracle_bytes(kind, N, K):
    W = _weights(kind, N, K, seed=N)
    ref = fm.quantize("t5", W)
    got = to_np(qmoe.quantize("t5", to_gpu(W)))
    assert got.shape == ref.shape
    if not (got == ref).all():
        i = int(np.argmax(got != ref))
        raise AssertionError(f"t5/{kind}: {(got != ref).sum()} bytes differ, first at {i}: "
                             f"got {got[i]} want {ref[i]}")


@pytest.mark.parametrize("N,K", [(5, 128), (64, 2048), (3, 640)])
def test_t5_dequant_bitexact(N, K):
    buf = fm.quantize("t5", _weights("outlier", N, K, seed=3))
    got = to_np(qmoe.dequantize("t5", to_gpu(buf), N, K))
    assert_bitexact(got, fm.dequantize_f32("t5", buf, N, K), f"t5 {N}x{K}")


def _grid_buf(N, K, rng):
    """Power-of-two scales and random trits (including the all-zero code)."""
    nb = K // 128
    t = rng.integers(-1, 2, (N, K)).astype(np.int8)
    d = np.float16(2.0) ** -rng.integers(3, 8, (N, nb)).astype(np.float16)
    return fm.pack("t5", {"t": t, "d": d.astype(np.float16)}, N, K)


@pytest.mark.parametrize("R", [1, 2, 3, 16])
@pytest.mark.parametrize("N,K", [(77, 1024), (5, 384), (130, 128)])
def test_t5_gemv_grid_exact_is_bitexact(R, N, K):
    """Every product and partial sum is exact in fp32 (small-integer
    activations, power-of-two scales), so the result must equal the exact
    one bit for bit, whatever the summation order."""
    rng = np.random.default_rng(R + N)
    buf = _grid_buf(N, K, rng)
    x = rng.integers(-4, 5, (R, K)).astype(np.float32)
    y_ref, _ = moe.gemv("t5", buf, N, K, x)
    y = to_np(qmoe.gemv("t5", to_gpu(buf), N, K, to_gpu(x)))
    assert_bitexact(y, y_ref.astype(np.float32), f"t5 {N}x{K} R={R}")


SHAPES = [(1, 128), (7, 384), (300, 1152), (33, 4096), (64, 14336), (5, 18816)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("R", [1, 2, 5, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_t5_gemv_within_bound(N, K, R, dtype):
    W = synth.normal((N, K), 0.02, 5, synth.DENSE, N)
    buf = fm.quantize("t5", W)
    x = synth.normal((R, K), 1.0, 5, synth.ACT, R)
    if dtype == "bf16":
        x = synth.bf16_round(x)
    xg = to_gpu(x) if dtype == "f32" else to_gpu(x).to(torch.bfloat16)
    y_ref, bound = moe.gemv("t5", buf, N, K, x)
    y = to_np(qmoe.gemv("t5", to_gpu(buf), N, K, xg))
    assert_within_bound(y, y_ref, bound, what=f"t5 {N}x{K} R={R} {dtype}")


def test_t5_gemv_llama_down_shape_sampled():
    """[4096, 14336] (a Llama-3.1-8B down projection) in T5, one row: the
    whole output against the oracle on sampled weight rows."""
    N, K = 4096, 14336
    W = synth.normal((N, K), 0.02, 6, synth.DENSE, 1)
    buf_dev = qmoe.quantize("t5", to_gpu(W))
    x = synth.normal((1, K), 1.0, 6, synth.ACT, 1)
    y = to_np(qmoe.gemv("t5", buf_dev, N, K, to_gpu(x)))
    rows = np.concatenate([np.arange(0, N, 97), [N - 1]])
    sub = fm.quantize("t5", W[rows])
    y_ref, bound = moe.gemv("t5", sub, len(rows), K, x)
    assert_within_bound(y[:, rows], y_ref, bound, what="t5 llama down")


def test_t5_batch_equals_single_calls():
    """qgemv_batch over T5 matrices: every output equals its qgemv_t5 call
    bit for bit (the row arithmetic does not depend on the launch)."""
    rng = np.random.default_rng(9)
    shapes = [(300, 1152, 1), (33, 4096, 2), (64, 14336, 1), (7, 384, 5), (1, 128, 16)]
    items, singles = [], []
    for i, (N, K, R) in enumerate(shapes):
        W = to_gpu(fm.quantize("t5", synth.normal((N, K), 0.02, 7, synth.DENSE, i)))
        x = to_gpu(rng.standard_normal((R, K)).astype(np.float32))
        singles.append(to_np(qmoe.gemv("t5", W, N, K, x)).copy())
        items.append(("t5", W, N, K, x, torch.empty((R, N), dtype=torch.float32, device="cuda")))
    outs = qmoe.gemv_batch(items)
    for (N, K, R), got, ref in zip(shapes, outs, singles):
        assert_bitexact(to_np(got), ref, f"t5 batch {N}x{K} R={R}")
