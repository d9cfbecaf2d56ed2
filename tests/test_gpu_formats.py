"""GPU parity of the block formats: device quantizer bytes == oracle quantizer
bytes, device dequantizer == exact values rounded to fp32 (bit-exact)."""
import os

import numpy as np
import pytest

from gpu_util import requires_gpu, to_gpu, to_np, assert_bitexact, torch
from oracle import formats as fm
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _weights(kind, N, K, seed):
    W = synth.normal((N, K), 0.02, seed, synth.GATE, 7)
    if kind == "outlier":
        W[:, ::97] *= 40
    elif kind == "constant":
        W[:] = np.float32(-0.013)
    elif kind == "zeros":
        W[:] = 0
        W[0, 5] = np.float32(0.02)
    elif kind == "wide":
        W *= np.float32(50.0)
    elif kind == "tiny":
        W *= np.float32(1e-4)
    return W


@pytest.mark.parametrize("fmt", fm.FORMATS)
@pytest.mark.parametrize("kind", ["normal", "outlier", "constant", "zeros", "wide", "tiny"])
@pytest.mark.parametrize("N,K", [(3, 256), (37, 2048), (2, 7168)])
def test_device_quantizer_matches_oracle_bytes(fmt, kind, N, K):
    W = _weights(kind, N, K, seed=N)
    ref = fm.quantize(fmt, W)
    got = to_np(qmoe.quantize(fmt, to_gpu(W)))
    assert got.shape == ref.shape
    if not (got == ref).all():
        i = int(np.argmax(got != ref))
        offs, _ = fm.plane_offsets(fmt, N, K)
        raise AssertionError(f"{fmt}/{kind}: {(got != ref).sum()} bytes differ, first at {i} "
                             f"(planes at {offs}): got {got[i]} want {ref[i]}")


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_device_quantizer_ragged_rows_and_640(fmt):
    K = 640 if fm.BLOCK[fmt] == 32 else 512
    W = _weights("normal", 2049, K, seed=11)
    assert (to_np(qmoe.quantize(fmt, to_gpu(W))) == fm.quantize(fmt, W)).all()


@pytest.mark.parametrize("fmt", fm.FORMATS)
@pytest.mark.parametrize("N,K", [(5, 256), (64, 2048), (3, 640)])
def test_dequant_bitexact_on_oracle_packed(fmt, N, K):
    if K % fm.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    W = _weights("outlier", N, K, seed=3)
    buf = fm.quantize(fmt, W)
    got = to_np(qmoe.dequantize(fmt, to_gpu(buf), N, K))
    assert_bitexact(got, fm.dequantize_f32(fmt, buf, N, K), fmt)


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_dequant_bitexact_on_random_bytes(fmt):
    """Any code pattern with finite scales (fp16 scales drawn over a wide range,
    subnormals included)."""
    N, K = 9, 512
    rng = np.random.default_rng(21)
    buf = rng.integers(0, 256, fm.tensor_bytes(fmt, N, K), dtype=np.uint8)
    offs, _ = fm.plane_offsets(fmt, N, K)
    sizes = fm.plane_bytes(fmt, N, K)
    f16 = lambda n: np.frombuffer((rng.standard_normal(n) * 10.0 ** rng.integers(-7, 3, n))
                                  .astype("<f2").tobytes(), np.uint8)
    if fmt in ("q8_0", "q4_0"):
        buf[offs[1]:offs[1] + sizes[1]] = f16(sizes[1] // 2)
    if fmt == "mxfp4":
        buf[offs[1]:offs[1] + sizes[1]] = rng.integers(1, 255, sizes[1])
    if fmt == "q4_k":
        meta = buf[offs[1]:offs[1] + sizes[1]].reshape(-1, 16)
        meta[:, 0:4] = f16(2 * meta.shape[0]).reshape(-1, 4)
    if fmt == "q6_k":
        buf[offs[3]:offs[3] + sizes[3]] = f16(sizes[3] // 2)
    got = to_np(qmoe.dequantize(fmt, to_gpu(buf), N, K))
    assert_bitexact(got, fm.dequantize_f32(fmt, buf, N, K), fmt)


def test_dequant_golden_blocks():
    from test_oracle_formats import _golden, _hand_built
    _, values = _golden()
    for case in values:
        fmt, N, K, buf = _hand_built(case)
        arr = np.frombuffer(bytes(buf), dtype=np.uint8)
        got = to_np(qmoe.dequantize(fmt, to_gpu(arr), N, K)).reshape(-1)
        for idx, expect, neg in values[case]:
            assert got[idx] == expect, (case, idx, got[idx], expect)


def test_mxfp4_nan_and_extreme_scales():
    N, K = 4, 32
    codes = np.arange(32) % 16
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    buf = np.zeros(fm.tensor_bytes("mxfp4", N, K), np.uint8)
    for n in range(N):
        buf[16 * n:16 * n + 16] = q
    buf[256:260] = [255, 0, 1, 252]          # NaN, subnormal scales, near the fp32 top
    got = to_np(qmoe.dequantize("mxfp4", to_gpu(buf), N, K))
    assert_bitexact(got, fm.dequantize_f32("mxfp4", buf, N, K), "mxfp4 extremes")
