"""GPU parity of qgemv_<fmt> against the oracle GEMV."""
import numpy as np
import pytest

from gpu_util import (requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound,
                      torch)
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import configs, layers, qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _grid_fields(fmt, N, K, rng, fp16_exact=False):
    """Quantized fields whose dequantized values are exact in fp32.  With
    fp16_exact (many activation rows run on the fp16 matrix cores) every
    weight value is also exact in fp16: the Q4_K min scale equals the block
    scale, so d*sc*q - dmin*m is an integer multiple of d below 2^11, and the
    Q6_K sub-block scales stay within +-63 so |sc*(q-32)| <= 2016."""
    nb = K // fm.BLOCK[fmt]
    p2 = lambda: np.float16(2.0 ** -int(rng.integers(3, 8)))
    if fmt == "q8_0":
        return {"q": rng.integers(-128, 128, (N, K)).astype(np.int8),
                "d": np.array([[p2() for _ in range(nb)] for _ in range(N)], np.float16)}
    if fmt == "q4_0":
        return {"q": rng.integers(0, 16, (N, K)).astype(np.uint8),
                "d": np.array([[p2() for _ in range(nb)] for _ in range(N)], np.float16)}
    if fmt == "mxfp4":
        return {"q": rng.integers(0, 16, (N, K)).astype(np.uint8),
                "e": rng.integers(120, 128, (N, nb)).astype(np.uint8)}
    if fmt == "q4_k":
        d = np.array([[p2() for _ in range(nb)] for _ in range(N)], np.float16)
        dmin = d.copy() if fp16_exact else \
            np.array([[p2() for _ in range(nb)] for _ in range(N)], np.float16)
        return {"q": rng.integers(0, 16, (N, K)).astype(np.uint8), "d": d, "dmin": dmin,
                "sc": rng.integers(0, 64, (N, nb, 8)).astype(np.uint8),
                "m": rng.integers(0, 64, (N, nb, 8)).astype(np.uint8)}
    lim = 64 if fp16_exact else 128
    return {"q": rng.integers(0, 64, (N, K)).astype(np.uint8),
            "sc": rng.integers(-lim + 1, lim, (N, nb, 16)).astype(np.int8),
            "d": np.array([[p2() for _ in range(nb)] for _ in range(N)], np.float16)}


@pytest.mark.parametrize("fmt", fm.FORMATS)
@pytest.mark.parametrize("R", [1, 3, 16])
def test_gemv_grid_exact_is_bitexact(fmt, R):
    """Power-of-two scales and small-integer activations: every product and
    partial sum is exact in fp32, so any summation order gives the exact
    result, which the oracle computes in float64."""
    N, K = 77, 1024
    rng = np.random.default_rng(R)
    buf = fm.pack(fmt, _grid_fields(fmt, N, K, rng, fp16_exact=R > 4), N, K)
    x = rng.integers(-4, 5, (R, K)).astype(np.float32)
    y_ref, _ = moe.gemv(fmt, buf, N, K, x)
    y = to_np(qmoe.gemv(fmt, to_gpu(buf), N, K, to_gpu(x)))
    assert_bitexact(y, y_ref.astype(np.float32), f"{fmt} R={R}")


SHAPES = [(1, 256), (5, 512), (64, 2048), (300, 640), (33, 7168), (4, 14336), (129, 4096)]


@pytest.mark.parametrize("fmt", fm.FORMATS)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("R", [1, 2, 6, 16, 17])
def test_gemv_within_bound(fmt, N, K, R):
    if K % fm.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    W = synth.normal((N, K), 0.02, 5, synth.DENSE, N)
    buf = fm.quantize(fmt, W)
    x = synth.normal((R, K), 1.0, 5, synth.ACT, R)
    y_ref, bound = moe.gemv(fmt, buf, N, K, x)
    y = to_np(qmoe.gemv(fmt, to_gpu(buf), N, K, to_gpu(x)))
    assert_within_bound(y, y_ref, bound, what=f"{fmt} {N}x{K} R={R}")


@pytest.mark.parametrize("fmt", ["q6_k", "q4_0"])
@pytest.mark.parametrize("R", [1, 2])
def test_gemv_k_beyond_lds_staging(fmt, R):
    """K = 28672 (a 70B-class FFN down projection): one activation row no
    longer fits the LDS staging, so the matrix-core path serves every R."""
    N, K = 40, 28672
    W = synth.normal((N, K), 0.02, 6, synth.DENSE, K)
    buf = fm.quantize(fmt, W)
    x = synth.normal((R, K), 1.0, 6, synth.ACT, R)
    y_ref, bound = moe.gemv(fmt, buf, N, K, x)
    y = to_np(qmoe.gemv(fmt, to_gpu(buf), N, K, to_gpu(x)))
    assert_within_bound(y, y_ref, bound, what=f"{fmt} K={K} R={R}")


@pytest.mark.parametrize("fmt", ["q4_k", "q8_0"])
def test_gemv_bf16_activations(fmt):
    N, K, R = 96, 7168, 16
    buf = fm.quantize(fmt, synth.normal((N, K), 0.02, 8, synth.DENSE))
    x = synth.bf16_round(synth.normal((R, K), 1.0, 8, synth.ACT))
    y_ref, bound = moe.gemv(fmt, buf, N, K, x)
    xb = to_gpu(x).to(torch.bfloat16)
    assert (to_np(xb.float()) == x).all()
    y = to_np(qmoe.gemv(fmt, to_gpu(buf), N, K, xb))
    assert_within_bound(y, y_ref, bound, what=f"{fmt} bf16")


def test_gemv_is_deterministic():
    N, K = 4096, 4096
    buf = to_gpu(fm.quantize("q4_k", synth.normal((N, K), 0.02, 9, synth.DENSE)))
    x = to_gpu(synth.normal((1, K), 1.0, 9, synth.ACT))
    a = to_np(qmoe.gemv("q4_k", buf, N, K, x))
    b = to_np(qmoe.gemv("q4_k", buf, N, K, x))
    assert (a == b).all()


def test_llama8b_layer_shapes_sampled_rows():
    """The seven matrices of a Llama-3.1-8B layer (Q4_K, down Q6_K) at full
    size on the device; the oracle checks 48 sampled rows of each."""
    cfg = configs.LLAMA8B_GEMV
    layer = layers.DenseLayer(cfg)
    rng = np.random.default_rng(0)
    xs = {}
    for i, (name, N, K, fmt) in enumerate(cfg.mats):
        x = synth.normal((1, K), 1.0, 0, synth.ACT, i)
        xs[name] = x
        y = to_np(qmoe.gemv(fmt, layer.mats[0][i], N, K, to_gpu(x)))
        rows = np.sort(rng.choice(N, 48, replace=False))
        rows[-1] = N - 1
        buf = fm.quantize(fmt, layer.matrix_fp32(i, torch.from_numpy(rows).cuda()))
        y_ref, bound = moe.gemv(fmt, buf, len(rows), K, x)
        assert_within_bound(y[:, rows], y_ref, bound, what=f"{name} {N}x{K}")
    assert layer.weight_bytes() == 137822208


# ------------------------------------------------------------- batched ---

def test_gemv_batch_equals_one_launch_per_matrix():
    """qgemv_batch runs each matrix exactly as qgemv does: mixed formats,
    shapes, dtypes and row counts (dot products, chunked rows, matrix cores,
    a K too long for two staged rows) in one launch, outputs equal bit for
    bit (qgemv's own parity with the oracle is tested above)."""
    rng = np.random.default_rng(7)
    cases = [("q4_k", 1000, 4096, 1, "f32"), ("q6_k", 640, 14336, 1, "f32"),
             ("q8_0", 96, 640, 3, "bf16"), ("q4_0", 2048, 2048, 6, "f32"),
             ("mxfp4", 33, 512, 16, "bf16"), ("q4_k", 64, 256, 2, "f32"),
             ("q6_k", 17, 1024, 4, "bf16")]
    items, singles = [], []
    for i, (fmt, N, K, R, dt) in enumerate(cases):
        w = synth.normal((N, K), 0.02, 30 + i, synth.DENSE)
        W = qmoe.quantize(fmt, to_gpu(w))
        x = synth.normal((R, K), 1.0, 40 + i, synth.ACT)
        xg = to_gpu(x) if dt == "f32" else to_gpu(synth.bf16_round(x)).to(torch.bfloat16)
        out = torch.full((R, N), float("nan"), dtype=torch.float32, device="cuda")
        items.append((fmt, W, N, K, xg, out))
        singles.append(qmoe.gemv(fmt, W, N, K, xg))
    outs = qmoe.gemv_batch(items)
    for (fmt, N, K, R, dt), a, b in zip(cases, outs, singles):
        assert_bitexact(to_np(a), to_np(b), what=f"batch {fmt} N={N} K={K} R={R}")


def test_gemv_batch_empty_and_zero_rows():
    assert qmoe.gemv_batch([]) == []
    W = qmoe.quantize("q8_0", to_gpu(synth.normal((8, 64), 0.02, 1, synth.DENSE)))
    x = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    qmoe.gemv_batch([("q8_0", W, 8, 64, x, out)])
    torch.cuda.synchronize()
