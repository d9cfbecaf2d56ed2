"""Pins of the MXFP8 (E4M3) activation quantizer and the MX GEMM reference
against the OCP Microscaling Formats v1.0 definitions, exhaustive search and
brute force."""
import itertools
import math

import numpy as np
import pytest

from oracle import brute
from oracle import formats as fm
from oracle import mx


def test_e4m3_values_named_in_the_format_definition():
    # OCP MX v1.0, FP8 E4M3: bias 7, max normal S.1111.110 = 448, min normal
    # 2^-6, min subnormal 2^-9, S.1111.111 is NaN, no infinities
    assert mx.e4m3_value(0x7E) == 448.0
    assert mx.e4m3_value(0xFE) == -448.0
    assert mx.e4m3_value(0x08) == 2.0 ** -6
    assert mx.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert mx.e4m3_value(0x01) == 2.0 ** -9
    assert mx.e4m3_value(0x38) == 1.0
    assert mx.e4m3_value(0xC0) == -2.0
    assert mx.e4m3_value(0x00) == 0.0 and math.copysign(1, mx.e4m3_value(0x80)) < 0
    assert np.isnan(mx.e4m3_value(0x7F)) and np.isnan(mx.e4m3_value(0xFF))


def test_e4m3_grid_is_monotonic_and_symmetric():
    pos = mx.e4m3_value(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(mx.e4m3_value(np.arange(0x80, 0xFF)), -pos)
    # 8 values per binade above the subnormals: each normal value is a
    # 4-significant-bit number
    for c in range(0x08, 0x7F):
        v = float(pos[c])
        f, e = math.frexp(v)
        assert (f * 16).is_integer()


def _nearest_by_search(m):
    """Exhaustive: the non-negative finite code with the smallest |v - m|,
    ties to the even code; m beyond 448 saturates."""
    best, bd = None, None
    for c in range(0x7F):
        d = abs(float(mx.e4m3_value(c)) - m)
        if best is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best


def test_encoder_against_exhaustive_search():
    grid = mx.e4m3_value(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(0)
    probes = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                             rng.uniform(0, 500, 400), rng.uniform(0, 0.05, 200),
                             [448.0, 449.0, 464.0, 480.0, 1e6]])
    got = mx.e4m3_code_of_magnitude(probes)
    for m, c in zip(probes, got):
        assert c == _nearest_by_search(float(m)), m


def test_ties_go_to_the_even_code():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38;
    # 1.1875 lies between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A
    assert mx.e4m3_code_of_magnitude(1.0625) == 0x38
    assert mx.e4m3_code_of_magnitude(1.1875) == 0x3A
    # subnormal tie: 1.5 * 2^-9 between 0x01 and 0x02 -> 0x02
    assert mx.e4m3_code_of_magnitude(1.5 * 2.0 ** -9) == 0x02


def test_quantizer_closed_forms():
    x = np.zeros((3, 64))
    x[0, 0] = 1.0          # amax 1 -> E = -8, 1.0 * 2^8 = 256 -> code 0x78, exact
    x[0, 5] = -0.5         # -128 -> 0xF0
    x[1, 0] = 1.99         # 1.99 * 256 = 509.44 saturates at 448 -> 1.75
    x[1, 40] = 3.0         # second block: amax 3 -> E = -7, 3 * 128 = 384 -> exact
    # row 2: all zero -> scale byte 0, codes 0
    codes, scales = mx.quantize_mxfp8(x)
    assert scales.tolist() == [[119, 0], [119, 120], [0, 0]]
    assert codes[0, 0] == 0x78 and codes[0, 5] == 0xF0
    assert codes[1, 0] == 0x7E and codes[1, 40] == mx.e4m3_code_of_magnitude(384.0)
    deq = mx.dequantize_mxfp8(codes, scales)
    assert deq[0, 0] == 1.0 and deq[0, 5] == -0.5
    assert deq[1, 0] == 1.75 and deq[1, 40] == 3.0
    assert (deq[2] == 0).all() and (codes[2] == 0).all()


def test_quantizer_error_bound():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, (16, 512)) * np.exp(rng.normal(0, 2, (16, 1)))
    codes, scales = mx.quantize_mxfp8(x)
    deq = mx.dequantize_mxfp8(codes, scales)
    blocks = np.abs(x).reshape(16, 16, 32)
    E = np.floor(np.log2(blocks.max(axis=-1))) - 8
    top = np.repeat(448.0 * np.exp2(E), 32, axis=1)
    sub = np.repeat(np.exp2(E - 9), 32, axis=1)       # E4M3 subnormal step
    ax = np.abs(x)
    err = np.abs(deq - x)
    clipped = ax > top
    assert np.all(err[clipped] == ax[clipped] - top[clipped])
    ok = ~clipped
    assert np.all(err[ok] <= np.maximum(ax[ok] * 2.0 ** -4, sub[ok] / 2))
    assert np.all(np.sign(deq) * np.sign(x) >= 0)


def test_mx_gemm_against_brute_force():
    rng = np.random.default_rng(2)
    N, K, R = 3, 64, 2
    W = rng.normal(0, 0.02, (N, K))
    buf = fm.quantize("mxfp4", W)
    X = rng.normal(0, 1, (R, K))
    y, bound = mx.mx_gemm(buf, N, K, X)
    codes, scales = mx.quantize_mxfp8(X)
    for r, n in itertools.product(range(R), range(N)):
        acc, acc_abs = 0.0, 0.0
        for k in range(K):
            xv = float(mx.e4m3_value(codes[r, k])) * 2.0 ** (int(scales[r, k // 32]) - 127)
            wv = brute.element("mxfp4", buf, N, K, n, k)
            acc += wv * xv
            acc_abs += abs(wv * xv)
        assert y[r, n] == pytest.approx(acc, rel=1e-12, abs=1e-15)
        assert bound[r, n] == pytest.approx(acc_abs, rel=1e-12)


def _e4m3_scalar(c):
    """E4M3 value from its bit fields (OCP MX v1.0), finite codes only."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    return s * (math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7))


_POS = [_e4m3_scalar(c) for c in range(0x7F)]


def _mxfp8_scalar(block):
    """One 32-value block quantized and dequantized element by element: the
    shared exponent from the largest magnitude, every element to the nearest
    of the 127 non-negative E4M3 values by search (ties to the even code,
    saturating at 448)."""
    amax = max(abs(v) for v in block)
    if amax == 0:
        return [0.0] * len(block)
    e = min(max(math.frexp(amax)[1] - 1 - 8 + 127, 0), 254)
    scale = math.ldexp(1.0, e - 127)
    out = []
    for v in block:
        m = abs(v) / scale
        best, bd = 0, None
        for c, g in enumerate(_POS):
            d = abs(g - m)
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        out.append(math.copysign(_POS[best] * scale, v) if best else 0.0)
    return out


def test_mx_expert_ffn_against_scalar_brute_force():
    """One MXFP4/MXFP4 expert on the block-scaled path, element by element:
    x quantized to MXFP8 per 32 values along H, g and u from the packed gate
    and up bytes, h = SiLU(g) u quantized per 32 values along F (the down
    projection's reduction axis), o from the packed down bytes.  Two rows and
    F = 96 (three blocks along F) so that quantizing along the wrong axis or
    over the wrong span changes the result."""
    rng = np.random.default_rng(11)
    H, F, R = 64, 96, 2
    gbuf = fm.quantize("mxfp4", rng.normal(0, 0.2, (F, H)))
    ubuf = fm.quantize("mxfp4", rng.normal(0, 0.2, (F, H)))
    dbuf = fm.quantize("mxfp4", rng.normal(0, 0.2, (H, F)))
    X = rng.normal(0, 1, (R, H)) * np.array([[1.0], [37.0]])
    o, bound = mx.mx_expert_ffn(gbuf, ubuf, dbuf, H, F, X)
    assert o.shape == (R, H) and bound.shape == (R, H)
    for r in range(R):
        xq = []
        for b in range(H // 32):
            xq += _mxfp8_scalar([float(v) for v in X[r, 32 * b:32 * b + 32]])
        g = [sum(brute.element("mxfp4", gbuf, F, H, n, k) * xq[k] for k in range(H))
             for n in range(F)]
        u = [sum(brute.element("mxfp4", ubuf, F, H, n, k) * xq[k] for k in range(H))
             for n in range(F)]
        h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
        hq = []
        for b in range(F // 32):
            hq += _mxfp8_scalar(h[32 * b:32 * b + 32])
        for n in range(H):
            terms = [brute.element("mxfp4", dbuf, H, F, n, j) * hq[j] for j in range(F)]
            assert o[r, n] == pytest.approx(sum(terms), rel=1e-12, abs=1e-14)
            assert bound[r, n] == pytest.approx(sum(abs(t) for t in terms), rel=1e-12)
