"""Pins for the oracle's block formats (CPU only).

Each check ties oracle/formats.py to something other than itself:
  * hand-built blocks, packed byte by byte here with plain Python integers,
    whose values were worked out by hand (tests/golden/closed_form_blocks.txt);
  * a second, element-by-element reader (oracle/brute.py) on random bytes;
  * quantizer error bounds derived from each quantization rule;
  * exact round trips on values that lie on a format's grid;
  * IEEE special cases of the fp16 rounding and the tie rule.
"""
import os
import struct

import numpy as np
import pytest

from oracle import brute
from oracle import formats as fm
from decode_moe_mul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_blocks.txt")


def _golden():
    layouts, values = [], {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "layout":
            offs = [int(v) for v in line[4].split(",")]
            layouts.append((line[1], int(line[2]), int(line[3]), offs, int(line[5])))
        elif line[0] == "value":
            values.setdefault(line[1], []).append((int(line[2]), float(line[3]),
                                                   line[3].startswith("-")))
    return layouts, values


def _f16b(v):
    return struct.pack("<e", v)


def _put(buf, off, data):
    buf[off:off + len(data)] = data


def _hand_built(case):
    """Bytes of the golden cases, written straight from the layout rules."""
    if case == "q8_0_a":
        buf = bytearray(512)
        _put(buf, 0, bytes((i - 16) & 255 for i in range(32)))
        _put(buf, 256, _f16b(1.0))
        return "q8_0", 1, 32, buf
    if case == "q8_0_b":
        buf = bytearray(512)
        q = [-128, 127] + [1] * 30
        _put(buf, 0, bytes(v & 255 for v in q))
        _put(buf, 256, _f16b(0.5))
        return "q8_0", 1, 32, buf
    if case == "q4_0_a":
        buf = bytearray(512)
        codes = [i % 16 for i in range(32)]
        _put(buf, 0, bytes(codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16)))
        _put(buf, 256, _f16b(0.5))
        return "q4_0", 1, 32, buf
    if case == "mxfp4_a":
        buf = bytearray(512)
        codes = [i % 16 for i in range(32)]
        row = bytes(codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16))
        _put(buf, 0, row + row)
        _put(buf, 256, bytes([127, 130]))
        return "mxfp4", 2, 32, buf
    if case == "q4_k_a":
        buf = bytearray(512)
        codes = [k % 16 for k in range(256)]
        _put(buf, 0, bytes(codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(128)))
        field = 0
        for j in range(8):
            field |= (j + 1) << (6 * j)
            field |= j << (48 + 6 * j)
        _put(buf, 256, _f16b(0.125) + _f16b(0.25) + field.to_bytes(12, "little"))
        return "q4_k", 1, 256, buf
    if case == "q6_k_a":
        buf = bytearray(1024)
        q = [k % 64 for k in range(256)]
        _put(buf, 0, bytes((q[2 * i] & 15) | ((q[2 * i + 1] & 15) << 4) for i in range(128)))
        qh = []
        for i in range(64):
            b = 0
            for r in range(4):
                b |= (q[4 * i + r] >> 4) << (2 * r)
            qh.append(b)
        _put(buf, 256, bytes(qh))
        _put(buf, 512, bytes((j - 8) & 255 for j in range(16)))
        _put(buf, 768, _f16b(1.0 / 16))
        return "q6_k", 1, 256, buf
    raise KeyError(case)


def test_layout_matches_golden():
    layouts, _ = _golden()
    for fmt, N, K, offs, total in layouts:
        o, t = fm.plane_offsets(fmt, N, K)
        assert o == offs and t == total, (fmt, N, K)


def test_tier_expert_sizes():
    # bytes per expert of the three tiers of the 512-expert layer (H 2048, F 640)
    hot = 2 * fm.tensor_bytes("q6_k", 640, 2048) + fm.tensor_bytes("q8_0", 2048, 640)
    mid = 2 * fm.tensor_bytes("q4_k", 640, 2048) + fm.tensor_bytes("q4_0", 2048, 640)
    cold = 2 * fm.tensor_bytes("mxfp4", 640, 2048) + fm.tensor_bytes("mxfp4", 2048, 640)
    assert (hot, mid, cold) == (3543040, 2211840, 2088960)


@pytest.mark.parametrize("case", ["q8_0_a", "q8_0_b", "q4_0_a", "mxfp4_a", "q4_k_a", "q6_k_a"])
def test_closed_form_blocks(case):
    _, values = _golden()
    fmt, N, K, buf = _hand_built(case)
    buf = np.frombuffer(bytes(buf), dtype=np.uint8)
    D = fm.dequantize(fmt, buf, N, K).reshape(-1)
    for idx, expect, neg in values[case]:
        assert D[idx] == expect, (case, idx, D[idx], expect)
        if expect == 0.0 and neg:           # an encoded negative zero
            assert np.signbit(D[idx])
        # the element-wise reader agrees
        n, k = divmod(idx, K)
        assert brute.element(fmt, bytes(buf), N, K, n, k) == expect


def test_mxfp4_nan_scale():
    fmt, N, K, buf = _hand_built("mxfp4_a")
    buf[256] = 255
    D = fm.dequantize(fmt, np.frombuffer(bytes(buf), dtype=np.uint8), N, K)
    assert np.isnan(D[0]).all() and not np.isnan(D[1]).any()


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_two_readers_agree_on_random_bytes(fmt):
    N, K = 3, 512
    rng = np.random.default_rng(5)
    buf = rng.integers(0, 256, fm.tensor_bytes(fmt, N, K), dtype=np.uint8)
    # keep fp16 scales finite and E8M0 scales away from the NaN code
    offs, _ = fm.plane_offsets(fmt, N, K)
    sizes = fm.plane_bytes(fmt, N, K)
    if fmt in ("q8_0", "q4_0"):
        buf[offs[1]:offs[1] + sizes[1]] = np.frombuffer(
            rng.standard_normal(sizes[1] // 2).astype("<f2").tobytes(), np.uint8)
    if fmt == "mxfp4":
        buf[offs[1]:offs[1] + sizes[1]] = rng.integers(100, 150, sizes[1])
    if fmt == "q4_k":
        meta = buf[offs[1]:offs[1] + sizes[1]].reshape(-1, 16)
        meta[:, 0:4] = np.frombuffer(rng.standard_normal(2 * meta.shape[0]).astype("<f2").tobytes(),
                                     np.uint8).reshape(-1, 4)
    if fmt == "q6_k":
        buf[offs[3]:offs[3] + sizes[3]] = np.frombuffer(
            rng.standard_normal(sizes[3] // 2).astype("<f2").tobytes(), np.uint8)
    D = fm.dequantize(fmt, buf, N, K)
    for n in range(N):
        for k in range(0, K, 7):
            assert D[n, k] == brute.element(fmt, bytes(buf), N, K, n, k), (n, k)


def test_fp16_rounding_special_cases():
    one = 1.0
    # tie between 1 and 1+2^-10 goes to even (1); just above goes up
    assert fm.fp16_rne(one + 2.0 ** -11) == 1.0
    assert fm.fp16_rne(one + 2.0 ** -11 + 2.0 ** -40) == 1.0 + 2.0 ** -10
    assert fm.fp16_rne(one + 3 * 2.0 ** -11) == 1.0 + 2 * 2.0 ** -10
    # subnormals are kept (smallest subnormal 2^-24) and ties go to even
    assert fm.fp16_rne(2.0 ** -24) == 2.0 ** -24
    assert fm.fp16_rne(2.0 ** -25) == 0.0
    assert fm.fp16_rne(3 * 2.0 ** -25) == 2.0 ** -23
    assert fm.fp16_rne(1.4e-5) == np.float16(1.4e-5)
    with np.errstate(over="ignore"):
        assert np.isinf(fm.fp16_rne(65520.0)) and fm.fp16_rne(65519.0) == 65504.0


def test_round_half_away():
    v = np.array([0.5, -0.5, 1.5, 2.5, -2.5, 0.49999999999999994, 3.4999, -7.5, 0.0])
    assert list(fm.round_half_away(v)) == [1, -1, 2, 3, -3, 0, 3, -8, 0]


def _weights(kind, N, K, seed=1):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return synth.normal((N, K), 0.02, seed, synth.GATE)
    W = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    if kind == "outlier":
        W[:, ::97] *= 40
    elif kind == "constant":
        W[:] = np.float32(-0.013)
    elif kind == "zeros":
        W[:] = 0
        W[0, 5] = np.float32(0.02)
    elif kind == "positive":
        W = np.abs(W)
    elif kind == "negative":
        W = -np.abs(W)
    return W


KINDS = ["normal", "outlier", "constant", "zeros", "positive", "negative"]


@pytest.mark.parametrize("kind", KINDS)
def test_q8_0_error_bound(kind):
    W = _weights(kind, 8, 512)
    f = fm.quantize_q8_0(W)
    D = fm.dequantize("q8_0", fm.quantize("q8_0", W), 8, 512)
    d = np.repeat(f["d"].astype(np.float64), 32, axis=1)
    assert (np.abs(D - W) <= 0.5 * d).all()
    assert f["q"].min() >= -127


@pytest.mark.parametrize("kind", KINDS)
def test_q4_0_error_bound(kind):
    W = _weights(kind, 8, 512)
    f = fm.quantize_q4_0(W)
    D = fm.dequantize("q4_0", fm.quantize("q4_0", W), 8, 512)
    d = np.repeat(f["d"].astype(np.float64), 32, axis=1)
    assert (np.abs(D - W) <= 0.5 * d).all()


@pytest.mark.parametrize("kind", KINDS)
def test_mxfp4_error_bound(kind):
    W = _weights(kind, 8, 512)
    f = fm.quantize_mxfp4(W)
    D = fm.dequantize("mxfp4", fm.quantize("mxfp4", W), 8, 512)
    scale = np.repeat(np.ldexp(1.0, f["e"].astype(np.int64) - 127), 32, axis=1)
    v = np.abs(W.astype(np.float64)) / scale          # element in scaled units
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    allowed = np.where(v > 6, v - 6, half_gap) * scale
    assert (np.abs(D - W) <= allowed).all()
    amax = np.abs(W.astype(np.float64)).reshape(8, -1, 32).max(-1)
    nz = amax > 0
    # the shared scale puts the block maximum in [4, 8) scaled units
    top = amax[nz] / np.ldexp(1.0, f["e"][nz].astype(np.int64) - 127)
    assert ((top >= 4) & (top < 8)).all()


@pytest.mark.parametrize("kind", KINDS)
def test_q4_k_error_bound(kind):
    W = _weights(kind, 4, 1024)
    f = fm.quantize_q4_k(W)
    D = fm.dequantize("q4_k", fm.quantize("q4_k", W), 4, 1024)
    d = np.repeat(f["d"].astype(np.float64), 256, axis=1)
    dmin = np.repeat(f["dmin"].astype(np.float64), 256, axis=1)
    sc = np.repeat(f["sc"].reshape(4, -1).astype(np.float64), 32, axis=1)
    bound = 0.5 * d * sc + 7.5 * d + 0.5 * dmin
    assert (np.abs(D - W) <= bound * (1 + 1e-12)).all()


@pytest.mark.parametrize("kind", KINDS)
def test_q6_k_error_bound(kind):
    W = _weights(kind, 4, 1024)
    f = fm.quantize_q6_k(W)
    D = fm.dequantize("q6_k", fm.quantize("q6_k", W), 4, 1024)
    d = np.repeat(f["d"].astype(np.float64), 256, axis=1)
    sc = np.repeat(f["sc"].reshape(4, -1).astype(np.float64), 16, axis=1)
    bound = 0.5 * d * np.abs(sc) + 15.5 * d
    assert (np.abs(D - W) <= bound * (1 + 1e-12)).all()


def test_grid_round_trip_q8_0_q4_0():
    rng = np.random.default_rng(3)
    d = 2.0 ** -7
    q8 = rng.integers(-127, 128, (4, 256))
    q8[:, ::32] = 127                                    # block max on the grid
    W = (q8 * d).astype(np.float32)
    f = fm.quantize_q8_0(W)
    assert (f["q"] == q8).all() and (f["d"] == d).all()
    q4 = rng.integers(1, 16, (4, 256))
    q4[:, ::32] = 1                                      # value -7 d
    W = ((q4 - 8) * d).astype(np.float32)
    f = fm.quantize_q4_0(W)
    assert (f["q"] == q4).all() and (f["d"] == d).all()


def test_grid_round_trip_mxfp4():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, (2, 64)).astype(np.uint8)
    codes[:, ::32] = 7                                   # +6 present in each block
    e = np.array([[120, 131], [127, 100]])
    W = (fm.e2m1_value(codes) * np.repeat(np.ldexp(1.0, e - 127), 32, axis=1)).astype(np.float32)
    f = fm.quantize_mxfp4(W)
    assert (f["e"] == e).all()
    # -0 and +0 dequantize identically; compare values, and codes off zero
    assert (fm.e2m1_value(f["q"]) == fm.e2m1_value(codes)).all()
    nz = (codes & 7) != 0
    assert (f["q"][nz] == codes[nz]).all()


def test_grid_round_trip_q6_k():
    rng = np.random.default_rng(6)
    d = 2.0 ** -12
    sc = rng.integers(1, 128, (2, 1, 16))
    sc[:, :, 3] = 127
    q = rng.integers(1, 64, (2, 1, 16, 16))         # code 0 (-32) would set the scale
    q[..., 0] = 63                                       # +31 in each sub-block
    W = (d * sc[..., None] * (q - 32)).reshape(2, 256).astype(np.float32)
    f = fm.quantize_q6_k(W)
    assert (f["d"] == d).all() and (f["sc"].reshape(sc.shape) == sc).all()
    assert (f["q"] == q.reshape(2, 256)).all()


def test_grid_round_trip_q4_k():
    rng = np.random.default_rng(7)
    d, dmin = 2.0 ** -10, 2.0 ** -9
    sc = rng.integers(1, 64, (2, 1, 8))
    sc[..., 2] = 63
    m = rng.integers(0, 64, (2, 1, 8))
    m[..., 5] = 63
    q = rng.integers(0, 16, (2, 1, 8, 32))
    q[..., 0] = 0
    q[..., 1] = 15
    W = (d * sc[..., None] * q - dmin * m[..., None]).reshape(2, 256).astype(np.float32)
    f = fm.quantize_q4_k(W)
    assert (f["d"] == d).all() and (f["dmin"] == dmin).all()
    assert (f["sc"].reshape(sc.shape) == sc).all() and (f["m"].reshape(m.shape) == m).all()
    assert (f["q"] == q.reshape(2, 256)).all()


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_pack_unpack_fields(fmt):
    W = _weights("normal", 6, 512)
    f = fm.QUANTIZE[fmt](W)
    u = fm.unpack(fmt, fm.pack(fmt, f, 6, 512), 6, 512)
    for key, val in f.items():
        got = u[key]
        if val.dtype == np.float16:
            assert (got == val.astype(np.float64)).all(), key
        else:
            assert (got.reshape(val.shape) == val.astype(np.int64)).all(), key


def test_dequantize_f32_is_rounded_exact():
    # a Q6_K block whose exact values need 25 bits: fp32 result is RNE
    W = _weights("normal", 2, 256)
    buf = fm.quantize("q6_k", W)
    exact = fm.dequantize("q6_k", buf, 2, 256)
    f32 = fm.dequantize_f32("q6_k", buf, 2, 256)
    assert (np.abs(f32.astype(np.float64) - exact) <= np.abs(exact) * 2.0 ** -24).all()


def test_q6_k_scale_is_fp16_subnormal_at_sigma_0_02():
    # N(0, 0.02) weights give Q6_K d below the fp16 normal range; it is kept
    f = fm.quantize_q6_k(_weights("normal", 4, 1024))
    d = f["d"].astype(np.float64)
    assert (d > 0).all() and (d < 2.0 ** -14).all()
