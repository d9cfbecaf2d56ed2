"""Pins for the oracle's ternary format T5 ("t5_g128_fp16"; CPU only).

The format is the one the "RTX 4080 SUPER native Windows 27B: NInfer 80 SM
port" page describes in section 九.2: ternary codes packed base-3, five weights
per byte, one FP16 scale per 128 weights, 1.75 bits per weight.  Each check
ties oracle/formats.py to something other than itself:
  * hand-built groups with hand-worked values (tests/golden/t5_blocks.txt);
  * every one of the 243 code bytes against a separate enumeration of the
    five-digit base-3 numbers;
  * the quantizer: every code is the best of {-1, 0, +1} for the stored
    scale, and the scale is the fp16 nearest to the exact mean |w| (computed
    with rationals);
  * exact round trips on values that lie on the grid;
  * the element-by-element reader of oracle/brute.py on random bytes, and the
    GEMV against its scalar loops.
"""
import fractions
import itertools
import os
import struct

import numpy as np
import pytest

from oracle import brute
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "t5_blocks.txt")


def _golden():
    layouts, values = [], {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "layout":
            layouts.append((line[1], int(line[2]), int(line[3]),
                            [int(v) for v in line[4].split(",")], int(line[5])))
        elif line[0] == "value":
            values.setdefault(line[1], []).append((int(line[2]), float(line[3])))
    return layouts, values


def _group(codes, d):
    assert len(codes) == 26
    return bytes(codes) + struct.pack("<e", d)


def _hand_built(case):
    if case == "t5_a":
        codes = [0, 242, 121, 196, 5] + [121] * 20 + [119]
        buf = bytearray(256)
        buf[0:28] = _group(codes, 0.5)
        return 1, 128, buf
    if case == "t5_b":
        buf = bytearray(256)
        zero = [121] * 26
        for blk in range(4):                    # row-major [N][nb] groups
            codes, d = (([242] + [121] * 25), 2.0) if blk == 3 else (zero, 1.0)
            buf[28 * blk:28 * blk + 28] = _group(codes, d)
        return 2, 256, buf
    raise KeyError(case)


def test_t5_layout_and_bits_per_weight():
    layouts, _ = _golden()
    for fmt, N, K, offs, total in layouts:
        o, t = fm.plane_offsets(fmt, N, K)
        assert o == offs and t == total, (fmt, N, K)
    assert fm.tensor_bytes("t5", 4096, 4096) * 8 / (4096 * 4096) == 1.75


@pytest.mark.parametrize("case", ["t5_a", "t5_b"])
def test_t5_closed_form_groups(case):
    _, values = _golden()
    N, K, buf = _hand_built(case)
    D = fm.dequantize("t5", np.frombuffer(bytes(buf), np.uint8), N, K).reshape(-1)
    for idx, expect in values[case]:
        assert D[idx] == expect, (case, idx, D[idx], expect)
        n, k = divmod(idx, K)
        assert brute.element("t5", bytes(buf), N, K, n, k) == expect


def test_t5_every_code_byte():
    # row r's first code byte is the r-th five-digit base-3 number, digits
    # enumerated most significant first by itertools (independent of the
    # oracle's repeated division)
    numbers = list(itertools.product(range(3), repeat=5))   # (c4, c3, c2, c1, c0)
    N, K = len(numbers), 128
    buf = bytearray(fm.tensor_bytes("t5", N, K))
    for r, digits in enumerate(numbers):
        c4, c3, c2, c1, c0 = digits
        code = c0 + 3 * c1 + 9 * c2 + 27 * c3 + 81 * c4
        assert code == r
        buf[28 * r:28 * r + 28] = _group([code] + [121] * 25, 1.0)
    D = fm.dequantize("t5", np.frombuffer(bytes(buf), np.uint8), N, K)
    for r, (c4, c3, c2, c1, c0) in enumerate(numbers):
        assert list(D[r, :5]) == [c0 - 1, c1 - 1, c2 - 1, c3 - 1, c4 - 1], r
        assert (D[r, 5:] == 0).all()


def _nearest_f16_is(d16, exact):
    """d16 is an fp16 value nearest to the rational `exact` (ties allowed)."""
    d = np.float16(d16)
    nb = [np.nextafter(d, np.float16(-np.inf)), np.nextafter(d, np.float16(np.inf))]
    err = abs(fractions.Fraction(float(d)) - exact)
    return all(err <= abs(fractions.Fraction(float(v)) - exact) for v in nb if np.isfinite(v))


@pytest.mark.parametrize("kind", ["normal", "heavy", "zeros_and_ties"])
def test_t5_quantizer_codes_are_optimal_for_the_scale(kind):
    rng = np.random.default_rng(3)
    W = synth.normal((4, 512), 0.02, 2, synth.DENSE)
    if kind == "heavy":
        W = (W * rng.standard_t(2, W.shape).astype(np.float32)).astype(np.float32)
    if kind == "zeros_and_ties":
        W[0, :128] = 0.0                               # all-zero group
        W[1, :128] = np.float32(0.25)                  # mean |w| = 0.25, t = +1
        W[1, 0:4] = [0.375, -0.375, 0.125, -0.125]     # halfway cases of 0.25
    f = fm.quantize_t5(W)
    d = np.repeat(f["d"].astype(np.float64).reshape(4, -1), 128, axis=1)
    t = f["t"].astype(np.float64)
    w = W.astype(np.float64)
    err = np.abs(w - d * t)
    best = np.min(np.abs(w[..., None] - d[..., None] * np.array([-1.0, 0.0, 1.0])), axis=-1)
    assert (err <= best).all()
    for n in range(4):
        for g in range(4):
            blk = W[n, 128 * g:128 * g + 128]
            exact = sum(fractions.Fraction(float(v)).__abs__() for v in blk) / 128
            assert _nearest_f16_is(f["d"][n, g], exact), (n, g)
    if kind == "zeros_and_ties":
        assert f["d"][0, 0] == 0 and (f["t"][0, :128] == 0).all()
        # 0.375 / 0.25 = 1.5 rounds away from zero and clamps to 1; 0.125 / 0.25 = 0.5 -> 1
        assert list(f["t"][1, :4]) == [1, -1, 1, -1]


def test_t5_round_trip_on_grid():
    rng = np.random.default_rng(4)
    d = 2.0 ** -6
    t = rng.choice([-1.0, 1.0], size=(3, 256))          # no zeros: mean |w| = d
    W = (d * t).astype(np.float32)
    buf = fm.quantize("t5", W)
    assert (fm.dequantize("t5", buf, 3, 256) == W.astype(np.float64)).all()


def test_t5_two_readers_agree_on_random_bytes():
    rng = np.random.default_rng(5)
    N, K = 3, 384
    buf = np.zeros(fm.tensor_bytes("t5", N, K), np.uint8)
    grp = buf[:N * (K // 128) * 28].reshape(-1, 28)
    grp[:, :26] = rng.integers(0, 243, (grp.shape[0], 26))
    grp[:, 26:28] = np.frombuffer(rng.standard_normal(grp.shape[0]).astype("<f2").tobytes(),
                                  np.uint8).reshape(-1, 2)
    D = fm.dequantize("t5", buf, N, K)
    for n in range(N):
        for k in range(0, K, 5):
            assert D[n, k] == brute.element("t5", bytes(buf), N, K, n, k), (n, k)


def test_t5_pack_unpack_fields():
    W = synth.normal((6, 512), 0.02, 1, synth.DENSE)
    f = fm.quantize_t5(W)
    u = fm.unpack("t5", fm.pack("t5", f, 6, 512), 6, 512)
    assert (u["t"] == f["t"].astype(np.int64)).all()
    assert (u["d"] == f["d"].astype(np.float64)).all()


def test_t5_gemv_matches_scalar_loops():
    N, K = 3, 256
    buf = fm.quantize("t5", synth.normal((N, K), 0.02, 1, synth.DENSE))
    x = synth.normal((2, K), 1.0, 1, synth.ACT)
    y, b = moe.gemv("t5", buf, N, K, x)
    ref = np.array(brute.gemv("t5", buf, N, K, x))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert (np.abs(y) <= b * (1 + 1e-12)).all()
