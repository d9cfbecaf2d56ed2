"""Pins of the int8 activation quantizer and the Q8_0 x int8 GEMV reference:
closed forms, exhaustive nearest-integer search, error bound, brute force."""
import itertools

import numpy as np
import pytest

from oracle import brute
from oracle import formats as fm
from oracle import int8


def test_closed_form_block():
    x = np.zeros((2, 64), np.float32)
    x[0, :6] = [127.0, -63.5, 0.5, -0.5, 1.49, 126.6]   # amax 127 -> d = 1
    x[1, 32] = -2.54                                       # second block: d = 0.02
    q, d = int8.quantize_act_q8(x)
    assert d.dtype == np.float32
    assert d[0, 0] == 1.0 and d[0, 1] == 0.0 and d[1, 0] == 0.0
    assert q[0, :6].tolist() == [127, -64, 1, -1, 1, 127]
    assert (q[0, 6:32] == 0).all() and (q[0, 32:] == 0).all() and (q[1, :32] == 0).all()
    assert q[1, 32] == -127 and d[1, 1] == np.float32(np.float32(2.54) / np.float32(127))


def _nearest_by_search(r):
    """Exhaustive: the integer in [-127, 127] nearest to r, ties away from 0."""
    best, bd = 0, None
    for c in range(-127, 128):
        dd = abs(r - c)
        if bd is None or dd < bd or (dd == bd and abs(c) > abs(best)):
            best, bd = c, dd
    return best


def test_codes_against_exhaustive_search():
    rng = np.random.default_rng(0)
    x = (rng.normal(0, 1, (4, 64)) * np.exp2(rng.integers(-20, 20, (4, 1)))).astype(np.float32)
    x[0, 3] = x[0, :32].max() * np.float32(0.5 / 127 * 21)  # lands near a half
    q, d = int8.quantize_act_q8(x)
    for r, k in itertools.product(range(4), range(64)):
        db = np.float32(d[r, k // 32])
        rr = float(np.float32(x[r, k]) / db) if db > 0 else 0.0
        assert q[r, k] == _nearest_by_search(rr), (r, k)


def test_error_bound_and_extremes():
    rng = np.random.default_rng(1)
    x = (rng.normal(0, 1, (16, 256)) * np.exp2(rng.integers(-30, 30, (16, 1)))).astype(np.float32)
    q, d = int8.quantize_act_q8(x)
    back = int8.dequantize_act_q8(q, d)
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(back - x) <= dd * (0.5 + 1e-6))
    # the largest magnitude of every block maps to +-127
    blk = np.abs(q.astype(np.int64)).reshape(16, 8, 32).max(-1)
    assert (blk == 127).all()


def test_gemv_against_brute_force():
    rng = np.random.default_rng(2)
    N, K, R = 3, 64, 2
    buf = fm.quantize("q8_0", rng.normal(0, 0.02, (N, K)))
    X = rng.normal(0, 1, (R, K)).astype(np.float32)
    y, bound = int8.gemv_q8_0_i8(buf, N, K, X)
    q, d = int8.quantize_act_q8(X)
    for r, n in itertools.product(range(R), range(N)):
        acc = acc_abs = 0.0
        for k in range(K):
            t = brute.element("q8_0", buf, N, K, n, k) * float(q[r, k]) * float(d[r, k // 32])
            acc += t
            acc_abs += abs(t)
        assert y[r, n] == pytest.approx(acc, rel=1e-12, abs=1e-15)
        assert bound[r, n] == pytest.approx(acc_abs, rel=1e-12)
