"""Pins for the oracle's GEMV, routing, permutation, expert FFN and layer.

Checked against things other than the oracle itself:
  * brute force: scalar loops straight from the packed bytes (oracle/brute.py)
    and enumeration of every k-subset for top-k;
  * exact integer arithmetic (grid-exact weights and integer activations);
  * library special cases: NumPy's stable argsort for the permutation;
  * invariants: top-1 routing with weight 1 equals the dense expert FFN,
    reordering tokens reorders outputs, shared-only routing returns the
    shared expert, bounds dominate values.
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import synth


def _expert_bank(H, F, fmts, seed=0):
    """Quantized experts: list of (fmt_gu, gate, up, fmt_d, down)."""
    bank = []
    for e, (fgu, fd) in enumerate(fmts):
        g = fm.quantize(fgu, synth.normal((F, H), 0.02, seed, synth.GATE, e))
        u = fm.quantize(fgu, synth.normal((F, H), 0.02, seed, synth.UP, e))
        d = fm.quantize(fd, synth.normal((H, F), 0.02, seed, synth.DOWN, e))
        bank.append((fgu, g, u, fd, d))
    return bank


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_gemv_matches_scalar_loops(fmt):
    N, K = 3, 256
    W = synth.normal((N, K), 0.02, 1, synth.DENSE)
    buf = fm.quantize(fmt, W)
    x = synth.normal((2, K), 1.0, 1, synth.ACT)
    y, b = moe.gemv(fmt, buf, N, K, x)
    ref = np.array(brute.gemv(fmt, buf, N, K, x))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert (np.abs(y) <= b * (1 + 1e-12)).all()


@pytest.mark.parametrize("fmt", fm.FORMATS)
def test_gemv_grid_exact_integers(fmt):
    """Weights with power-of-two scales and integer activations: every partial
    sum is an exact multiple of a power of two, so the float64 result must
    equal the integer computation exactly."""
    N, K = 5, 512
    rng = np.random.default_rng(11)
    fields = {}
    nb = K // fm.BLOCK[fmt]
    if fmt == "q8_0":
        fields = {"q": rng.integers(-127, 128, (N, K)).astype(np.int8),
                  "d": np.full((N, nb), 2.0 ** -6, dtype=np.float16)}
        qint, scale_num = fields["q"].astype(np.int64), 1
    elif fmt == "q4_0":
        fields = {"q": rng.integers(0, 16, (N, K)).astype(np.uint8),
                  "d": np.full((N, nb), 2.0 ** -6, dtype=np.float16)}
        qint, scale_num = fields["q"].astype(np.int64) - 8, 1
    elif fmt == "mxfp4":
        fields = {"q": rng.integers(0, 16, (N, K)).astype(np.uint8),
                  "e": np.full((N, nb), 127 - 5, dtype=np.uint8)}
        # E2M1 values times 2 are integers: 0,1,2,3,4,6,8,12
        mag2 = np.array([0, 1, 2, 3, 4, 6, 8, 12])
        c = fields["q"].astype(np.int64)
        qint = np.where(c & 8, -mag2[c & 7], mag2[c & 7])
        scale_num = 1                                   # value = qint * 2^-6
    elif fmt == "q4_k":
        sc = rng.integers(0, 64, (N, nb, 8))
        m = rng.integers(0, 64, (N, nb, 8))
        q = rng.integers(0, 16, (N, K))
        fields = {"q": q.astype(np.uint8), "d": np.full((N, nb), 2.0 ** -6, np.float16),
                  "dmin": np.full((N, nb), 2.0 ** -6, np.float16),
                  "sc": sc.astype(np.uint8), "m": m.astype(np.uint8)}
        qint = np.repeat(sc.reshape(N, -1), 32, 1) * q - np.repeat(m.reshape(N, -1), 32, 1)
        scale_num = 1
    else:
        sc = rng.integers(-128, 128, (N, nb, 16))
        q = rng.integers(0, 64, (N, K))
        fields = {"q": q.astype(np.uint8), "sc": sc.astype(np.int8),
                  "d": np.full((N, nb), 2.0 ** -6, np.float16)}
        qint = np.repeat(sc.reshape(N, -1), 16, 1) * (q - 32)
        scale_num = 1
    buf = fm.pack(fmt, fields, N, K)
    x = rng.integers(-3, 4, (3, K))
    y, _ = moe.gemv(fmt, buf, N, K, x.astype(np.float32))
    exact = (x @ qint.T) * scale_num
    assert (y == exact * 2.0 ** -6).all()


def test_topk_matches_subset_enumeration():
    rng = np.random.default_rng(2)
    for trial in range(40):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        logits = rng.standard_normal((1, E)).round(1)      # rounding makes ties
        ids = moe.topk(logits, k)[0]
        assert list(ids) == brute.topk_by_enumeration(list(logits[0]), k)


def test_topk_ties_and_nan():
    logits = np.array([[1.0, 3.0, 3.0, np.nan, 2.0, 3.0]])
    assert list(moe.topk(logits, 4)[0]) == [1, 2, 5, 4]
    assert list(moe.topk(np.full((1, 4), np.nan), 2)[0]) == [0, 1]
    with np.errstate(invalid="ignore"):
        assert list(moe.topk(np.array([[-np.inf, np.nan, -1.0]]), 2)[0]) == [2, 0]


def test_router_logits_scalar_loops():
    """logits[t, e] = sum_h x[t, h] Wr[e, h] + b[e], summed by hand."""
    x = synth.normal((3, 40), 1.0, 5, synth.ACT)
    Wr = synth.normal((7, 40), 0.02, 5, synth.ROUTER)
    b = synth.rank_prior(7, 0.5)
    got = moe.router_logits(x, Wr, b)
    for t in range(3):
        for e in range(7):
            want = sum(float(x[t, h]) * float(Wr[e, h]) for h in range(40)) + float(b[e])
            assert got[t, e] == pytest.approx(want, rel=1e-12, abs=1e-14)
    assert np.array_equal(moe.router_logits(x, Wr), moe.router_logits(x, Wr, np.zeros(7)))


def test_topk_gap_is_the_selection_margin():
    """topk_gap = (smallest kept logit) - (largest dropped logit), with the kept
    set taken from the k-subset enumeration; 0 on a tie across the cut, inf
    when every expert is kept."""
    rng = np.random.default_rng(7)
    for trial in range(60):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        T = 3
        logits = rng.standard_normal((T, E)).round(1)      # rounding makes ties
        gap = moe.topk_gap(logits, k)
        for t in range(T):
            row = [float(v) for v in logits[t]]
            kept = brute.topk_by_enumeration(row, k)
            dropped = [e for e in range(E) if e not in kept]
            want = (min(row[e] for e in kept) - max(row[e] for e in dropped)
                    if dropped else math.inf)
            assert gap[t] == want, (row, k)
            assert gap[t] >= 0
    assert moe.topk_gap(np.array([[1.0, 2.0, 2.0, 0.5]]), 1)[0] == 0.0   # tie at the cut
    assert moe.topk_gap(np.array([[1.0, 2.0, 2.0, 0.5]]), 2)[0] == 1.0
    assert moe.topk_gap(np.array([[1.0, 2.0, 3.0]]), 3)[0] == math.inf


def test_topk_gap_bounds_the_perturbation_that_keeps_the_selection():
    """The property the GPU routing tests rely on: perturbing every logit by
    less than gap / 2 cannot change the kept set (the near-tie protocol
    compares ids only for tokens whose gap exceeds twice the logit error)."""
    rng = np.random.default_rng(8)
    T, E, k = 200, 64, 6
    logits = rng.standard_normal((T, E))
    gap = moe.topk_gap(logits, k)
    base = moe.topk(logits, k)
    for t in range(T):
        err = 0.499 * gap[t]
        for _ in range(5):
            pert = logits[t] + rng.uniform(-err, err, E)
            got = moe.topk(pert[None, :], k)[0]
            assert set(got.tolist()) == set(base[t].tolist())
    # and a perturbation of just over gap / 2 at the two logits across the
    # cut swaps them
    t = 0
    srt = np.argsort(-logits[t], kind="stable")
    pert = logits[t].copy()
    pert[srt[k - 1]] -= 0.51 * gap[t]
    pert[srt[k]] += 0.51 * gap[t]
    got = moe.topk(pert[None, :], k)[0]
    assert srt[k] in got and srt[k - 1] not in got


def test_route_weights():
    x = synth.normal((5, 64), 1.0, 0, synth.ACT)
    Wr = synth.normal((12, 64), 0.02, 0, synth.ROUTER)
    ids, p, logits = moe.route(x, Wr, None, 3)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)
    # weights follow the logit order and equal exp differences exactly
    sel = np.take_along_axis(logits, ids, 1)
    assert (np.diff(sel, axis=1) <= 0).all()
    assert np.allclose(p[:, 1] / p[:, 0], np.exp(sel[:, 1] - sel[:, 0]), rtol=1e-14)
    ids1, p1, _ = moe.route(x, Wr, None, 1)
    assert (p1 == 1.0).all() and (ids1[:, 0] == logits.argmax(1)).all()
    ids_s, p_s, _ = moe.route(x, Wr, None, 2, n_shared=2)
    assert (ids_s[:, 2:] == [12, 13]).all() and (p_s[:, 2:] == 1.0).all()


def test_route_bias_shifts_selection():
    x = synth.normal((1, 16), 1.0, 0, synth.ACT)
    Wr = np.zeros((6, 16), np.float32)
    b = np.array([0, 0, 5, 0, 0, 4], np.float32)
    ids, p, _ = moe.route(x, Wr, b, 2)
    assert list(ids[0]) == [2, 5]
    assert np.isclose(p[0, 0], 1 / (1 + np.exp(-1.0)), rtol=1e-15)


@pytest.mark.parametrize("seed", range(4))
def test_permute_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    T, k, E = 37, 5, 9
    ids = rng.integers(-2, E + 2, (T, k)).astype(np.int32)   # includes invalid ids
    ids[3] = -1
    offsets, perm, inv = moe.permute(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert (offsets == np.concatenate([[0], np.cumsum(counts)])).all()
    order = np.argsort(np.where(valid, flat, E), kind="stable")[:valid.sum()]
    n = valid.sum()
    assert (perm[:n] == order).all() and (perm[n:] == -1).all()
    assert (inv[~valid] == -1).all()
    assert (inv[perm[:n]] == np.arange(n)).all()


def test_permute_degenerate():
    offsets, perm, inv = moe.permute(np.zeros((0, 3), np.int32), 4)
    assert list(offsets) == [0] * 5 and perm.size == 0
    offsets, perm, inv = moe.permute(np.full((6, 2), 2, np.int32), 4)  # one expert takes all
    assert list(offsets) == [0, 0, 0, 12, 12] and list(perm) == list(range(12))


def test_top1_weight1_equals_dense_ffn():
    H, F = 256, 32
    bank = _expert_bank(H, F, [("q8_0", "q8_0"), ("q4_k", "q4_0"), ("mxfp4", "mxfp4")])
    x = synth.normal((4, H), 1.0, 3, synth.ACT)
    for e in range(3):
        ids = np.full((4, 1), e, np.int32)
        y, b = moe.moe_layer(x, ids, np.ones((4, 1)), lambda i: bank[i], H, F, 3)
        r = moe.expert_ffn(bank[e], H, F, x)
        assert (y == r["o"]).all() and (b == r["bound_o"]).all()


def test_layer_matches_brute_force_q8_0():
    H, F, E, k, T = 64, 32, 4, 2, 3
    bank = _expert_bank(H, F, [("q8_0", "q8_0")] * E)
    x = synth.normal((T, H), 1.0, 4, synth.ACT)
    Wr = synth.normal((E, H), 0.02, 4, synth.ROUTER)
    ids, p, _ = moe.route(x, Wr, None, k)
    y, b = moe.moe_layer(x, ids, p, lambda i: bank[i], H, F, E)
    ref = np.array(brute.moe_layer(x, ids, p, lambda i: bank[i], H, F, E))
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-14)
    assert (np.abs(y) <= b * (1 + 1e-12)).all()


def test_layer_matches_brute_force_tiered():
    H, F, E = 256, 64, 6
    tiers = [("q6_k", "q8_0")] * 2 + [("q4_k", "q4_0")] * 2 + [("mxfp4", "mxfp4")] * 2
    bank = _expert_bank(H, F, tiers, seed=5)
    x = synth.normal((2, H), 1.0, 5, synth.ACT)
    ids = np.array([[0, 2, 4], [5, 3, 1]], np.int32)
    p = synth.random_weights(2, 3, 5)
    y, _ = moe.moe_layer(x, ids, p, lambda i: bank[i], H, F, E)
    ref = np.array(brute.moe_layer(x, ids, p, lambda i: bank[i], H, F, E))
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-14)


def test_token_reorder_invariance():
    H, F, E, k, T = 64, 32, 5, 2, 7
    bank = _expert_bank(H, F, [("q8_0", "q4_0")] * E)
    x = synth.normal((T, H), 1.0, 6, synth.ACT)
    Wr = synth.normal((E, H), 0.02, 6, synth.ROUTER)
    ids, p, _ = moe.route(x, Wr, None, k)
    y, _ = moe.moe_layer(x, ids, p, lambda i: bank[i], H, F, E)
    sigma = np.random.default_rng(0).permutation(T)
    ids2, p2, _ = moe.route(x[sigma], Wr, None, k)
    assert (ids2 == ids[sigma]).all()
    y2, _ = moe.moe_layer(x[sigma], ids2, p2, lambda i: bank[i], H, F, E)
    assert np.allclose(y2, y[sigma], rtol=1e-13, atol=1e-16)


def test_permuted_ffn_plus_combine_equals_layer():
    H, F, E, k, T = 64, 32, 6, 3, 5
    bank = _expert_bank(H, F, [("q8_0", "q8_0")] * E, seed=8)
    x = synth.normal((T, H), 1.0, 8, synth.ACT)
    ids = synth.random_ids(T, k, E, 8)
    ids[1, 2] = -1                                            # skipped slot
    ids[2, 0] = E + 3                                         # out of range: skipped
    p = synth.random_weights(T, k, 8)
    offsets, perm, inv = moe.permute(ids, E)
    o, bo = moe.ffn_permuted(x, ids, offsets, perm, lambda i: bank[i], H, F, k)
    y, b = moe.combine(o, inv, p, T, k)
    y2, b2 = moe.moe_layer(x, ids, p, lambda i: bank[i], H, F, E)
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-16)
    assert (np.isnan(o[offsets[-1]:])).all()


def test_shared_only_gives_shared():
    T, k, H = 3, 2, 16
    shared = synth.normal((T, H), 1.0, 9, synth.ACT)
    o = np.zeros((0, H))
    y, b = moe.combine(o, np.full(T * k, -1), np.ones((T, k)), T, k, shared=shared)
    assert (y == shared).all()


def test_rank_prior_tier_shares():
    """With the calibrated prior (lam = 0.5) the hot tier [0,128) takes about
    85 % of the 512-expert top-10 assignments, and every tier is used -- the
    frequency skew the tiering relies on."""
    E, H, k, T = 512, 2048, 10, 400
    x = synth.normal((T, H), 1.0, 0, synth.ACT)
    Wr = synth.normal((E, H), 0.02, 0, synth.ROUTER)
    ids, _, _ = moe.route(x, Wr, synth.rank_prior(E, 0.5), k)
    hot = (ids < 128).mean()
    cold = (ids >= 410).mean()
    assert 0.78 < hot < 0.92 and cold > 0.002
