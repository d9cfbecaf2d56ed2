"""GPU parity of moe_route and moe_permute.

Routing ids are integers decided by floating point: the device decides in
fp32, the oracle in fp64.  The test requires (a) the device ids to be the
exact top-k of the device's own fp32 logits (checked as a property: chosen
logits dominate the rest, ties to the lower id), (b) device logits within the
fp32 dot-product bound of the oracle's, and (c) device ids equal to the oracle
ids on every token whose fp64 decision margin exceeds twice that token's
largest logit error; tokens inside that margin are counted and their ids
checked to be a valid top-k under the tolerance.
"""
import numpy as np
import pytest

from gpu_util import requires_gpu, to_gpu, to_np, assert_within_bound, torch
from oracle import moe
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _check_topk_property(logits, ids, k):
    """ids[t] is the top-k of logits[t] (descending, ties to lower id)."""
    T, E = logits.shape
    for t in range(T):
        key = np.where(np.isnan(logits[t]), -np.inf, logits[t])
        order = np.lexsort((np.arange(E), -key))[:k]
        assert list(ids[t, :k]) == list(order), t


def _route_case(T, H, E, k, bias, x_dtype="f32", dup_rows=False, n_shared=0, seed=0):
    x = synth.normal((T, H), 1.0, seed, synth.ACT, T)
    if x_dtype == "bf16":
        x = synth.bf16_round(x)
    Wr = synth.normal((E, H), 0.02, seed, synth.ROUTER)
    if dup_rows:
        Wr[E // 2] = Wr[1]          # exact ties between experts 1 and E/2
        Wr[E - 1] = Wr[1]
    b = synth.rank_prior(E, 0.5) if bias else None
    xg = to_gpu(x) if x_dtype == "f32" else to_gpu(x).to(torch.bfloat16)
    ids, p, lg = qmoe.route(xg, to_gpu(Wr), None if b is None else to_gpu(b), k,
                            n_shared=n_shared, logits=True)
    ids, p, lg = to_np(ids), to_np(p), to_np(lg)
    ids_ref, p_ref, lg_ref = moe.route(x, Wr, b, k, n_shared=n_shared)
    # (b) logits within the dot-product bound
    bound = np.abs(x.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    if b is not None:
        bound = bound + np.abs(b.astype(np.float64))
    assert_within_bound(lg, lg_ref, bound, rel=1e-5, what="router logits")
    # (a) ids are the exact top-k of the device logits
    _check_topk_property(lg, ids, k)
    # (c) agreement with the fp64 decision outside the near-tie margin
    err = np.abs(lg.astype(np.float64) - lg_ref).max(axis=1)
    gap = moe.topk_gap(lg_ref, k)
    decided = gap > 2 * err
    assert (ids[decided, :k] == ids_ref[decided, :k]).all()
    # weights: a logit error of at most eps moves log p_i by at most 2 eps, so
    # |dp_i| <= p_i (2 eps + fp32 rounding of exp and the division)
    same = (ids == ids_ref).all(axis=1)
    eps = err[same][:, None]
    tol = p_ref[same] * (2.0 * eps + 1e-6) + 1e-7
    assert (np.abs(p[same] - p_ref[same]) <= tol).all()
    assert np.allclose(p[:, :k].sum(1), 1.0, atol=1e-6)
    if n_shared:
        assert (ids[:, k:] == np.arange(E, E + n_shared)).all() and (p[:, k:] == 1.0).all()
    return int((~decided).sum())


@pytest.mark.parametrize("T,H,E,k,bias", [(4, 512, 16, 2, False), (1, 2048, 512, 10, True),
                                          (6, 2048, 512, 10, True), (16, 7168, 256, 8, False),
                                          (64, 2048, 512, 10, True), (33, 256, 40, 5, False)])
def test_route(T, H, E, k, bias):
    _route_case(T, H, E, k, bias)


def test_route_prefill_chunk():
    """2048 rows through the fp32 router GEMM path; near-ties are reported."""
    near = _route_case(2048, 2048, 512, 10, True)
    assert near < 20


def test_route_bf16_and_shared():
    _route_case(16, 7168, 256, 8, False, x_dtype="bf16", n_shared=1)


def test_route_exact_ties_go_to_lower_id():
    T, H, E, k = 8, 256, 64, 6
    x = synth.normal((T, H), 1.0, 3, synth.ACT)
    Wr = synth.normal((E, H), 0.02, 3, synth.ROUTER)
    Wr[40] = Wr[7]
    Wr[63] = Wr[7]
    Wr[7] *= 0
    Wr[7] += np.float32(0.05) * x.mean(0)          # make 7 (and its twins) popular
    Wr[40] = Wr[7]
    Wr[63] = Wr[7]
    ids, p, lg = qmoe.route(to_gpu(x), to_gpu(Wr), None, k, logits=True)
    ids, lg = to_np(ids), to_np(lg)
    assert (lg[:, 7] == lg[:, 40]).all() and (lg[:, 7] == lg[:, 63]).all()
    _check_topk_property(lg, ids, k)
    for t in range(T):
        row = list(ids[t])
        if 40 in row:
            assert 7 in row and row.index(7) < row.index(40)


@pytest.mark.parametrize("T,E,k,period", [(6, 512, 10, 64), (6, 512, 10, 32), (16, 256, 9, 16),
                                           (3, 300, 12, 64), (2, 512, 64, 8)])
def test_route_ties_within_and_across_lanes(T, E, k, period):
    """Experts e and e + period share a router row, so their logits are exactly
    equal: with period 64 every lane of the top-k wave holds equal keys in all
    its slots (ties within a lane), with 32, 16 or 8 also across lanes.  Both
    the chunk path (moe_route) and the fused decode routing must pick the
    top k by logit with ties to the lower id, in that order."""
    H = 256
    x = synth.normal((T, H), 1.0, 21, synth.ACT, T)
    base = synth.normal((period, H), 0.02, 21, synth.ROUTER)
    Wr = np.ascontiguousarray(base[np.arange(E) % period])
    ids, p, lg = qmoe.route(to_gpu(x), to_gpu(Wr), None, k, logits=True)
    ids, lg = to_np(ids), to_np(lg)
    assert (lg[:, :period] == lg[:, period:2 * period]).all()
    _check_topk_property(lg, ids, k)
    got = _route_decode_vs_two_calls(to_gpu(x), to_gpu(Wr), None, k)
    _check_topk_property(to_np(got[5]), to_np(got[0]), k)


def test_route_k1_weights_are_one():
    x = synth.normal((5, 512), 1.0, 4, synth.ACT)
    Wr = synth.normal((16, 512), 0.02, 4, synth.ROUTER)
    ids, p = qmoe.route(to_gpu(x), to_gpu(Wr), None, 1)
    assert (to_np(p) == 1.0).all()


def test_route_nan_row_does_not_crash():
    x = synth.normal((3, 256), 1.0, 5, synth.ACT)
    x[1, 7] = np.nan
    Wr = synth.normal((16, 256), 0.02, 5, synth.ROUTER)
    ids, p = qmoe.route(to_gpu(x), to_gpu(Wr), None, 4)
    ids, p = to_np(ids), to_np(p)
    assert list(ids[1]) == [0, 1, 2, 3]               # NaN ranks last: lowest ids
    assert np.isfinite(p[0]).all() and np.isfinite(p[2]).all()


# ------------------------------------------------------------- permute ---

@pytest.mark.parametrize("T,k,E", [(1, 10, 512), (6, 10, 512), (16, 9, 257), (4, 2, 16),
                                   (2048, 10, 512), (3000, 7, 8192), (1, 1, 1), (700, 64, 33)])
def test_permute_bitexact(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(-3, E + 3, (T, k)).astype(np.int32)   # invalid ids and duplicates
    ids[rng.random((T, k)) < 0.05] = -1
    off, perm, inv = (to_np(t) for t in qmoe.permute(to_gpu(ids), E))
    off_r, perm_r, inv_r = moe.permute(ids, E)
    assert (off == off_r).all() and (perm == perm_r).all() and (inv == inv_r).all()


def test_permute_one_expert_takes_all_and_all_invalid():
    ids = np.full((100, 4), 3, np.int32)
    off, perm, inv = (to_np(t) for t in qmoe.permute(to_gpu(ids), 8))
    assert list(off) == [0, 0, 0, 0, 400, 400, 400, 400, 400]
    assert (perm == np.arange(400)).all() and (inv == np.arange(400)).all()
    ids = np.full((5, 3), -1, np.int32)
    off, perm, inv = (to_np(t) for t in qmoe.permute(to_gpu(ids), 8))
    assert (off == 0).all() and (perm == -1).all() and (inv == -1).all()


def test_permute_is_deterministic_and_stable_under_repeat():
    rng = np.random.default_rng(1)
    ids = to_gpu(rng.integers(0, 512, (2048, 10)).astype(np.int32))
    a = [to_np(t) for t in qmoe.permute(ids, 512)]
    b = [to_np(t) for t in qmoe.permute(ids, 512)]
    assert all((x == y).all() for x, y in zip(a, b))


# ------------------------------------------------- fused decode routing ---

def _route_decode_vs_two_calls(x, Wr, b, k, n_shared=0, ws=None):
    """moe_route_decode must reproduce moe_route + moe_permute bit for bit
    (same fp32 sums in the same order, same top-k and the same sort)."""
    E = Wr.shape[0]
    ids, p, lg = qmoe.route(x, Wr, b, k, n_shared=n_shared, logits=True)
    off, perm, inv = qmoe.permute(ids, E + n_shared)
    got = qmoe.route_decode(x, Wr, b, k, n_shared=n_shared, logits=True, ws=ws)
    want = (ids, p, off, perm, inv, lg)
    for name, g, w in zip(("ids", "p", "offsets", "perm", "inv", "logits"), got, want):
        g, w = to_np(g), to_np(w)
        assert g.shape == w.shape, name
        assert np.array_equal(g, w, equal_nan=True), name
    # and the permutation is the oracle's sort of those ids
    off_r, perm_r, inv_r = moe.permute(to_np(ids), E + n_shared)
    assert (to_np(got[2]) == off_r).all() and (to_np(got[3]) == perm_r).all()
    assert (to_np(got[4]) == inv_r).all()
    return got


@pytest.mark.parametrize("T,H,E,k,bias,n_shared,dt", [
    (1, 2048, 512, 10, True, 0, "f32"), (6, 2048, 512, 10, True, 0, "f32"),
    (16, 7168, 256, 8, False, 1, "bf16"), (4, 512, 16, 2, False, 0, "f32"),
    (3, 256, 40, 5, False, 2, "f32"), (16, 4096, 512, 8, True, 0, "bf16"), (2, 1024, 500, 6, True, 3, "f32"),
    (1, 7168, 1, 1, False, 0, "f32"), (9, 3072, 129, 64, False, 0, "f32")])
def test_route_decode_matches_route_then_permute(T, H, E, k, bias, n_shared, dt):
    x = synth.normal((T, H), 1.0, 11, synth.ACT, T)
    Wr = synth.normal((E, H), 0.02, 11, synth.ROUTER)
    b = to_gpu(synth.rank_prior(E, 0.5)) if bias else None
    xg = to_gpu(x) if dt == "f32" else to_gpu(x).to(torch.bfloat16)
    _route_decode_vs_two_calls(xg, to_gpu(Wr), b, k, n_shared)


def test_route_decode_ties_and_nan():
    T, H, E, k = 8, 256, 64, 6
    x = synth.normal((T, H), 1.0, 3, synth.ACT)
    Wr = synth.normal((E, H), 0.02, 3, synth.ROUTER)
    Wr[7] = np.float32(0.05) * x.mean(0)
    Wr[40] = Wr[7]
    Wr[63] = Wr[7]
    x[5, 3] = np.nan
    got = _route_decode_vs_two_calls(to_gpu(x), to_gpu(Wr), None, k)
    assert list(to_np(got[0])[5]) == [0, 1, 2, 3, 4, 5]


def test_route_decode_reuses_its_workspace():
    """The workspace counters return to zero: back-to-back calls on one
    workspace, with different inputs and fewer rows, stay exact."""
    H, E, k = 2048, 512, 10
    ws = qmoe.route_decode_workspace(16, H, E)
    Wr = to_gpu(synth.normal((E, H), 0.02, 12, synth.ROUTER))
    for i, T in enumerate((16, 16, 5, 1, 16)):
        x = to_gpu(synth.normal((T, H), 1.0, 20 + i, synth.ACT, T))
        _route_decode_vs_two_calls(x, Wr, None, k, ws=ws)
    assert (to_np(ws[:256]) == 0).all()


def test_route_decode_zero_rows_zero_offsets():
    Wr = to_gpu(synth.normal((32, 256), 0.02, 1, synth.ROUTER))
    x = torch.zeros((0, 256), dtype=torch.float32, device="cuda")
    ids, p, off, perm, inv = qmoe.route_decode(x, Wr, None, 4, n_shared=1)
    torch.cuda.synchronize()
    assert off.shape == (34,) and (to_np(off) == 0).all()
