"""Helpers for the GPU parity tests (test infrastructure)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import formats as fm  # noqa: E402

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def to_gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_bitexact(got, ref, what=""):
    got = np.asarray(got, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    if not same.all():
        i = np.argwhere(~same)[0]
        raise AssertionError(f"{what}: {(~same).sum()} values differ; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} want {ref[tuple(i)]!r}")


def assert_within_bound(got, ref, bound, rel=1e-3, what=""):
    """|got - ref| <= rel * bound element-wise (the parity bar for floats:
    1e-3 x sum |w x| of each output)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    err = np.abs(got - ref)
    lim = rel * bound + 1e-30
    bad = ~(err <= lim)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; worst ratio "
                             f"{np.nanmax(err / lim):.3g}; first at {i}: got {got[i]} want "
                             f"{ref[i]} bound {bound[i]}")
    return float(np.max(err / lim)) if err.size else 0.0


def oracle_expert(layer, e):
    """(fmt_gu, gate, up, fmt_d, down) packed by the oracle's quantizer from the
    layer's fp32 weights of expert e."""
    t = layer.cfg.tier_of(e)
    wg, wu, wd = layer.expert_fp32(e)
    return (t.fmt_gate_up, fm.quantize(t.fmt_gate_up, wg), fm.quantize(t.fmt_gate_up, wu),
            t.fmt_down, fm.quantize(t.fmt_down, wd))


class ExpertCache:
    def __init__(self, layer):
        self.layer = layer
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            self.cache[e] = oracle_expert(self.layer, e)
        return self.cache[e]
