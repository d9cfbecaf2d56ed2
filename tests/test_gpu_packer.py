"""A bank packed by the tier planner runs through the layer kernels and
computes the original layer's function: routing and output in original ids
against the oracle, with each expert quantized in the format of its tier."""
import dataclasses

import numpy as np
import pytest

from gpu_util import requires_gpu, to_np, assert_within_bound, torch
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import layers, packer, synth
from decode_moe_mul_amd.configs import MoEConfig, Tier

pytestmark = [pytest.mark.gpu, requires_gpu]

BASE = MoEConfig("packed_e24", H=256, E=24, k=4, F=320, tiers=(Tier(0, 24, "q8_0", "q8_0"),),
                 rows=(6,), prior_lambda=0.5, seed=11)


def _plan(plain):
    c = BASE
    Wr, bias = to_np(plain.Wr), to_np(plain.bias)
    calib = synth.normal((256, c.H), 1.0, 5, synth.ACT, 256)
    ids, _, _ = moe.route(calib, Wr, bias, c.k)
    imp = packer.routing_counts(ids, c.E)
    cost = [packer.expert_bytes(c.H, c.F, fg, fd) for fg, fd in packer.DEFAULT_FORMATS]
    budget = c.E * cost[1] + 5 * (cost[0] - cost[1])        # room for about 7 hot experts
    plan = packer.plan_tiers(imp, c.H, c.F, budget_bytes=budget)
    assert len(plan.tiers()) == 3
    return plan, Wr, bias


_cache = {}


def _packed():
    """(packed layer, plan, original router rows, original bias, original-id layer)"""
    if "layer" not in _cache:
        plain = layers.MoELayer(BASE)          # original ids: expert e's weights, router row e
        plan, Wr, bias = _plan(plain)
        cfg = dataclasses.replace(BASE, tiers=plan.tiers())
        _cache["layer"] = (layers.MoELayer(cfg, order=plan.order), plan, Wr, bias, plain)
    return _cache["layer"]


def test_pack_bank_matches_the_layers_banks():
    layer, plan, _, _, plain = _packed()
    c = layer.cfg
    packed = packer.pack_bank(plan, c.H, c.F, plain.expert_fp32_device)
    Wn, bn = packer.permute_router(plan, plain.Wr, plain.bias)
    assert torch.equal(layer.Wr, Wn) and torch.equal(layer.bias, bn)
    assert len(packed) == len(layer.banks[0])
    for (b, e, fg, fd, g, u, d), t, (lg, lu, ld) in zip(packed, plan.tiers(), layer.banks[0]):
        assert (b, e, fg, fd) == (t.e_begin, t.e_end, t.fmt_gate_up, t.fmt_down)
        for got, want in ((g, lg), (u, lu), (d, ld)):
            assert torch.equal(got, want)


@pytest.mark.parametrize("T,prefill", [(1, False), (6, False), (16, False), (40, True)])
def test_packed_layer_equals_the_original_layer(T, prefill):
    layer, plan, Wr, bias, plain = _packed()
    c = layer.cfg
    x = synth.normal((T, c.H), 1.0, 21, synth.ACT, T)
    y, ws = layer.forward(torch.from_numpy(x).cuda(), prefill=prefill)
    y = to_np(y)
    ids_new = to_np(ws["ids"])
    # the oracle routes with the original router and bias, in original ids
    ids_ref, p_ref, lg = moe.route(x, Wr, bias, c.k)
    lg_bound = np.abs(x.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    decided = moe.topk_gap(lg, c.k) > 2 * 1e-5 * lg_bound.max(axis=1)
    same = (plan.order[ids_new] == ids_ref).all(axis=1)
    assert same[decided].all()
    rows = np.flatnonzero(same)
    assert rows.size > 0
    new_id = plan.new_id
    cache = {}

    def expert(e):                      # original id e, in its planned tier's formats
        if e not in cache:
            t = c.tier_of(int(new_id[e]))
            wg, wu, wd = plain.expert_fp32(e)
            cache[e] = (t.fmt_gate_up, fm.quantize(t.fmt_gate_up, wg),
                        fm.quantize(t.fmt_gate_up, wu), t.fmt_down, fm.quantize(t.fmt_down, wd))
        return cache[e]

    y_ref, bound = moe.moe_layer(x[rows], ids_ref[rows], p_ref[rows], expert, c.H, c.F, c.E)
    assert_within_bound(y[rows], y_ref, bound, what=f"packed layer T={T}")
