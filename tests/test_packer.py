"""Budgeted tier planner (host logic): the page's split, the budget rule
against brute force, byte sizes against the oracle's layouts, re-indexing
invariance of routing.  Runs on the CPU (loads the library for its layout
queries only)."""
import itertools

import numpy as np
import pytest

from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import configs, packer, synth


def _oracle_expert_bytes(H, F, fg, fd):
    return 2 * fm.tensor_bytes(fg, F, H) + fm.tensor_bytes(fd, H, F)


def test_unbudgeted_split_is_the_pages_25_55_20_at_512_experts():
    # "Three RTX 3090 Qwen3.8-Flash-Next guide", 优化策略二: top 25 %, middle
    # 55 %, tail 20 % of 512 experts -> 128 / 282 / 102, the tiers of the
    # tiered 512-expert decode and prefill workloads
    imp = np.random.default_rng(0).random(512)
    plan = packer.plan_tiers(imp, 2048, 640)
    assert plan.bounds == ((0, 128), (128, 410), (410, 512))
    assert plan.tiers() == configs.TIERED_TIERS


def test_hot_tier_size_matches_the_pages_figure():
    # the same page's memory picture: the hot tier (Q6_K gate/up, Q8_0 down)
    # takes about 22 GB; its model has 48 hidden layers of 512 experts with
    # hidden 2048 and expert width 640 (the down projection's 640 is named
    # in the same section)
    per_expert = packer.expert_bytes(2048, 640, "q6_k", "q8_0")
    hot = 128 * 48 * per_expert
    assert abs(hot / 1e9 - 22) < 0.05 * 22


@pytest.mark.parametrize("fg,fd", [("q6_k", "q8_0"), ("q4_k", "q4_0"), ("mxfp4", "mxfp4"),
                                   ("q4_0", "q8_0"), ("q8_0", "q6_k")])
@pytest.mark.parametrize("H,F", [(2048, 640), (256, 256), (7168, 2048)])
def test_expert_bytes_match_the_oracle_layouts(fg, fd, H, F):
    if F % fm.BLOCK[fd] or H % fm.BLOCK[fg]:
        with pytest.raises(ValueError, match="multiple of"):
            packer.expert_bytes(H, F, fg, fd)
    else:
        assert packer.expert_bytes(H, F, fg, fd) == _oracle_expert_bytes(H, F, fg, fd)


def test_640_wide_down_rejects_256_value_formats():
    # the page: a 640-wide down projection cannot take a 256-aligned format
    for fd in ("q4_k", "q6_k"):
        with pytest.raises(ValueError, match="down format .* multiple of 256"):
            packer.plan_tiers(np.ones(8), 2048, 640,
                              formats=(("q6_k", fd), ("q4_k", "q4_0"), ("mxfp4", "mxfp4")))
    with pytest.raises(ValueError, match="tier formats"):
        packer.plan_tiers(np.ones(8), 2048, 640,
                          formats=(("t5", "q8_0"), ("q4_k", "q4_0"), ("mxfp4", "mxfp4")))


def test_order_is_descending_importance_ties_to_lower_id():
    rng = np.random.default_rng(3)
    imp = rng.integers(0, 5, size=40).astype(float)     # many ties
    plan = packer.plan_tiers(imp, 256, 256)
    want = sorted(range(40), key=lambda e: (-imp[e], e))
    assert plan.order.tolist() == want
    assert (plan.new_id[plan.order] == np.arange(40)).all()


def _brute_plan(E, H, F, formats, budget):
    """Enumerate every (hot, tail) split: the largest hot tier that fits with
    the page's tail of floor(0.2 E); if none fits, hot = 0 and the smallest
    tail >= floor(0.2 E) that fits."""
    cost = [_oracle_expert_bytes(H, F, fg, fd) for fg, fd in formats]
    size = lambda h, t: h * cost[0] + (E - h - t) * cost[1] + t * cost[2]
    t0 = (E * 20) // 100
    fits = [h for h in range(E - t0 + 1) if size(h, t0) <= budget]
    if fits:
        return max(fits), t0
    tails = [t for t in range(t0, E + 1) if size(0, t) <= budget]
    return (0, min(tails)) if tails else None


@pytest.mark.parametrize("E", [1, 2, 5, 7, 10, 13, 24])
def test_budget_rule_against_brute_force(E):
    H, F = 256, 256
    formats = packer.DEFAULT_FORMATS
    cost = [_oracle_expert_bytes(H, F, fg, fd) for fg, fd in formats]
    imp = np.random.default_rng(E).random(E)
    lo, hi = E * cost[2], E * cost[0] + 1
    budgets = sorted(set(np.linspace(lo - 1, hi, 97).astype(int).tolist()
                         + [E * c for c in cost] + [E * cost[2] - 1]))
    prev_hot, prev_tail = -1, E + 1
    for B in budgets:
        want = _brute_plan(E, H, F, formats, B)
        if want is None:
            with pytest.raises(ValueError, match="below the all-tail size"):
                packer.plan_tiers(imp, H, F, budget_bytes=B)
            continue
        plan = packer.plan_tiers(imp, H, F, budget_bytes=B)
        hot, tail = want
        assert plan.bounds == ((0, hot), (hot, E - tail), (E - tail, E)), (E, B)
        assert plan.bytes <= B
        # a bigger budget never demotes an expert
        assert hot >= prev_hot and tail <= prev_tail
        prev_hot, prev_tail = hot, tail


def test_plan_bytes_and_tier_membership_follow_importance():
    E, H, F = 64, 2048, 640
    imp = np.random.default_rng(5).gamma(0.5, size=E)
    plan = packer.plan_tiers(imp, H, F, budget_bytes=int(1.1 * E * packer.expert_bytes(
        H, F, "q4_k", "q4_0")))
    tier_of = np.empty(E, dtype=int)
    total = 0
    for i, t in enumerate(plan.tiers()):
        orig = plan.order[t.e_begin:t.e_end]
        tier_of[orig] = i
        total += len(orig) * _oracle_expert_bytes(H, F, t.fmt_gate_up, t.fmt_down)
    assert total == plan.bytes
    # every expert of a higher tier is at least as important as any lower one
    for a, b in itertools.combinations(range(len(plan.tiers())), 2):
        assert imp[tier_of == a].min() >= imp[tier_of == b].max()


def test_routing_counts():
    ids = np.array([[0, 3, -1], [3, 3, 9], [5, 0, 12]])
    got = packer.routing_counts(ids, 10)
    want = np.zeros(10)
    for e in ids.reshape(-1):
        if 0 <= e < 10:
            want[e] += 1
    assert (got == want).all()


def test_bad_inputs():
    with pytest.raises(ValueError):
        packer.plan_tiers([], 256, 256)
    with pytest.raises(ValueError, match="finite"):
        packer.plan_tiers([1.0, np.nan], 256, 256)
    with pytest.raises(ValueError, match="most to fewest"):
        packer.plan_tiers(np.ones(4), 256, 256,
                          formats=(("mxfp4", "mxfp4"), ("q4_k", "q4_0"), ("q6_k", "q8_0")))


def test_reindexed_router_selects_the_same_experts():
    # re-indexing the router rows and the logit bias by the plan leaves every
    # token's routing unchanged up to the renaming new id -> order[new id]
    E, H, k, T = 48, 64, 6, 40
    Wr = synth.normal((E, H), 0.05, 1, synth.ROUTER, 0)
    bias = synth.rank_prior(E, 0.5)
    x = synth.normal((T, H), 1.0, 1, synth.ACT, T)
    imp = np.random.default_rng(9).random(E)
    plan = packer.plan_tiers(imp, 256, 256)
    Wn, bn = packer.permute_router(plan, Wr, bias)
    ids0, p0, _ = moe.route(x, Wr, bias, k)
    ids1, p1, _ = moe.route(x, Wn, bn, k)
    assert (plan.order[ids1] == ids0).all()
    assert np.array_equal(p0, p1)
