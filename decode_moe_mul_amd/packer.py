"""Budgeted tier planning and packing of a routed-expert bank.

The "Three RTX 3090 Qwen3.8-Flash-Next guide" page describes an offline
packer (sections 优化策略一 and 优化策略二, and the offline repacking step of
its deployment walk-through):
  * experts are ranked by an importance score (the page uses the routing
    frequency recorded in an importance matrix) and re-indexed in that order,
    so that a precision tier is a contiguous range of expert ids;
  * the ranked experts are split into three tiers: the top 25 % in the
    highest-precision formats (Q6_K gate/up, Q8_0 down), the middle 55 % in
    4-bit formats and the tail 20 % in the lowest (MXFP4 for down), under a
    byte budget;
  * a down projection whose inner width (F = 640 there) is not a multiple of
    256 cannot take a 256-value block format, so the down formats are all
    32-value block formats.

``plan_tiers`` makes that decision for one bank of E experts (hidden H, FFN
width F):
  * order: descending importance, ties to the lower original id;
  * without a budget: hot = round(0.25 E), tail = floor(0.20 E), middle = the
    rest (128 / 282 / 102 for E = 512);
  * with a budget (bytes of expert weights): the tail keeps floor(0.20 E)
    experts and the hot tier takes as many of the most important experts as
    fit with everyone else in the middle tier; when even an empty hot tier
    does not fit, the tail grows from the least important end until the bank
    fits.  A budget below the all-tail size is an error.
The page gives the fractions and the budget but not how the two interact;
the rules above are this module's reading.

``pack_bank`` quantizes the experts in the plan's order with the library's
device quantizer into one buffer per tier and matrix, and ``permute_router``
re-indexes the router rows and the per-expert logit bias the same way, so the
re-indexed layer computes the same function: output row t is unchanged and
routed id j of the new layer is original id ``order[j]``.
"""
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

from . import configs as C
from . import qmoe

# (gate/up, down) formats per tier, most bytes first.  The 4-bit middle tier
# uses Q4_K / Q4_0 where the page names IQ4_XS / IQ4_NL, which this library
# does not implement; the tail's gate/up uses MXFP4 in place of IQ3_XXS.
DEFAULT_FORMATS = (("q6_k", "q8_0"), ("q4_k", "q4_0"), ("mxfp4", "mxfp4"))
FRACTIONS = (0.25, 0.55, 0.20)
TIER_FORMATS = ("q8_0", "q4_0", "mxfp4", "q4_k", "q6_k")


def _block(fmt):
    return qmoe.lib().qmoe_block_size(qmoe.FORMATS[fmt])


def expert_bytes(H, F, fmt_gate_up, fmt_down):
    """Bytes of one expert: gate and up [F, H], down [H, F]."""
    for fmt, K, what in ((fmt_gate_up, H, "gate/up"), (fmt_down, F, "down")):
        if fmt not in TIER_FORMATS:
            raise ValueError(f"{fmt!r} is not one of the expert tier formats {TIER_FORMATS}")
        if K % _block(fmt):
            raise ValueError(f"{what} format {fmt} needs its inner width {K} to be a "
                             f"multiple of {_block(fmt)}")
    return 2 * qmoe.tensor_bytes(fmt_gate_up, F, H) + qmoe.tensor_bytes(fmt_down, H, F)


@dataclass(frozen=True)
class TierPlan:
    order: np.ndarray                      # new id -> original expert id
    bounds: Tuple[Tuple[int, int], ...]    # [begin, end) of new ids per tier, hot first
    formats: Tuple[Tuple[str, str], ...]   # (gate/up, down) per tier
    bytes: int                             # expert weight bytes of the bank

    @property
    def new_id(self):
        """original expert id -> new id."""
        inv = np.empty_like(self.order)
        inv[self.order] = np.arange(self.order.size, dtype=self.order.dtype)
        return inv

    def tiers(self):
        """The non-empty tiers as ``Tier(e_begin, e_end, fmt_gate_up, fmt_down)``."""
        return tuple(C.Tier(b, e, fg, fd) for (b, e), (fg, fd) in zip(self.bounds, self.formats)
                     if e > b)


def routing_counts(ids, E):
    """Importance scores from a calibration pass: how often each expert was
    routed to (ids outside [0, E) are ignored)."""
    ids = np.asarray(ids).reshape(-1)
    ids = ids[(ids >= 0) & (ids < E)]
    return np.bincount(ids, minlength=E).astype(np.float64)


def plan_tiers(importance: Sequence[float], H: int, F: int,
               formats=DEFAULT_FORMATS, budget_bytes: Optional[int] = None) -> TierPlan:
    imp = np.asarray(importance, dtype=np.float64).reshape(-1)
    E = imp.size
    if E == 0:
        raise ValueError("empty expert bank")
    if len(formats) != 3:
        raise ValueError("need three (gate/up, down) tier formats")
    if not np.isfinite(imp).all():
        raise ValueError("importance scores must be finite")
    order = np.lexsort((np.arange(E), -imp)).astype(np.int64)
    cost = [expert_bytes(H, F, fg, fd) for fg, fd in formats]
    if not cost[0] >= cost[1] >= cost[2]:
        raise ValueError(f"tier formats must go from most to fewest bytes per expert: {cost}")

    def size(h, t):
        return h * cost[0] + (E - h - t) * cost[1] + t * cost[2]

    tail = int(np.floor(FRACTIONS[2] * E))
    if budget_bytes is None:
        hot = min(int(np.floor(FRACTIONS[0] * E + 0.5)), E - tail)
    else:
        budget = int(budget_bytes)
        if budget < E * cost[2]:
            raise ValueError(f"budget {budget} B is below the all-tail size {E * cost[2]} B")
        if size(0, tail) <= budget:
            extra = cost[0] - cost[1]
            hot = E - tail if extra == 0 else min(E - tail, (budget - size(0, tail)) // extra)
        else:
            hot = 0
            extra = cost[1] - cost[2]          # > 0: size(0, tail) > budget >= size(0, E)
            tail = min(E, tail + -(-(size(0, tail) - budget) // extra))
    hot, tail = int(hot), int(tail)
    return TierPlan(order=order, bounds=((0, hot), (hot, E - tail), (E - tail, E)),
                    formats=tuple((fg, fd) for fg, fd in formats), bytes=int(size(hot, tail)))


def permute_router(plan: TierPlan, Wr, bias=None):
    """Router rows [E, H] and the per-expert logit bias [E] in new-id order
    (works for NumPy arrays and torch tensors)."""
    idx = plan.order
    if not isinstance(Wr, np.ndarray):
        import torch
        idx = torch.as_tensor(idx, device=Wr.device)
    return Wr[idx], (None if bias is None else bias[idx])


def pack_bank(plan: TierPlan, H, F, expert_fp32, device="cuda"):
    """Quantize every expert into its tier with the device quantizer.

    ``expert_fp32(original_id)`` returns the expert's float32 CUDA tensors
    (gate [F, H], up [F, H], down [H, F]).  Returns a list of (e_begin, e_end,
    fmt_gate_up, fmt_down, gate, up, down), one per non-empty tier, each
    matrix bank a uint8 buffer holding its experts back to back in new-id
    order: the argument ``qmoe.tiers_struct`` takes."""
    torch = qmoe._torch()
    out = []
    for t in plan.tiers():
        n = t.e_end - t.e_begin
        sg = qmoe.tensor_bytes(t.fmt_gate_up, F, H)
        sd = qmoe.tensor_bytes(t.fmt_down, H, F)
        # zeroed: the quantizer leaves the alignment padding between planes alone
        g = torch.zeros(n * sg, dtype=torch.uint8, device=device)
        u = torch.zeros(n * sg, dtype=torch.uint8, device=device)
        d = torch.zeros(n * sd, dtype=torch.uint8, device=device)
        for i in range(n):
            wg, wu, wd = expert_fp32(int(plan.order[t.e_begin + i]))
            qmoe.quantize(t.fmt_gate_up, wg, out=g[i * sg:(i + 1) * sg])
            qmoe.quantize(t.fmt_gate_up, wu, out=u[i * sg:(i + 1) * sg])
            qmoe.quantize(t.fmt_down, wd, out=d[i * sd:(i + 1) * sd])
            del wg, wu, wd
        out.append((t.e_begin, t.e_end, t.fmt_gate_up, t.fmt_down, g, u, d))
    return out
