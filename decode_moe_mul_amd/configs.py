"""The workloads: layer shapes, precision tiers and routing priors.

Sources on the pages:
  * tiered 512-expert, top-10 layer with FFN width 640 and three precision
    tiers by expert rank -- "Three RTX 3090 Qwen3.8-Flash-Next guide" page,
    sections "瓶颈分析" and "优化策略二"; 6 rows for an MTP verify of 5
    candidates -- same page, "瓶颈分析" item 3;
  * grouped 16-session decode over Q4_K routed experts with a Q8 shared
    expert -- "DwarfStar on 8x L40S" page, sections "120 t/s 的秘密微批次分组解码"
    and "快速上手";
  * 2048-token prefill chunks -- same page, same section;
  * dense single-token GEMV at Llama-3.1-8B layer shapes -- "RTX 3090 Llama 70B
    three-tier cache" page, section 一 (results table) and 4.4.

Readings (the pages leave these open):
  * tier sizes: hot = 25 % of 512 = 128, tail = floor(20 % of 512) = 102,
    middle = the remaining 282; ids [0,128), [128,410), [410,512);
  * the Zipf(s=1.1) rank prior is an additive logit bias b_e = -lam*ln(e+1)
    with lam calibrated to 0.5, so every tier is actually exercised (with
    lam = 1.1 literally, the tail tier receives no token at all);
  * weights and router are N(0, 0.02) everywhere; activations N(0, 1);
  * the shared expert is expert id E (one past the routed ids), always
    selected with weight 1.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Tier:
    e_begin: int
    e_end: int
    fmt_gate_up: str
    fmt_down: str


@dataclass(frozen=True)
class MoEConfig:
    name: str
    H: int
    E: int              # routed experts
    k: int              # routed experts per token
    F: int
    tiers: Tuple[Tier, ...]
    rows: Tuple[int, ...]
    x_dtype: str = "f32"            # "f32" or "bf16"
    prior_lambda: Optional[float] = None
    n_shared: int = 0
    shared_fmt: str = "q8_0"
    sigma_w: float = 0.02
    sigma_router: float = 0.02
    seed: int = 0

    @property
    def E_total(self):
        return self.E + self.n_shared

    def all_tiers(self):
        t = list(self.tiers)
        if self.n_shared:
            t.append(Tier(self.E, self.E + self.n_shared, self.shared_fmt, self.shared_fmt))
        return tuple(t)

    def tier_of(self, e):
        for t in self.all_tiers():
            if t.e_begin <= e < t.e_end:
                return t
        raise ValueError(e)


@dataclass(frozen=True)
class DenseConfig:
    name: str
    mats: Tuple[Tuple[str, int, int, str], ...]   # (name, N, K, fmt)
    rows: int = 1
    sigma_w: float = 0.02
    seed: int = 0


TINY = MoEConfig("tiny_q8_0", H=512, E=16, k=2, F=256,
                 tiers=(Tier(0, 16, "q8_0", "q8_0"),), rows=(4,))

LLAMA8B_GEMV = DenseConfig("llama3_8b_layer_gemv", mats=(
    ("q", 4096, 4096, "q4_k"), ("k", 1024, 4096, "q4_k"),
    ("v", 1024, 4096, "q4_k"), ("o", 4096, 4096, "q4_k"),
    ("gate", 14336, 4096, "q4_k"), ("up", 14336, 4096, "q4_k"),
    ("down", 4096, 14336, "q6_k")))

# the same layer's matrices in the ternary T5 format (1.75 bits per weight,
# "RTX 4080 SUPER native Windows 27B: NInfer 80 SM port" page, section 九.2)
LLAMA8B_GEMV_T5 = DenseConfig("llama3_8b_layer_gemv_t5", mats=tuple(
    (name, N, K, "t5") for (name, N, K, _) in LLAMA8B_GEMV.mats))

TIERED_TIERS = (Tier(0, 128, "q6_k", "q8_0"),
                Tier(128, 410, "q4_k", "q4_0"),
                Tier(410, 512, "mxfp4", "mxfp4"))

TIERED = MoEConfig("tiered_e512_top10", H=2048, E=512, k=10, F=640,
                   tiers=TIERED_TIERS, rows=(1, 6), prior_lambda=0.5)

GROUPED = MoEConfig("grouped16_e256_top8", H=7168, E=256, k=8, F=2048,
                    tiers=(Tier(0, 256, "q4_k", "q4_k"),), rows=(16,),
                    x_dtype="bf16", n_shared=1, shared_fmt="q8_0")

PREFILL = MoEConfig("prefill2048_tiered_e512_top10", H=2048, E=512, k=10,
                    F=640, tiers=TIERED_TIERS, rows=(2048,), prior_lambda=0.5)

ALL = {c.name: c for c in (TINY, TIERED, GROUPED, PREFILL)}
