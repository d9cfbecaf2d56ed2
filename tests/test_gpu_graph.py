"""A decode layer call (moe_route_decode -> moe_ffn_tiered -> moe_combine)
captured in a HIP graph and replayed gives the eager call's outputs bit for
bit, replay after replay, with eager calls on other inputs in between (the
routing workspace's counter must be back at zero after every call, captured
or not).  A whole decode layer replayed as one graph per step is the pages'
decode loop (the "RTX 4080 SUPER native Windows 27B" page, section 九 item 5).
"""
import numpy as np
import pytest

from gpu_util import requires_gpu, to_np, assert_bitexact, torch
from decode_moe_mul_amd import configs, layers, synth
from decode_moe_mul_amd.configs import MoEConfig, Tier

pytestmark = [pytest.mark.gpu, requires_gpu]

SMALL_SHARED = MoEConfig("graph_small_shared", H=512, E=8, k=2, F=256,
                         tiers=(Tier(0, 8, "q4_k", "q4_k"),), rows=(16,), x_dtype="bf16",
                         n_shared=1, shared_fmt="q8_0")

_cache = {}


def _layer(cfg):
    if cfg.name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[cfg.name] = layers.MoELayer(cfg)
    return _cache[cfg.name]


def _x(cfg, T, seed):
    x = synth.normal((T, cfg.H), 1.0, seed, synth.ACT, T)
    xg = torch.from_numpy(x).cuda()
    return xg.to(torch.bfloat16) if cfg.x_dtype == "bf16" else xg


KEYS = ("y", "ids", "p", "offsets", "perm", "inv")


@pytest.mark.parametrize("cfg,T", [(configs.TIERED, 1), (configs.TIERED, 6),
                                   (SMALL_SHARED, 16), (configs.TINY, 4)],
                         ids=lambda v: getattr(v, "name", v))
def test_graph_replay_equals_eager(cfg, T):
    layer = _layer(cfg)
    x = _x(cfg, T, 21)
    x_other = _x(cfg, T, 22)
    _, ws = layer.forward(x)
    want = {k: to_np(ws[k]).copy() for k in KEYS}
    _, _ = layer.forward(x_other)
    other = {k: to_np(ws[k]).copy() for k in KEYS}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in KEYS:
            ws[k].fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        for k in KEYS:
            got = to_np(ws[k])
            if want[k].dtype == np.float32:
                assert_bitexact(got, want[k], f"{cfg.name} T={T} replay {rep} {k}")
            else:
                assert (got == want[k]).all(), f"{cfg.name} T={T} replay {rep} {k}"
        # an eager call on other rows between replays: still its own result
        layer.forward(x_other)
        torch.cuda.synchronize()
        assert_bitexact(to_np(ws["y"]), other["y"], f"{cfg.name} T={T} eager after replay {rep}")
    # the routing counter is back at zero (first 256 bytes of its workspace)
    if "route" in ws and layer._fused(T, False):
        assert (to_np(ws["route"][:256]) == 0).all()
