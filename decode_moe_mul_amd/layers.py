"""Synthetic quantized layers on the GPU and the layer call sequence.

``MoELayer`` holds a routed-expert layer (router, optional rank prior, expert
banks per precision tier, optional shared experts) built from seeded device
normals and packed by the library's own quantizer; ``forward`` runs
moe_route -> moe_permute -> moe_ffn_tiered (or qgemm_grouped_prefill) ->
moe_combine on the current stream with preallocated workspaces.

``DenseLayer`` holds the quantized matrices of one dense transformer layer and
runs qgemv on them.

Both can keep several copies of their weights at distinct addresses so that a
benchmark can rotate through more bytes than the GPU's caches hold.
"""
import numpy as np

from . import configs as C
from . import qmoe
from . import synth


def _torch():
    import torch
    return torch


class MoELayer:
    def __init__(self, cfg, seed=None, device="cuda", copies=1, order=None):
        """order: optional re-indexing of the routed experts (new id ->
        original id, as a tier plan makes): routed expert e of this layer is
        the synthetic expert order[e], with its router row and logit bias."""
        torch = _torch()
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self.device = device
        H, E, F = cfg.H, cfg.E, cfg.F
        self.order = np.arange(E) if order is None else np.asarray(order, dtype=np.int64)
        if sorted(self.order.tolist()) != list(range(E)):
            raise ValueError("order must be a permutation of the routed expert ids")
        idx = torch.as_tensor(self.order, device=device)
        self.Wr = synth.normal_device((E, H), cfg.sigma_router, self.seed, synth.ROUTER, 0,
                                      device)[idx].contiguous()
        self.bias = None
        if cfg.prior_lambda is not None:
            self.bias = torch.from_numpy(synth.rank_prior(E, cfg.prior_lambda)).to(device)[idx].contiguous()
        self.tiers = cfg.all_tiers()
        banks = []
        for t in self.tiers:
            n = t.e_end - t.e_begin
            sg = qmoe.tensor_bytes(t.fmt_gate_up, F, H)
            sd = qmoe.tensor_bytes(t.fmt_down, H, F)
            g = torch.zeros(n * sg, dtype=torch.uint8, device=device)
            u = torch.zeros(n * sg, dtype=torch.uint8, device=device)
            d = torch.zeros(n * sd, dtype=torch.uint8, device=device)
            for i in range(n):
                wg, wu, wd = self.expert_fp32_device(t.e_begin + i)
                qmoe.quantize(t.fmt_gate_up, wg, out=g[i * sg:(i + 1) * sg])
                qmoe.quantize(t.fmt_gate_up, wu, out=u[i * sg:(i + 1) * sg])
                qmoe.quantize(t.fmt_down, wd, out=d[i * sd:(i + 1) * sd])
                del wg, wu, wd
            banks.append((g, u, d))
        self.banks = [banks] + [[tuple(b.clone() for b in bk) for bk in banks]
                                for _ in range(copies - 1)]
        self.tier_arrays = [qmoe.tiers_struct(
            [(t.e_begin, t.e_end, t.fmt_gate_up, t.fmt_down, g, u, d)
             for t, (g, u, d) in zip(self.tiers, bk)]) for bk in self.banks]
        self._ws = {}

    # ----------------------------------------------------------- weights --
    def _keys(self, e):
        if e < self.cfg.E:
            return (synth.GATE, synth.UP, synth.DOWN), int(self.order[e])
        return (synth.SH_GATE, synth.SH_UP, synth.SH_DOWN), e - self.cfg.E

    def expert_fp32_device(self, e):
        c = self.cfg
        (kg, ku, kd), idx = self._keys(e)
        nd = lambda shape, tag: synth.normal_device(shape, c.sigma_w, self.seed, tag, idx, self.device)
        return nd((c.F, c.H), kg), nd((c.F, c.H), ku), nd((c.H, c.F), kd)

    def expert_fp32(self, e):
        """The fp32 weights of expert e on the host (gate, up, down)."""
        return tuple(w.cpu().numpy() for w in self.expert_fp32_device(e))

    def expert_bytes(self, e):
        t = self.cfg.tier_of(e)
        c = self.cfg
        return (2 * qmoe.tensor_bytes(t.fmt_gate_up, c.F, c.H)
                + qmoe.tensor_bytes(t.fmt_down, c.H, c.F))

    def weight_bytes(self, ids):
        """Algorithmic weight bytes one call streams: router + every distinct
        valid expert in ids (shared experts included)."""
        flat = np.unique(np.asarray(ids).reshape(-1))
        flat = flat[(flat >= 0) & (flat < self.cfg.E_total)]
        return self.cfg.E * self.cfg.H * 4 + sum(self.expert_bytes(int(e)) for e in flat)

    # -------------------------------------------------------------- call --
    def workspaces(self, T, prefill=False):
        key = (T, prefill)
        if key not in self._ws:
            c = self.cfg
            torch = _torch()
            kt = c.k + c.n_shared
            A = T * kt
            dev = self.device
            ws = {
                "route": (qmoe.route_decode_workspace(T, c.H, c.E, dev) if self._fused(T, prefill)
                          else qmoe.route_workspace(T, c.H, c.E, dev)),
                "ids": torch.empty((T, kt), dtype=torch.int32, device=dev),
                "p": torch.empty((T, kt), dtype=torch.float32, device=dev),
                "offsets": torch.empty(c.E_total + 1, dtype=torch.int32, device=dev),
                "perm": torch.empty(max(A, 1), dtype=torch.int32, device=dev),
                "inv": torch.empty(max(A, 1), dtype=torch.int32, device=dev),
                "o": torch.empty((max(A, 1), c.H), dtype=torch.float32, device=dev),
                "y": torch.empty((T, c.H), dtype=torch.float32, device=dev),
                "ffn": (qmoe.prefill_workspace(T, kt, c.E_total, c.H, c.F, dev) if prefill
                        else qmoe.ffn_workspace(T, kt, c.F, dev)),
            }
            if not prefill and T <= 16:
                ws["layer"] = qmoe.layer_decode_workspace(T, c.H, c.E, c.F, c.k, c.n_shared, dev)
            self._ws[key] = ws
        return self._ws[key]

    def check_one_launch(self, T):
        """Raise if a one-launch call with T rows reported a barrier time-out
        since the last check (the workspace's sticky error word)."""
        qmoe.check_layer_decode(self.workspaces(T)["layer"])

    def _fused(self, T, prefill):
        """Decode rows route and permute in one launch (moe_route_decode)."""
        c = self.cfg
        kt = c.k + c.n_shared
        return (not prefill and T <= 16 and c.E <= 512
                and ((T * kt + 63) // 64) * 64 + 16 + c.E_total <= 8192)

    def forward(self, x, copy=0, prefill=False, one_launch=False, mx=False, check=True):
        """y [T, H] for activations x [T, H] (float32 or bfloat16).  The
        intermediate ids, p, offsets, perm, inv (and o, unless one_launch)
        stay in the workspace dict returned second.  one_launch: the whole
        decode layer as moe_layer_decode (T <= 16); with check (the default)
        the call is waited for and its barrier error word read (a timing
        loop passes check=False and calls check_one_launch(T) afterwards).
        mx (with prefill): the MXFP4/MXFP4 tiers on the block-scaled matrix
        cores (qgemm_grouped_prefill_mx)."""
        c = self.cfg
        T = x.shape[0]
        ws = self.workspaces(T, prefill)
        L = qmoe.lib()
        s = qmoe._stream()
        kt = c.k + c.n_shared
        if one_launch:
            arr = self.tier_arrays[copy]
            qmoe._check(L.moe_layer_decode(
                arr, len(arr), c.E, c.H, c.F, qmoe._p(x), qmoe._dtype_code(x), T,
                qmoe._p(self.Wr), qmoe._p(self.bias), c.k, c.n_shared, qmoe._p(ws["ids"]),
                qmoe._p(ws["p"]), qmoe._p(ws["offsets"]), qmoe._p(ws["perm"]),
                qmoe._p(ws["inv"]), qmoe._p(ws["y"]), qmoe._p(ws["layer"]), ws["layer"].numel(),
                s), "moe_layer_decode")
            if check:
                qmoe.check_layer_decode(ws["layer"])
            return ws["y"], ws
        if self._fused(T, prefill):
            qmoe._check(L.moe_route_decode(
                qmoe._p(x), qmoe._dtype_code(x), T, c.H, qmoe._p(self.Wr), qmoe._p(self.bias),
                c.E, c.k, c.n_shared, qmoe._p(ws["ids"]), qmoe._p(ws["p"]), None,
                qmoe._p(ws["offsets"]), qmoe._p(ws["perm"]), qmoe._p(ws["inv"]),
                qmoe._p(ws["route"]), ws["route"].numel(), s), "moe_route_decode")
        else:
            qmoe._check(L.moe_route(qmoe._p(x), qmoe._dtype_code(x), T, c.H, qmoe._p(self.Wr),
                                    qmoe._p(self.bias), c.E, c.k, c.n_shared,
                                    qmoe._p(ws["ids"]), qmoe._p(ws["p"]), None,
                                    qmoe._p(ws["route"]), ws["route"].numel(), s), "moe_route")
            qmoe._check(L.moe_permute(qmoe._p(ws["ids"]), T, kt, c.E_total,
                                      qmoe._p(ws["offsets"]), qmoe._p(ws["perm"]),
                                      qmoe._p(ws["inv"]), s), "moe_permute")
        fn = ((L.qgemm_grouped_prefill_mx if mx else L.qgemm_grouped_prefill) if prefill
              else L.moe_ffn_tiered)
        arr = self.tier_arrays[copy]
        qmoe._check(fn(arr, len(arr), c.E_total, c.H, c.F, qmoe._p(x), qmoe._dtype_code(x), T, kt,
                       qmoe._p(ws["offsets"]), qmoe._p(ws["perm"]), qmoe._p(ws["o"]),
                       qmoe._p(ws["ffn"]), ws["ffn"].numel(), s), "expert ffn")
        qmoe._check(L.moe_combine(qmoe._p(ws["o"]), qmoe._p(ws["inv"]), qmoe._p(ws["p"]), T, kt,
                                  c.H, None, qmoe._p(ws["y"]), s), "moe_combine")
        return ws["y"], ws


class DenseLayer:
    """The quantized matrices of one dense layer (qgemv per matrix)."""

    def __init__(self, cfg, seed=None, device="cuda", copies=1):
        torch = _torch()
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self.device = device
        mats = []
        for i, (name, N, K, fmt) in enumerate(cfg.mats):
            w = synth.normal_device((N, K), cfg.sigma_w, self.seed, synth.DENSE, i, device)
            mats.append(qmoe.quantize(fmt, w))
            del w
        self.mats = [mats] + [[m.clone() for m in mats] for _ in range(copies - 1)]
        self.out = [torch.empty((cfg.rows, N), dtype=torch.float32, device=device)
                    for (_, N, _, _) in cfg.mats]

    def matrix_fp32(self, i, rows=None):
        _, N, K, _ = self.cfg.mats[i]
        w = synth.normal_device((N, K), self.cfg.sigma_w, self.seed, synth.DENSE, i, self.device)
        w = w if rows is None else w[rows]
        return w.cpu().numpy()

    def weight_bytes(self):
        return sum(qmoe.tensor_bytes(f, N, K) for (_, N, K, f) in self.cfg.mats)

    def forward(self, x, copy=0, batched=False):
        """Every matrix against its input (x, or x[name] per matrix): one
        qgemv launch per matrix, or all of them in one qgemv_batch launch
        (the inputs are independent here)."""
        items = []
        for i, (name, N, K, fmt) in enumerate(self.cfg.mats):
            xin = x[name] if isinstance(x, dict) else x
            items.append((fmt, self.mats[copy][i], N, K, xin, self.out[i]))
        if batched:
            return qmoe.gemv_batch(items)
        return [qmoe.gemv(f, W, N, K, xin, out=o) for (f, W, N, K, xin, o) in items]
