"""moe_route_decode_noalloc (the library's own device scratch instead of a
caller workspace) against moe_route_decode with a workspace, through the C
ABI: equal outputs bit for bit on two calls in a row, the second smaller, and
a size beyond the scratch rejected before any launch."""
import ctypes

import numpy as np
import pytest

from gpu_util import requires_gpu, to_np, torch
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(T, H, E, bf16, seed, prior):
    x = torch.from_numpy(synth.normal((T, H), 1.0, seed, synth.ACT, T)).cuda()
    if bf16:
        x = x.to(torch.bfloat16)
    Wr = torch.from_numpy(synth.normal((E, H), 0.02, seed, synth.ROUTER, 0)).cuda()
    b = torch.from_numpy(synth.rank_prior(E, 0.5)).cuda() if prior else None
    return x, Wr, b


def _call(noalloc, x, Wr, b, k, n_shared):
    L = qmoe.lib()
    T, H = x.shape
    E = Wr.shape[0]
    kt = k + n_shared
    dev = x.device
    ids = torch.full((T, kt), -5, dtype=torch.int32, device=dev)
    p = torch.full((T, kt), -5.0, dtype=torch.float32, device=dev)
    lg = torch.full((T, E), -5.0, dtype=torch.float32, device=dev)
    off = torch.full((E + n_shared + 1,), -5, dtype=torch.int32, device=dev)
    perm = torch.full((T * kt,), -5, dtype=torch.int32, device=dev)
    inv = torch.full((T * kt,), -5, dtype=torch.int32, device=dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dt = qmoe.BF16 if x.dtype == torch.bfloat16 else qmoe.F32
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = L.moe_route_decode_noalloc(P(x), dt, T, H, P(Wr), P(b), E, k, n_shared, P(ids),
                                        P(p), P(lg), P(off), P(perm), P(inv), s)
    else:
        ws = qmoe.route_decode_workspace(T, H, E, dev)
        st = L.moe_route_decode(P(x), dt, T, H, P(Wr), P(b), E, k, n_shared, P(ids), P(p),
                                P(lg), P(off), P(perm), P(inv), P(ws), ws.numel(), s)
    assert st == 0, L.qmoe_last_error().decode()
    return {n: to_np(t).copy() for n, t in
            (("ids", ids), ("p", p), ("logits", lg), ("offsets", off), ("perm", perm),
             ("inv", inv))}


def test_noalloc_route_decode_equals_workspace_call_twice():
    cases = [(16, 7168, 256, 8, 1, True, False),   # grouped 16-row layer shape, bf16
             (1, 2048, 512, 10, 0, False, True)]   # then a smaller call: tiered, 1 row
    for T, H, E, k, n_shared, bf16, prior in cases:
        x, Wr, b = _inputs(T, H, E, bf16, 3, prior)
        want = _call(False, x, Wr, b, k, n_shared)
        got = _call(True, x, Wr, b, k, n_shared)
        for name in want:
            a, r = got[name], want[name]
            if a.dtype == np.float32:
                assert np.array_equal(a.view(np.uint32), r.view(np.uint32)), (T, name)
            else:
                assert np.array_equal(a, r), (T, name)
        # repeat on the same scratch: the counter was left at zero
        again = _call(True, x, Wr, b, k, n_shared)
        assert all(np.array_equal(again[n], got[n]) for n in got)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    L = qmoe.lib()
    cap = L.moe_route_decode_noalloc_max_bytes()
    assert cap == 1 << 20
    T, H, E = 16, 65536, 512
    assert L.moe_route_decode_workspace_size(T, H, E) > cap
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    P = ctypes.c_void_p(dummy.data_ptr())
    st = L.moe_route_decode_noalloc(P, qmoe.F32, T, H, P, None, E, 4, 0, P, P, None, P, P, P,
                                    None)
    assert st == -2 and b"scratch" in L.qmoe_last_error()
