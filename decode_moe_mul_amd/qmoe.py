"""Thin Python binding of libqmoe.so (include/qmoe.h).

Argument marshalling only: every step runs in the HIP kernels of the library.
Tensors are torch tensors on the GPU (PyTorch supplies device memory and the
current stream); the functions allocate outputs and workspaces with torch and
pass raw pointers.  If the library is missing, the first call raises -- there
is no fallback path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqmoe.so")

FORMATS = {"q8_0": 0, "q4_0": 1, "mxfp4": 2, "q4_k": 3, "q6_k": 4, "t5": 5}
F32, BF16 = 0, 1
MAX_TIERS = 8

_lib = None


class QmoeError(RuntimeError):
    pass


MAX_BATCH = 16


class GemvDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("R", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class Tier(ctypes.Structure):
    _fields_ = [("e_begin", ctypes.c_int32), ("e_end", ctypes.c_int32),
                ("fmt_gate_up", ctypes.c_int32), ("fmt_down", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p)]


_VP, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = {
    "qmoe_abi_version": (_I, []),
    "qmoe_status_string": (ctypes.c_char_p, [_I]),
    "qmoe_last_error": (ctypes.c_char_p, []),
    "qmoe_block_size": (_I, [_I]),
    "qmoe_tensor_bytes": (_SZ, [_I, _I, _I]),
    "qmoe_plane_offsets": (_I, [_I, _I, _I, ctypes.POINTER(_SZ)]),
    "qmoe_device_cu_count": (_I, []),
    "moe_route_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_route": (_I, [_VP, _I, _I, _I, _VP, _VP, _I, _I, _I, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_permute": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP, _VP]),
    "moe_route_decode_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_route_decode": (_I, [_VP, _I, _I, _I, _VP, _VP, _I, _I, _I, _VP, _VP, _VP, _VP, _VP,
                              _VP, _VP, _SZ, _VP]),
    "moe_route_decode_noalloc_max_bytes": (_SZ, []),
    "moe_route_decode_noalloc": (_I, [_VP, _I, _I, _I, _VP, _VP, _I, _I, _I, _VP, _VP, _VP, _VP,
                                      _VP, _VP, _VP]),
    "moe_ffn_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_ffn_tiered": (_I, [ctypes.POINTER(Tier), _I, _I, _I, _I, _VP, _I, _I, _I, _VP, _VP,
                            _VP, _VP, _SZ, _VP]),
    "qgemm_grouped_prefill_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "qgemm_grouped_prefill": (_I, [ctypes.POINTER(Tier), _I, _I, _I, _I, _VP, _I, _I, _I, _VP,
                                   _VP, _VP, _VP, _SZ, _VP]),
    "qgemm_grouped_prefill_mx": (_I, [ctypes.POINTER(Tier), _I, _I, _I, _I, _VP, _I, _I, _I, _VP,
                                      _VP, _VP, _VP, _SZ, _VP]),
    "moe_combine": (_I, [_VP, _VP, _VP, _I, _I, _I, _VP, _VP, _VP]),
    "qquantize_act_mxfp8": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP]),
    "qquantize_act_q8": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP]),
    "qgemv_q8_0_i8": (_I, [_VP, _I, _I, _VP, _VP, _I, _VP, _VP]),
    "qgemm_mxfp4_mxfp8": (_I, [_VP, _I, _I, _VP, _VP, _I, _VP, _VP]),
    "qgemm_q8_0_i8": (_I, [_VP, _I, _I, _VP, _VP, _I, _VP, _VP]),
    "moe_layer_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_layer_decode": (_I, [ctypes.POINTER(Tier), _I, _I, _I, _I, _VP, _I, _I, _VP, _VP, _I,
                              _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "qmoe_stream_read": (_I, [_VP, _SZ, _I, _VP, _VP]),
    "qmoe_wave_latency": (_I, [_VP, _VP]),
    "qmoe_profile_enable": (_I, [_I]),
    "qmoe_profile_reset": (_I, []),
    "qmoe_profile_only": (_I, [ctypes.c_char_p]),
    "qmoe_profile_read": (_I, [ctypes.c_char_p, ctypes.POINTER(_I),
                               ctypes.POINTER(ctypes.c_double)]),
}
for _f in FORMATS:
    _SIGNATURES[f"qquantize_{_f}"] = (_I, [_VP, _I, _I, _VP, _VP])
    _SIGNATURES[f"qdequant_{_f}"] = (_I, [_VP, _I, _I, _VP, _VP])
    _SIGNATURES[f"qgemv_{_f}"] = (_I, [_VP, _I, _I, _VP, _I, _I, _VP, _VP])
_SIGNATURES["qgemv_batch"] = (_I, [_VP, _I, _VP])


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QmoeError(f"{LIB_PATH} is missing: build it with "
                            "`python -m decode_moe_mul_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        L = lib()
        raise QmoeError(f"{what}: {L.qmoe_status_string(status).decode()} "
                        f"({L.qmoe_last_error().decode()})")


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise QmoeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _need(cond, msg):
    if not cond:
        raise QmoeError(msg)


def _cuda_contig(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous CUDA tensors")


def _alloc_bytes(n, device):
    """uint8 device buffer of >= n bytes with a 256-byte aligned start."""
    torch = _torch()
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ meta --

def abi_version():
    return lib().qmoe_abi_version()


def tensor_bytes(fmt, N, K):
    n = lib().qmoe_tensor_bytes(FORMATS[fmt], N, K)
    _need(n > 0 or N == 0, f"{fmt}: K={K} is not a multiple of the block")
    return n


def plane_offsets(fmt, N, K):
    offs = (ctypes.c_size_t * 4)()
    n = lib().qmoe_plane_offsets(FORMATS[fmt], N, K, offs)
    _check(0 if n > 0 else n, "qmoe_plane_offsets")
    return list(offs[:n])


def cu_count():
    return lib().qmoe_device_cu_count()


# --------------------------------------------------------------- formats --

def quantize(fmt, w, out=None):
    """fp32 [N, K] CUDA tensor -> packed uint8 tensor (plane layout)."""
    torch = _torch()
    _need(w.dtype == torch.float32 and w.dim() == 2, "w must be a float32 [N, K] tensor")
    _cuda_contig(w)
    N, K = w.shape
    if out is None:
        out = torch.zeros(tensor_bytes(fmt, N, K), dtype=torch.uint8, device=w.device)
    _check(getattr(lib(), f"qquantize_{fmt}")(_p(w), N, K, _p(out), _stream()), f"qquantize_{fmt}")
    return out


def dequantize(fmt, W, N, K, out=None):
    torch = _torch()
    _cuda_contig(W)
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    _check(getattr(lib(), f"qdequant_{fmt}")(_p(W), N, K, _p(out), _stream()), f"qdequant_{fmt}")
    return out


def gemv_batch(items):
    """One launch for several independent GEMVs.  items: (fmt, W, N, K, x, out)
    tuples as gemv takes them (out required, [R, N] fp32); returns the outs."""
    torch = _torch()
    if len(items) > MAX_BATCH:
        raise ValueError(f"at most {MAX_BATCH} matrices per batch")
    descs = (GemvDesc * max(len(items), 1))()
    keep = []
    for i, (fmt, W, N, K, x, out) in enumerate(items):
        x2 = x if x.dim() == 2 else x.reshape(1, -1)
        _cuda_contig(W, x2, out)
        _need(x2.shape[1] == K, "x has the wrong length")
        _need(tuple(out.shape) == (x2.shape[0], N) and out.dtype == torch.float32,
              "out must be fp32 [R, N]")
        keep.append(x2)
        descs[i] = GemvDesc(FORMATS[fmt], N, K, _dtype_code(x2), x2.shape[0], 0,
                            _p(W), _p(x2), _p(out))
    _check(lib().qgemv_batch(descs, len(items), _stream()), "qgemv_batch")
    return [it[5] for it in items]


def gemv(fmt, W, N, K, x, out=None):
    """y [R, N] = x [R, K] . deq(W)^T."""
    torch = _torch()
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    _cuda_contig(W, x2)
    _need(x2.shape[1] == K, "x has the wrong length")
    R = x2.shape[0]
    if out is None:
        out = torch.empty((R, N), dtype=torch.float32, device=x.device)
    _check(getattr(lib(), f"qgemv_{fmt}")(_p(W), N, K, _p(x2), _dtype_code(x2), R, _p(out),
                                          _stream()), f"qgemv_{fmt}")
    return out


# --------------------------------------------------------------- routing --

def route_workspace(T, H, E, device="cuda"):
    return _alloc_bytes(lib().moe_route_workspace_size(T, H, E), device)


def route(x, Wr, bias, k, n_shared=0, logits=False, ws=None):
    """ids [T, k+n_shared] int32, p [T, k+n_shared] fp32 (and logits [T, E])."""
    torch = _torch()
    _cuda_contig(x, Wr, bias)
    T, H = x.shape
    E = Wr.shape[0]
    kt = k + n_shared
    ids = torch.empty((T, kt), dtype=torch.int32, device=x.device)
    p = torch.empty((T, kt), dtype=torch.float32, device=x.device)
    lg = torch.empty((T, E), dtype=torch.float32, device=x.device) if logits else None
    if ws is None:
        ws = route_workspace(T, H, E, x.device)
    _check(lib().moe_route(_p(x), _dtype_code(x), T, H, _p(Wr), _p(bias), E, k, n_shared,
                           _p(ids), _p(p), _p(lg), _p(ws), ws.numel(), _stream()), "moe_route")
    return (ids, p, lg) if logits else (ids, p)


def route_decode_workspace(T, H, E, device="cuda"):
    """Workspace of moe_route_decode: zero-filled, as its counters require."""
    torch = _torch()
    n = lib().moe_route_decode_workspace_size(T, H, E)
    return torch.zeros(max(int(n), 1), dtype=torch.uint8, device=device)


def route_decode(x, Wr, bias, k, n_shared=0, logits=False, ws=None):
    """moe_route + moe_permute in one launch (T <= 16):
    ids, p, offsets, perm, inv_perm (and logits [T, E])."""
    torch = _torch()
    _cuda_contig(x, Wr, bias)
    T, H = x.shape
    E = Wr.shape[0]
    kt = k + n_shared
    dev = x.device
    ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
    p = torch.empty((T, kt), dtype=torch.float32, device=dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None
    offsets = torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev)
    if ws is None:
        ws = route_decode_workspace(T, H, E, dev)
    _check(lib().moe_route_decode(_p(x), _dtype_code(x), T, H, _p(Wr), _p(bias), E, k, n_shared,
                                  _p(ids), _p(p), _p(lg), _p(offsets), _p(perm), _p(inv),
                                  _p(ws), ws.numel(), _stream()), "moe_route_decode")
    out = (ids, p, offsets, perm, inv)
    return out + (lg,) if logits else out


def route_decode_noalloc(x, Wr, bias, k, n_shared=0, logits=False, out=None):
    """moe_route_decode_noalloc: as route_decode, with the library's own
    device scratch instead of a workspace (the call allocates nothing; the
    output tensors are allocated here unless `out` = (ids, p, offsets, perm,
    inv_perm[, logits]) is given)."""
    torch = _torch()
    _cuda_contig(x, Wr, bias)
    T, H = x.shape
    E = Wr.shape[0]
    kt = k + n_shared
    dev = x.device
    if out is None:
        out = (torch.empty((T, kt), dtype=torch.int32, device=dev),
               torch.empty((T, kt), dtype=torch.float32, device=dev),
               torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev),
               torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev),
               torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev))
        if logits:
            out = out + (torch.empty((T, E), dtype=torch.float32, device=dev),)
    ids, p, offsets, perm, inv = out[:5]
    lg = out[5] if len(out) > 5 else None
    _check(lib().moe_route_decode_noalloc(_p(x), _dtype_code(x), T, H, _p(Wr), _p(bias), E, k,
                                          n_shared, _p(ids), _p(p), _p(lg), _p(offsets),
                                          _p(perm), _p(inv), _stream()),
           "moe_route_decode_noalloc")
    return out


def permute(ids, E, out=None):
    """offsets [E+1], perm [A], inv_perm [A] (int32) of ids [T, k]."""
    torch = _torch()
    _cuda_contig(ids)
    _need(ids.dtype == torch.int32, "ids must be int32")
    T, k = ids.shape if ids.dim() == 2 else (ids.numel(), 1)
    A = T * k
    if out is None:
        out = (torch.empty(E + 1, dtype=torch.int32, device=ids.device),
               torch.empty(max(A, 1), dtype=torch.int32, device=ids.device),
               torch.empty(max(A, 1), dtype=torch.int32, device=ids.device))
    offsets, perm, inv = out
    _check(lib().moe_permute(_p(ids), T, k, E, _p(offsets), _p(perm), _p(inv), _stream()),
           "moe_permute")
    return offsets, perm[:A], inv[:A]


# ------------------------------------------------------------ expert FFN --

def tiers_struct(tiers):
    """tiers: iterable of (e_begin, e_end, fmt_gate_up, fmt_down, gate, up,
    down) with packed uint8 CUDA tensors -> ctypes array (keep tensors alive)."""
    tiers = list(tiers)
    arr = (Tier * len(tiers))()
    for i, (b, e, fgu, fd, g, u, d) in enumerate(tiers):
        _cuda_contig(g, u, d)
        arr[i] = Tier(b, e, FORMATS[fgu], FORMATS[fd], g.data_ptr(), u.data_ptr(), d.data_ptr())
    return arr


def ffn_workspace(T, k, F, device="cuda"):
    return _alloc_bytes(lib().moe_ffn_workspace_size(T, k, F), device)


def prefill_workspace(T, k, E, H, F, device="cuda"):
    return _alloc_bytes(lib().qgemm_grouped_prefill_workspace_size(T, k, E, H, F), device)


def _ffn_call(name, tiers, E, H, F, x, k, offsets, perm, out, ws):
    torch = _torch()
    _cuda_contig(x, offsets, perm)
    T = x.shape[0]
    arr = tiers if isinstance(tiers, ctypes.Array) else tiers_struct(tiers)
    if out is None:
        out = torch.empty((max(T * k, 1), H), dtype=torch.float32, device=x.device)
    fn = getattr(lib(), name)
    _check(fn(arr, len(arr), E, H, F, _p(x), _dtype_code(x), T, k, _p(offsets), _p(perm),
              _p(out), _p(ws), 0 if ws is None else ws.numel(), _stream()), name)
    return out


def ffn_tiered(tiers, E, H, F, x, k, offsets, perm, out=None, ws=None):
    """o [T*k, H] in permuted order (decode kernels)."""
    if ws is None:
        ws = ffn_workspace(x.shape[0], k, F, x.device)
    return _ffn_call("moe_ffn_tiered", tiers, E, H, F, x, k, offsets, perm, out, ws)


def grouped_prefill(tiers, E, H, F, x, k, offsets, perm, out=None, ws=None):
    """o [T*k, H] in permuted order (matrix-core grouped GEMM)."""
    if ws is None:
        ws = prefill_workspace(x.shape[0], k, E, H, F, x.device)
    return _ffn_call("qgemm_grouped_prefill", tiers, E, H, F, x, k, offsets, perm, out, ws)


def grouped_prefill_mx(tiers, E, H, F, x, k, offsets, perm, out=None, ws=None):
    """As grouped_prefill, with MXFP4/MXFP4 tiers on the block-scaled matrix
    cores against MXFP8 activations."""
    if ws is None:
        ws = prefill_workspace(x.shape[0], k, E, H, F, x.device)
    return _ffn_call("qgemm_grouped_prefill_mx", tiers, E, H, F, x, k, offsets, perm, out, ws)


def combine(o, inv_perm, p, T, k, H, shared=None, out=None):
    torch = _torch()
    _cuda_contig(o, inv_perm, p, shared)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=o.device)
    _check(lib().moe_combine(_p(o), _p(inv_perm), _p(p), T, k, H, _p(shared), _p(out),
                             _stream()), "moe_combine")
    return out


def quantize_act_mxfp8(x):
    """Activations [R, K] (float32 or bfloat16) -> MXFP8 codes [R, K] uint8
    (E4M3) and scales [R, K/32] uint8 (E8M0)."""
    torch = _torch()
    _cuda_contig(x)
    R, K = x.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, max(K // 32, 1)), dtype=torch.uint8, device=x.device)
    _check(lib().qquantize_act_mxfp8(_p(x), _dtype_code(x), R, K, _p(codes), _p(scales),
                                     _stream()), "qquantize_act_mxfp8")
    return codes, scales


def quantize_act_q8(x):
    """Activations [R, K] (float32 or bfloat16) -> int8 codes [R, K] and fp32
    block scales [R, K/32]."""
    torch = _torch()
    _cuda_contig(x)
    R, K = x.shape
    q = torch.empty((R, K), dtype=torch.int8, device=x.device)
    d = torch.empty((R, max(K // 32, 1)), dtype=torch.float32, device=x.device)
    _check(lib().qquantize_act_q8(_p(x), _dtype_code(x), R, K, _p(q), _p(d), _stream()),
           "qquantize_act_q8")
    return q, d


def gemv_q8_0_i8(W, N, K, q, d, out=None):
    """y [R, N] = Q8_0 W [N, K] times the int8 activations (q, d)."""
    torch = _torch()
    _cuda_contig(W, q, d)
    R = q.shape[0]
    if out is None:
        out = torch.empty((R, N), dtype=torch.float32, device=q.device)
    _check(lib().qgemv_q8_0_i8(_p(W), N, K, _p(q), _p(d), R, _p(out), _stream()),
           "qgemv_q8_0_i8")
    return out


def gemm_q8_0_i8(W, N, K, q, d, out=None):
    """y [R, N] = Q8_0 W [N, K] times the int8 activations (q, d) on the
    int8 matrix cores (prefill-sized R)."""
    torch = _torch()
    _cuda_contig(W, q, d)
    R = q.shape[0]
    if out is None:
        out = torch.empty((R, N), dtype=torch.float32, device=q.device)
    _check(lib().qgemm_q8_0_i8(_p(W), N, K, _p(q), _p(d), R, _p(out), _stream()),
           "qgemm_q8_0_i8")
    return out


def gemm_mxfp4_mxfp8(W, N, K, codes, scales, out=None):
    """y [R, N] = W (MXFP4 [N, K]) times the MXFP8 activations."""
    torch = _torch()
    _cuda_contig(W, codes, scales)
    R = codes.shape[0]
    if out is None:
        out = torch.empty((R, N), dtype=torch.float32, device=codes.device)
    _check(lib().qgemm_mxfp4_mxfp8(_p(W), N, K, _p(codes), _p(scales), R, _p(out), _stream()),
           "qgemm_mxfp4_mxfp8")
    return out


def layer_decode_workspace(T, H, E, F, k, n_shared=0, device="cuda"):
    """Workspace of moe_layer_decode: zero-filled, as its barrier counter requires."""
    torch = _torch()
    n = lib().moe_layer_decode_workspace_size(T, H, E, F, k, n_shared)
    return torch.zeros(max(int(n), 1), dtype=torch.uint8, device=device)


def layer_decode_error(ws):
    """The error word of a moe_layer_decode workspace (waits for the stream):
    nonzero once a grid-barrier wait of some call on it ran out, which makes
    that call's outputs invalid.  The word stays set until cleared."""
    torch = _torch()
    torch.cuda.current_stream().synchronize()
    return int(ws[:4].view(torch.int32).item())


def check_layer_decode(ws):
    """Raise QmoeError if the workspace's error word is set (clearing it, so
    that the workspace can be used again)."""
    if layer_decode_error(ws):
        ws[:4].zero_()
        raise QmoeError("moe_layer_decode: a grid-barrier wait ran out; the outputs of the "
                        "calls since the workspace was last checked are invalid")


def layer_decode(tiers, E, H, F, x, Wr, bias, k, n_shared=0, out=None, ws=None, check=True):
    """The whole routed-expert layer for decode rows (T <= 16) in one launch:
    y [T, H] and the routing ids, p, offsets, perm, inv_perm.  check: wait
    for the call and raise if its barrier error word is set (callers that
    queue many calls may pass False and call check_layer_decode(ws) once
    afterwards: the word is sticky)."""
    torch = _torch()
    _cuda_contig(x, Wr, bias)
    T = x.shape[0]
    dev = x.device
    kt, E_total = k + n_shared, E + n_shared
    arr = tiers if isinstance(tiers, ctypes.Array) else tiers_struct(tiers)
    ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
    p = torch.empty((T, kt), dtype=torch.float32, device=dev)
    offsets = torch.empty(E_total + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * kt, 1), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = layer_decode_workspace(T, H, E, F, k, n_shared, dev)
    _check(lib().moe_layer_decode(arr, len(arr), E, H, F, _p(x), _dtype_code(x), T, _p(Wr),
                                  _p(bias), k, n_shared, _p(ids), _p(p), _p(offsets), _p(perm),
                                  _p(inv), _p(out), _p(ws), ws.numel(), _stream()),
           "moe_layer_decode")
    if check:
        check_layer_decode(ws)
    return out, ids, p, offsets, perm, inv


# ------------------------------------------------------------ measurement --

def wave_latency():
    """qmoe_wave_latency: one wave's dependent-step latencies (shader cycles)
    and the routing top-k's cost, as a dict."""
    torch = _torch()
    out = torch.zeros(8, dtype=torch.int64, device="cuda")
    _check(lib().qmoe_wave_latency(_p(out), _stream()), "qmoe_wave_latency")
    v = out.cpu().tolist()
    return {"valu_dependent_cycles": v[0], "dpp_wave_max_cycles": v[1],
            "ballot_round_trip_cycles": v[2], "wave_topk_512_k10_cycles": v[3],
            "lane_sort_8_cycles": v[4], "shader_clock_mhz": v[5]}


def stream_read(buf, blocks_per_cu=8, sink=None):
    """One streaming read of the CUDA tensor buf (qmoe_stream_read)."""
    torch = _torch()
    _cuda_contig(buf)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().qmoe_stream_read(_p(buf), nbytes, blocks_per_cu, _p(sink), _stream()),
           "qmoe_stream_read")
    return sink


# -------------------------------------------------------------- profiling --

def profile_enable(on=True):
    _check(lib().qmoe_profile_enable(1 if on else 0), "qmoe_profile_enable")


def profile_only(name=None):
    """Record only launches of kernel `name` (None: all)."""
    _check(lib().qmoe_profile_only(None if name is None else name.encode()), "qmoe_profile_only")


def profile_reset():
    _check(lib().qmoe_profile_reset(), "qmoe_profile_reset")


def profile_read(name):
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(lib().qmoe_profile_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)),
           "qmoe_profile_read")
    return n.value, ms.value
