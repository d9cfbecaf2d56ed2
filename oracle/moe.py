"""Oracle for the routed-expert layer and the dense quantized GEMV (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the path computes, step by step, as the pages state it:
  * router: a light linear layer scores every expert for each token and the
    top-k experts are kept ("Three RTX 3090 Qwen3.8-Flash-Next guide" page,
    section "瓶颈分析": 512 experts per layer, 10 picked per token);
  * the experts of a layer are re-indexed by selection frequency so that a
    precision tier is a contiguous id range, and the routed matmul only
    computes ids inside a tier's [min, max) range, skipping the rest
    explicitly (same page, sections "优化策略一", "优化策略三");
  * ids outside the valid range -- in particular a -1 "skip" sentinel -- must
    never be dereferenced (same page, "关键 Bug 修复与调试踩坑记录", items 1
    and 3);
  * each expert is a SwiGLU FFN: gate and up projections, SiLU(gate) * up,
    then the down projection (same page, bug item 4; "RTX 3090 Llama 70B
    three-tier cache" page, section 4.4);
  * the dense single-token quantized GEMV y = W x ("RTX 3090 Llama 70B
    three-tier cache" page, section 4.4, GEMV operator);
  * a grouped decode serves many session rows in one pass ("DwarfStar on 8x
    L40S" page, section "120 t/s 的秘密微批次分组解码").

Readings where the pages are silent (each listed in the design notes):
  * top-k keeps the k largest logits, ties to the lower expert id; slots are
    ordered by descending logit (ties lower id first); NaN logits rank below
    every number;
  * routing weights are the softmax over all experts renormalised over the
    kept k, i.e. the softmax over the kept logits;
  * an additive per-expert logit bias (the rank prior) enters both selection
    and weights;
  * always-on shared experts are appended after the k routed slots with ids
    E, E+1, ... and weight exactly 1;
  * the expert permutation is a stable counting sort of the flat assignment
    index a = t*k + i by expert id; invalid ids are left out of it.
"""
import numpy as np

from . import formats as fm


# ----------------------------------------------------------------- GEMV ----

def gemv(fmt, buf, N, K, x):
    """y[r, n] = sum_k deq(W)[n, k] * x[r, k]  and the bound
    B[r, n] = sum_k |deq(W)[n, k] * x[r, k]|, both float64."""
    W = fm.dequantize(fmt, buf, N, K)
    xd = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return xd @ W.T, np.abs(xd) @ np.abs(W).T


# --------------------------------------------------------------- routing ---

def router_logits(x, Wr, bias=None):
    """logits[t, e] = sum_h x[t, h] * Wr[e, h] + b[e] in float64."""
    logits = np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def topk(logits, k):
    """Ids of the k largest logits per row, ties to the lower id, slots in
    descending-logit order.  NaN ranks below every number."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    key = np.where(np.isnan(logits), -np.inf, logits)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # primary key: larger logit first; secondary: smaller id first
        order = np.lexsort((np.arange(E), -key[t]))
        ids[t] = order[:k]
    return ids


def softmax_over(logits, ids):
    """p[t, i] = exp(l[t, ids[t,i]]) / sum_j exp(l[t, ids[t,j]])."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), ids, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    return w / w.sum(axis=1, keepdims=True)


def route(x, Wr, bias, k, n_shared=0):
    """Router GEMV, top-k, renormalised softmax; shared experts appended.
    Returns ids [T, k+n_shared] int32, p [T, k+n_shared] float64,
    logits [T, E] float64."""
    logits = router_logits(x, Wr, bias)
    T, E = logits.shape
    ids = topk(logits, k)
    p = softmax_over(logits, ids)
    if n_shared:
        sh = np.tile(np.arange(E, E + n_shared, dtype=np.int32), (T, 1))
        ids = np.concatenate([ids, sh], axis=1)
        p = np.concatenate([p, np.ones((T, n_shared))], axis=1)
    return ids, p, logits


def topk_gap(logits, k):
    """Per token: logit of rank k minus logit of rank k+1 (float64), the
    margin by which the selection is decided; inf when k == E."""
    srt = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    if k >= srt.shape[1]:
        return np.full(srt.shape[0], np.inf)
    return srt[:, k - 1] - srt[:, k]


# ----------------------------------------------------------- permutation ---

def permute(ids, E):
    """Stable counting sort of flat assignments a = t*k + i by expert id.
    offsets[e] = number of valid assignments with id < e (offsets[E] = total
    valid); perm[pos] = a for pos < offsets[E], else -1; inv_perm[a] = pos,
    or -1 when ids.flat[a] is not in [0, E)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    A = flat.size
    valid = (flat >= 0) & (flat < E)
    counts = np.zeros(E, dtype=np.int64)
    for a in range(A):
        if valid[a]:
            counts[flat[a]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    perm = np.full(A, -1, dtype=np.int64)
    inv = np.full(A, -1, dtype=np.int64)
    for a in range(A):                       # ascending a => stable
        if valid[a]:
            e = flat[a]
            perm[cursor[e]] = a
            inv[a] = cursor[e]
            cursor[e] += 1
    return offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


# ---------------------------------------------------------------- experts --

def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_ffn(expert, H, F, X):
    """One expert on rows X [m, H].  ``expert`` is a tuple
    (fmt_gate_up, gate_bytes, up_bytes, fmt_down, down_bytes) with gate/up
    [F, H] and down [H, F].  Returns o [m, H], bound_o [m, H], h [m, F],
    g, u [m, F] and their bounds."""
    fgu, gbuf, ubuf, fd, dbuf = expert
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    g, bg = gemv(fgu, gbuf, F, H, X)
    u, bu = gemv(fgu, ubuf, F, H, X)
    h = silu(g) * u
    o, bo = gemv(fd, dbuf, H, F, h)
    return {"o": o, "bound_o": bo, "h": h, "g": g, "u": u,
            "bound_g": bg, "bound_u": bu}


def ffn_permuted(x, ids, offsets, perm, get_expert, H, F, k):
    """What the routed FFN writes: o[pos] for every valid position pos of the
    permutation (o[pos] = expert(ids.flat[a])(x[a // k]) with a = perm[pos]),
    with its bound.  Rows pos >= offsets[E] are NaN (never written)."""
    x = np.asarray(x, dtype=np.float64)
    flat = np.asarray(ids).reshape(-1)
    A = flat.size
    o = np.full((A, H), np.nan)
    bo = np.full((A, H), np.nan)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        pos = np.arange(lo, hi)
        rows = np.asarray(perm)[pos] // k
        r = expert_ffn(get_expert(e), H, F, x[rows])
        o[pos] = r["o"]
        bo[pos] = r["bound_o"]
    return o, bo


def combine(o, inv_perm, p, T, k, shared=None):
    """y[t] = sum_{i<k} p[t,i] * o[inv_perm[t*k+i]] (slots with inv_perm < 0
    skipped) + shared[t]; and its bound sum |p*o| + |shared|."""
    o = np.asarray(o, dtype=np.float64)
    H = o.shape[1]
    p = np.asarray(p, dtype=np.float64).reshape(T, k)
    inv = np.asarray(inv_perm).reshape(T, k)
    y = np.zeros((T, H))
    b = np.zeros((T, H))
    for t in range(T):
        for i in range(k):
            if inv[t, i] >= 0:
                y[t] += p[t, i] * o[inv[t, i]]
                b[t] += np.abs(p[t, i] * o[inv[t, i]])
    if shared is not None:
        s = np.asarray(shared, dtype=np.float64)
        y += s
        b += np.abs(s)
    return y, b


def moe_layer(x, ids, p, get_expert, H, F, E):
    """The routed-expert layer given routing decisions:
    y[t] = sum_i p[t,i] * FFN_{ids[t,i]}(x[t]) over valid ids, with the
    parity bound B_y[t, n] = sum_i p[t,i] * sum_j |Wd[n,j] * h_{t,i}[j]|.
    Each expert is evaluated once on all the rows routed to it."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    p = np.asarray(p, dtype=np.float64)
    T, k = ids.shape
    y = np.zeros((T, H))
    b = np.zeros((T, H))
    for e in np.unique(ids):
        if e < 0 or e >= E:
            continue
        ts, slots = np.nonzero(ids == e)
        r = expert_ffn(get_expert(int(e)), H, F, x[ts])
        for j, (t, i) in enumerate(zip(ts, slots)):
            y[t] += p[t, i] * r["o"][j]
            b[t] += p[t, i] * r["bound_o"][j]
    return y, b
