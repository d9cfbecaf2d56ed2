"""GPU parity of the routed-expert layer: moe_ffn_tiered, moe_combine,
qgemm_grouped_prefill and whole layers at every workload shape.

Routing follows the near-tie protocol of test_gpu_route.py: tokens whose fp64
top-k margin is within twice the fp32 logit error are excluded from the
element comparison (and counted); all other tokens must match the oracle
within 1e-3 * sum_i p_i * sum_j |Wd[n, j] h_j| per output element.
"""
import numpy as np
import pytest

from gpu_util import (requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound,
                      ExpertCache, torch)
from oracle import formats as fm
from oracle import moe
from decode_moe_mul_amd import configs, layers, qmoe, synth
from decode_moe_mul_amd.configs import MoEConfig, Tier

pytestmark = [pytest.mark.gpu, requires_gpu]

SMALL_TIERED = MoEConfig("small_tiered", H=256, E=12, k=3, F=64,
                         tiers=(Tier(0, 4, "q6_k", "q8_0"), Tier(4, 9, "q4_k", "q4_0"),
                                Tier(9, 12, "mxfp4", "mxfp4")), rows=(5,))
SMALL_SHARED = MoEConfig("small_shared", H=512, E=8, k=2, F=256,
                         tiers=(Tier(0, 8, "q4_k", "q4_k"),), rows=(16,), x_dtype="bf16",
                         n_shared=1, shared_fmt="q8_0")

_layers = {}


def _layer(cfg):
    if cfg.name not in _layers:
        _layers.clear()                       # keep one large layer resident at a time
        torch.cuda.empty_cache()
        _layers[cfg.name] = layers.MoELayer(cfg)
    return _layers[cfg.name]


def _x(cfg, T, seed=0):
    x = synth.normal((T, cfg.H), 1.0, seed, synth.ACT, T)
    if cfg.x_dtype == "bf16":
        x = synth.bf16_round(x)
        return x, to_gpu(x).to(torch.bfloat16)
    return x, to_gpu(x)


def _check_layer(cfg, T, rows_checked=None, seed=0, prefill=False, cols=None, one_launch=False):
    layer = _layer(cfg)
    x, xg = _x(cfg, T, seed)
    y, ws = layer.forward(xg, prefill=prefill, one_launch=one_launch)
    y = to_np(y)
    ids = to_np(ws["ids"])
    p = to_np(ws["p"])
    Wr = to_np(layer.Wr)
    b = None if layer.bias is None else to_np(layer.bias)
    ids_ref, p_ref, lg_ref = moe.route(x, Wr, b, cfg.k, cfg.n_shared)
    # near-tie protocol: tokens whose decision is within the logit error
    lg_bound = np.abs(x.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    gap = moe.topk_gap(lg_ref, cfg.k)
    decided = gap > 2 * 1e-5 * lg_bound.max(axis=1)
    same = (ids == ids_ref).all(axis=1)
    assert same[decided].all(), "routing differs on a token outside the near-tie margin"
    rows = np.arange(T) if rows_checked is None else np.asarray(rows_checked)
    rows = rows[same[rows]]
    assert rows.size > 0
    cache = ExpertCache(layer)
    if cols is None:
        y_ref, bound = moe.moe_layer(x[rows], ids_ref[rows], p_ref[rows], cache, cfg.H, cfg.F,
                                     cfg.E_total)
        assert_within_bound(y[rows], y_ref, bound, what=f"{cfg.name} T={T}")
    else:
        # sampled output columns: only those rows of each down matrix are needed
        for t in rows:
            yt, bt = np.zeros(len(cols)), np.zeros(len(cols))
            for i, e in enumerate(ids_ref[t]):
                tier = cfg.tier_of(int(e))
                wg, wu, wd = layer.expert_fp32(int(e))
                g, _ = moe.gemv(tier.fmt_gate_up, fm.quantize(tier.fmt_gate_up, wg), cfg.F, cfg.H, x[t:t + 1])
                u, _ = moe.gemv(tier.fmt_gate_up, fm.quantize(tier.fmt_gate_up, wu), cfg.F, cfg.H, x[t:t + 1])
                h = moe.silu(g) * u
                o, bo = moe.gemv(tier.fmt_down, fm.quantize(tier.fmt_down, wd[cols]), len(cols), cfg.F, h)
                yt += p_ref[t, i] * o[0]
                bt += p_ref[t, i] * bo[0]
            assert_within_bound(y[t, cols], yt, bt, what=f"{cfg.name} token {t}")
    return layer, y, ws


def test_tiny_q8_0_layer():
    _check_layer(configs.TINY, 4)


def test_small_tiered_layer_all_tiers_hit():
    layer, y, ws = _check_layer(SMALL_TIERED, 40)
    ids = to_np(ws["ids"])
    assert (ids < 4).any() and ((ids >= 4) & (ids < 9)).any() and (ids >= 9).any()


def test_small_shared_bf16_layer():
    _check_layer(SMALL_SHARED, 16)


WIDE_HIDDEN = MoEConfig("wide_hidden", H=28672, E=4, k=2, F=64,
                        tiers=(Tier(0, 2, "q6_k", "q8_0"), Tier(2, 4, "q4_k", "q4_0")),
                        rows=(3,))


@pytest.mark.parametrize("T", [1, 3])
def test_hidden_too_wide_for_lds_staging(T):
    """A 28672-wide hidden row does not fit the LDS staging of the dot-product
    path; the gate/up phase then runs every expert on the matrix cores."""
    _check_layer(WIDE_HIDDEN, T)


@pytest.mark.parametrize("T", [1, 6])
def test_tiered_layer_full_size(T):
    """512 experts, top-10, hidden 2048, FFN 640, three tiers, rank prior."""
    _check_layer(configs.TIERED, T)


def _check_all_tokens_sampled_cols(cfg, T, cols, seed=0, prefill=False, one_launch=False,
                                   x=None):
    """Every token of a full-size layer call against the oracle on the
    sampled output columns `cols` (all columns of h, so every gate/up row is
    checked through them).  The near-tie protocol of _check_layer applies;
    the oracle runs one distinct expert per job on a process pool."""
    import oracle_pool
    layer = _layer(cfg)
    if x is None:
        x, xg = _x(cfg, T, seed)
    else:
        xg = to_gpu(x).to(torch.bfloat16) if cfg.x_dtype == "bf16" else to_gpu(x)
    y, ws = layer.forward(xg, prefill=prefill, one_launch=one_launch)
    y = to_np(y)
    ids = to_np(ws["ids"])
    Wr = to_np(layer.Wr)
    b = None if layer.bias is None else to_np(layer.bias)
    ids_ref, p_ref, lg_ref = moe.route(x, Wr, b, cfg.k, cfg.n_shared)
    lg_bound = np.abs(x.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    decided = moe.topk_gap(lg_ref, cfg.k) > 2 * 1e-5 * lg_bound.max(axis=1)
    same = (ids == ids_ref).all(axis=1)
    assert same[decided].all(), "routing differs on a token outside the near-tie margin"
    rows = np.nonzero(same)[0]
    assert rows.size >= T - max(1, T // 100), f"only {rows.size} of {T} tokens routed alike"
    experts = np.unique(ids_ref[rows])

    def jobs():
        for e in experts:
            ts = rows[(ids_ref[rows] == e).any(axis=1)]
            t = cfg.tier_of(int(e))
            wg, wu, wd = layer.expert_fp32(int(e))
            yield (t.fmt_gate_up, wg, wu, t.fmt_down, np.ascontiguousarray(wd[cols]), x[ts])

    outs = oracle_pool.run(oracle_pool.expert_job, jobs())
    y_ref = np.zeros((T, len(cols)))
    bound = np.zeros((T, len(cols)))
    for e, (o, bo) in zip(experts, outs):
        ts = rows[(ids_ref[rows] == e).any(axis=1)]
        for j, t in enumerate(ts):
            for i in np.nonzero(ids_ref[t] == e)[0]:
                y_ref[t] += p_ref[t, i] * o[j]
                bound[t] += p_ref[t, i] * bo[j]
    assert_within_bound(y[rows][:, cols], y_ref[rows], bound[rows],
                        what=f"{cfg.name} T={T} all tokens, {len(cols)} columns")
    return layer, ws, rows


def _grouped_x_with_all_row_counts(T=16):
    """Decode rows of the grouped layer whose routing gives routed experts
    with 1, 2 and at least 3 rows (the first seed that does): at hidden 7168
    the dot-product blocking is 2 rows, so experts with 3 or more rows (and
    the 16-row shared expert) take the matrix-core branch."""
    cfg = configs.GROUPED
    layer = _layer(cfg)
    for seed in range(8):
        x, xg = _x(cfg, T, seed)
        _, ws = layer.forward(xg)
        counts = np.diff(to_np(ws["offsets"]))[:cfg.E]
        if (counts == 1).any() and (counts == 2).any() and (counts >= 3).any():
            return x, seed
    raise AssertionError("no seed gives experts with 1, 2 and >= 3 rows")


def test_grouped_layer_full_size_all_tokens():
    """256 Q4_K experts + Q8_0 shared, hidden 7168, FFN 2048, 16 bf16 rows:
    all 16 tokens against the oracle on 64 sampled output columns, with a
    routing that exercises the one-row and two-row dot products and the
    matrix-core branch (experts with >= 3 rows, the shared expert)."""
    x, seed = _grouped_x_with_all_row_counts()
    cols = np.sort(np.random.default_rng(0).choice(7168, 64, replace=False))
    _, ws, rows = _check_all_tokens_sampled_cols(configs.GROUPED, 16, cols, x=x)
    counts = np.diff(to_np(ws["offsets"]))
    assert counts[configs.GROUPED.E] == 16       # the shared expert sees every row
    assert rows.size == 16


def test_ffn_and_combine_isolated_with_sentinels_and_duplicates():
    cfg = SMALL_TIERED
    layer = _layer(cfg)
    T, k = 9, 4
    x, xg = _x(cfg, T, seed=3)
    ids = synth.random_ids(T, k, cfg.E, 3, distinct=False)   # duplicates within a token
    ids[0, 1] = -1                                            # skip sentinel
    ids[2, 3] = cfg.E + 5                                     # out of range: skipped
    ids[4] = 2                                                # one expert, four times
    p = synth.random_weights(T, k, 3)
    off, perm, inv = qmoe.permute(to_gpu(ids), cfg.E)
    off_r, perm_r, inv_r = moe.permute(ids, cfg.E)
    assert (to_np(off) == off_r).all() and (to_np(perm) == perm_r).all()
    o = qmoe.ffn_tiered(layer.tier_arrays[0], cfg.E, cfg.H, cfg.F, xg, k, off, perm)
    cache = ExpertCache(layer)
    o_ref, bo = moe.ffn_permuted(x, ids, off_r, perm_r, cache, cfg.H, cfg.F, k)
    n = off_r[-1]
    assert_within_bound(to_np(o)[:n], o_ref[:n], bo[:n], what="ffn permuted rows")
    shared = synth.normal((T, cfg.H), 1.0, 4, synth.ACT)
    y = qmoe.combine(o, inv, to_gpu(p), T, k, cfg.H, shared=to_gpu(shared))
    y_ref, _ = moe.combine(o_ref, inv_r, p, T, k, shared=shared)
    # the error of each o row is bounded by its own bound, so the output's is
    # sum_i p_i * B_o[inv_i] (+ |shared| for the fp32 addition)
    by = np.abs(shared).astype(np.float64)
    for t in range(T):
        for s_ in range(k):
            if inv_r[t * k + s_] >= 0:
                by[t] += p[t, s_] * bo[inv_r[t * k + s_]]
    assert_within_bound(to_np(y), y_ref, by, what="combine")


def test_combine_exact_order():
    """combine is a fixed-order fp32 fma chain: compare with the same chain."""
    T, k, H = 7, 5, 64
    rng = np.random.default_rng(2)
    o = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    inv[3] = -1
    p = synth.random_weights(T, k, 2)
    y = to_np(qmoe.combine(to_gpu(o), to_gpu(inv), to_gpu(p), T, k, H))
    ref = np.zeros((T, H), np.float32)
    for t in range(T):
        for s in range(k):
            if inv[t * k + s] >= 0:
                ref[t] = (p[t, s].astype(np.float64) * o[inv[t * k + s]] + ref[t]).astype(np.float32)
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()


def test_token_reorder_permutes_outputs_bitexactly():
    cfg = configs.TIERED
    layer = _layer(cfg)
    x, xg = _x(cfg, 6, seed=5)
    y1 = to_np(layer.forward(xg)[0]).copy()
    sigma = np.array([3, 0, 5, 1, 4, 2])
    y2 = to_np(layer.forward(xg[torch.from_numpy(sigma).cuda()].contiguous())[0])
    assert_bitexact(y2, y1[sigma], "reordered tokens")


def test_layer_is_deterministic():
    cfg = configs.TIERED
    layer = _layer(cfg)
    _, xg = _x(cfg, 6, seed=6)
    a = to_np(layer.forward(xg)[0]).copy()
    b = to_np(layer.forward(xg)[0])
    assert (a == b).all()


def test_empty_and_zero_token_calls():
    cfg = SMALL_TIERED
    layer = _layer(cfg)
    xg = torch.empty((0, cfg.H), dtype=torch.float32, device="cuda")
    ids, p = qmoe.route(xg, layer.Wr, layer.bias, cfg.k)
    assert ids.shape == (0, cfg.k)


# -------------------------------------------------------------- prefill ---

# The prefill path rounds x, the dequantized weights and h to fp16 (2^-11).  Its
# error relative to sum|w x| falls like 1/sqrt(K), so these layers keep
# reduction lengths of several hundred values or more with fewer experts.
PREFILL_TIERED = MoEConfig("prefill_tiered_small", H=2048, E=24, k=6, F=640,
                           tiers=(Tier(0, 6, "q6_k", "q8_0"), Tier(6, 19, "q4_k", "q4_0"),
                                  Tier(19, 24, "mxfp4", "mxfp4")), rows=(300,),
                           prior_lambda=0.5)
PREFILL_SHARED = MoEConfig("prefill_shared_small", H=1024, E=16, k=4, F=1024,
                           tiers=(Tier(0, 16, "q4_k", "q4_k"),), rows=(200,), x_dtype="bf16",
                           n_shared=1, shared_fmt="q8_0")
# ragged everywhere: H = 34 units of 32 and F = 10 units (K steps of 4 units
# end short in both passes), H not a multiple of the 128-column down tile,
# experts with more rows than one 128-row tile
PREFILL_RAGGED = MoEConfig("prefill_ragged", H=1088, E=10, k=3, F=320,
                           tiers=(Tier(0, 4, "q8_0", "q8_0"), Tier(4, 8, "q4_0", "q4_0"),
                                  Tier(8, 10, "mxfp4", "mxfp4")), rows=(260,),
                           prior_lambda=0.5)


@pytest.mark.parametrize("cfg,T", [(PREFILL_TIERED, 300), (PREFILL_SHARED, 200),
                                   (PREFILL_RAGGED, 260)])
def test_prefill_small_layers(cfg, T):
    _check_layer(cfg, T, prefill=True)


@pytest.mark.parametrize("cfg,T", [(PREFILL_TIERED, 300), (PREFILL_RAGGED, 260)])
@pytest.mark.parametrize("prefill", [True, False])
def test_partial_routing_writes_only_the_kept_rows(cfg, T, prefill):
    """offsets[E] < T*k: the expert FFN (qgemm_grouped_prefill or
    moe_ffn_tiered) on a routing that keeps only some experts' rows gives
    those rows exactly as the full call does (each kept expert has the same
    rows, so the same tiles) and leaves o[pos] for pos >= offsets[E]
    untouched."""
    layer = _layer(cfg)
    _, xg = _x(cfg, T, seed=5)
    _, ws = layer.forward(xg, prefill=prefill)
    o_full = to_np(ws["o"]).copy()
    offs = to_np(ws["offsets"]).astype(np.int64)
    perm = to_np(ws["perm"])
    cnt = np.diff(offs)
    E, kt = cfg.E_total, cfg.k + cfg.n_shared
    # every other expert in order of row count, and the busiest one
    nz = np.nonzero(cnt > 0)[0]
    nz = nz[np.argsort(cnt[nz], kind="stable")]
    keep = np.zeros(E, bool)
    keep[nz[0::2]] = True
    keep[nz[-1]] = True
    off2 = np.zeros(E + 1, np.int32)
    off2[1:] = np.cumsum(np.where(keep, cnt, 0))
    p2 = np.zeros(T * kt, np.int32)
    p2[:off2[E]] = np.concatenate([perm[offs[e]:offs[e + 1]] for e in np.nonzero(keep)[0]])
    o2 = torch.full_like(ws["o"], 12345.0)
    L = qmoe.lib()
    fn = L.qgemm_grouped_prefill if prefill else L.moe_ffn_tiered
    arr = layer.tier_arrays[0]
    off_t, p_t = to_gpu(off2), to_gpu(p2)
    qmoe._check(fn(arr, len(arr), E, cfg.H, cfg.F, qmoe._p(xg), qmoe._dtype_code(xg), T, kt,
                   qmoe._p(off_t), qmoe._p(p_t), qmoe._p(o2), qmoe._p(ws["ffn"]),
                   ws["ffn"].numel(), qmoe._stream()), "expert ffn")
    got = to_np(o2)
    for e in np.nonzero(keep)[0]:
        assert_bitexact(got[off2[e]:off2[e + 1]], o_full[offs[e]:offs[e + 1]],
                        f"{cfg.name} prefill={prefill} expert {e}")
    assert (got[off2[E]:] == 12345.0).all()


def test_prefill_matches_decode_path():
    cfg = configs.TIERED
    layer = _layer(cfg)
    _, xg = _x(cfg, 64, seed=7)
    yd = to_np(layer.forward(xg)[0]).copy()
    yp = to_np(layer.forward(xg, prefill=True)[0])
    # both are within 1e-3 of the exact layer; their difference is bounded by
    # the sum of the two allowances (relative to the output's own bound)
    scale = np.abs(yd).max()
    assert np.abs(yd - yp).max() <= 2e-2 * scale


def test_prefill_chunk_full_size_all_tokens():
    """2048 tokens through the 512-expert tiered layer on the matrix cores:
    every token against the oracle on 64 sampled output columns."""
    cols = np.sort(np.random.default_rng(3).choice(2048, 64, replace=False))
    _check_all_tokens_sampled_cols(configs.PREFILL, 2048, cols, prefill=True)


# ------------------------------------------------ one-launch decode layer --

ONE_LAUNCH_CASES = [(configs.TINY, 4), (SMALL_TIERED, 1), (SMALL_TIERED, 5), (SMALL_TIERED, 16),
                    (SMALL_SHARED, 16), (SMALL_SHARED, 2), (configs.TIERED, 1),
                    (configs.TIERED, 6), (configs.TIERED, 3)]


def _counter_words(ws):
    """The counters (first 16384 bytes of the workspace): nonzero
    words, at most 3 listed; [] when all are zero as every call must leave them."""
    w = to_np(ws["layer"][:16384].view(torch.int32))
    return w[w != 0][:3].tolist()


@pytest.mark.parametrize("cfg,T", ONE_LAUNCH_CASES, ids=lambda v: getattr(v, "name", v))
def test_one_launch_layer_matches_oracle(cfg, T):
    _, _, ws = _check_layer(cfg, T, seed=7, one_launch=True)
    assert _counter_words(ws) == []


@pytest.mark.parametrize("cfg,T", ONE_LAUNCH_CASES, ids=lambda v: getattr(v, "name", v))
def test_one_launch_layer_equals_separate_calls_bitexactly(cfg, T):
    """Same arithmetic as route_decode + ffn_tiered + combine: ids, p,
    offsets, perm, inv_perm and y are equal bit for bit."""
    layer = _layer(cfg)
    _, xg = _x(cfg, T, seed=8)
    y, ws = layer.forward(xg)
    ref = {k: to_np(ws[k]).copy() for k in ("y", "ids", "p", "offsets", "perm", "inv")}
    for k in ("y", "ids", "p", "offsets", "perm", "inv"):
        ws[k].fill_(-7)
    layer.forward(xg, one_launch=True)
    for k, v in ref.items():
        got = to_np(ws[k])
        if v.dtype == np.float32:
            assert_bitexact(got, v, f"{cfg.name} T={T} {k}")
        else:
            assert (got == v).all(), f"{cfg.name} T={T} {k}"
    assert _counter_words(ws) == []


def test_one_launch_grouped_full_size_all_tokens():
    """The 16-row grouped layer in one launch (hidden 7168: the dot-product
    blocking drops to 2 rows, so the shared expert and experts with 3 or more
    rows run on the matrix cores in both phases): all 16 tokens on 64
    sampled columns."""
    x, _ = _grouped_x_with_all_row_counts()
    cols = np.sort(np.random.default_rng(1).choice(7168, 64, replace=False))
    _check_all_tokens_sampled_cols(configs.GROUPED, 16, cols, x=x, one_launch=True)


def test_one_launch_repeated_calls_reuse_the_counter():
    """Calls of different row counts back to back on one workspace each leave
    the barrier counter at zero and give the same results as before."""
    cfg = configs.TIERED
    layer = _layer(cfg)
    outs = {}
    for rep in range(2):
        for T in (1, 6, 1, 16):
            _, xg = _x(cfg, T, seed=10 + T)
            y, ws = layer.forward(xg, one_launch=True)
            yv = to_np(y).copy()
            assert _counter_words(ws) == []
            if T in outs:
                assert (outs[T] == yv).all()
            outs[T] = yv


def test_one_launch_wide_hidden_on_the_matrix_cores():
    """A 28672-wide hidden row does not fit the LDS staging of the dot-product
    path; the one-launch layer then runs every gate/up item on the matrix
    cores, as moe_ffn_tiered does, and equals the separate calls bit for bit."""
    layer = _layer(WIDE_HIDDEN)
    _, xg = _x(WIDE_HIDDEN, 3)
    y_sep = to_np(layer.forward(xg)[0]).copy()
    y, ws = layer.forward(xg, one_launch=True)
    assert_bitexact(to_np(y), y_sep, "wide hidden one launch")
    assert _counter_words(ws) == []


def test_one_launch_limits():
    cfg = SMALL_TIERED
    layer = _layer(cfg)
    _, xg = _x(cfg, 17)
    with pytest.raises(RuntimeError, match="rows"):
        qmoe.layer_decode(layer.tier_arrays[0], cfg.E, cfg.H, cfg.F, xg, layer.Wr, layer.bias,
                          cfg.k)
