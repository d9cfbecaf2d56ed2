"""MXFP8 activation quantizer (bit-exact) and the block-scaled MXFP4 x MXFP8
GEMM (exact-grid bit-exact; random data within the parity bound) against the
oracle."""
import numpy as np
import pytest

from gpu_util import requires_gpu, to_gpu, to_np, assert_bitexact, assert_within_bound, torch
from oracle import formats as fm
from oracle import mx
from decode_moe_mul_amd import qmoe, synth

pytestmark = [pytest.mark.gpu, requires_gpu]


def _cases():
    rng = np.random.default_rng(0)
    yield "normal", rng.normal(0, 1, (7, 2048)).astype(np.float32)
    yield "scaled rows", (rng.normal(0, 1, (9, 96)) * np.exp2(rng.integers(-40, 40, (9, 1)))).astype(np.float32)
    x = np.zeros((6, 64), np.float32)
    x[0, :32] = 1.0                                  # exact powers of two
    x[1, 0] = 1.99                                   # saturates at 448 * 2^-8
    x[1, 1:32] = rng.uniform(-1, 1, 31)
    x[2, 0], x[2, 1] = 256.0, 1.0625                 # tie: 1.0625 * 2^0 -> even code
    x[2, 2], x[2, 3] = 1.1875, -1.1875
    x[3, 0], x[3, 1:8] = 1.0, np.float32(2.0 ** -15) * np.arange(1, 8)   # E4M3 subnormals
    x[4, 32:] = -0.0                                 # zero block of negative zeros
    x[5] = rng.uniform(-3e-38, 3e-38, 64)            # amax near the fp32 normal floor
    yield "special", x
    # every E4M3 value times its block scale, plus the midpoints between them
    grid = mx.e4m3_value(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids, -mids])
    pad = (-len(vals)) % 31
    vals = np.concatenate([vals, np.zeros(pad)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((vals.shape[0], 1), 448.0), vals], axis=1)  # pin E = 0
    yield "grid and midpoints", (blocks.reshape(1, -1) * 2.0 ** -3).astype(np.float32)


@pytest.mark.parametrize("name,x", list(_cases()), ids=[c[0] for c in _cases()])
def test_activation_quantizer_bitexact(name, x):
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    rc, rs = mx.quantize_mxfp8(x.astype(np.float64))
    assert (to_np(scales) == rs).all(), name
    got = to_np(codes)
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{name}: {len(bad)} codes differ, first {tuple(bad[0])}: {got[tuple(bad[0])]:#x} vs {rc[tuple(bad[0])]:#x}"


def test_activation_quantizer_bf16_input():
    x = synth.bf16_round(synth.normal((5, 256), 1.0, 3, synth.ACT, 5))
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x).to(torch.bfloat16))
    rc, rs = mx.quantize_mxfp8(x.astype(np.float64))
    assert (to_np(codes) == rc).all() and (to_np(scales) == rs).all()


def _w(N, K, seed, sigma=0.02):
    return synth.normal((N, K), sigma, seed, synth.GATE, 0)


@pytest.mark.parametrize("N,K,R", [(16, 128, 16), (48, 256, 33), (130, 384, 70)])
def test_gemm_exact_grid_bitexact(N, K, R):
    """Weights with E8M0 = 127 (unit scale) and activation codes on a coarse
    grid with unit scales: every product and every partial sum is exact in
    fp32, so any summation order gives the oracle's value exactly (this also
    pins the operand layout: a wrong pairing of K positions changes sums)."""
    rng = np.random.default_rng(N + K + R)
    wcodes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    buf = fm.pack("mxfp4", {"q": wcodes, "e": np.full((N, K // 32), 127, np.uint8)}, N, K)
    # zero or E4M3 values 1 .. 3.75 (steps of 1/8), both signs: products are
    # multiples of 1/16 below 23, sums stay below 2^14
    acodes = np.where(rng.random((R, K)) < 0.2, 0, rng.integers(0x38, 0x48, (R, K)))
    acodes = (acodes | (rng.integers(0, 2, (R, K)) << 7)).astype(np.uint8)
    ascales = np.full((R, K // 32), 127, np.uint8)
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, to_gpu(acodes), to_gpu(ascales)))
    ref = mx.dequantize_mxfp8(acodes, ascales) @ fm.dequantize("mxfp4", buf, N, K).T
    assert_bitexact(y, ref, f"exact grid {N}x{K} R={R}")


@pytest.mark.parametrize("N,K,R", [(640, 2048, 40), (2048, 640, 33), (130, 384, 70), (16, 128, 1),
                                   (256, 1024, 129)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_gemm_within_bound(N, K, R, x_dtype):
    x = synth.normal((R, K), 1.0, 7, synth.ACT, R)
    if x_dtype == "bf16":
        x = synth.bf16_round(x)
    W = _w(N, K, 11)
    buf = fm.quantize("mxfp4", W)
    xg = to_gpu(x) if x_dtype == "f32" else to_gpu(x).to(torch.bfloat16)
    codes, scales = qmoe.quantize_act_mxfp8(xg)
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, codes, scales))
    ref, bound = mx.mx_gemm(buf, N, K, x.astype(np.float64))
    assert_within_bound(y, ref, bound, what=f"mx gemm {N}x{K} R={R}")


def test_gemm_full_size_sampled_columns():
    """A Llama-size MXFP4 matrix [14336, 4096] against 256 rows: the oracle
    checks 48 sampled output columns (MXFP4 quantizes each weight row on its
    own, so the sampled rows' bytes are the full matrix's)."""
    N, K, R = 14336, 4096, 256
    W = synth.normal_device((N, K), 0.02, 3, synth.UP, 0, "cuda")
    buf = qmoe.quantize("mxfp4", W)
    x = synth.normal((R, K), 1.0, 9, synth.ACT, 1)
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    y = to_np(qmoe.gemm_mxfp4_mxfp8(buf, N, K, codes, scales))
    cols = np.sort(np.random.default_rng(4).choice(N, 48, replace=False))
    Wc = to_np(W[torch.from_numpy(cols).cuda()])
    ref, bound = mx.mx_gemm(fm.quantize("mxfp4", Wc), len(cols), K, x.astype(np.float64))
    assert_within_bound(y[:, cols], ref, bound, what="mx gemm 14336x4096 sampled")


def test_quantized_activation_error_against_fp_activations():
    """Context, not parity: the MXFP8 activations move each output by a few
    parts in a thousand of sum |w x| against the unquantized product."""
    N, K, R = 640, 2048, 64
    x = synth.normal((R, K), 1.0, 5, synth.ACT, 2)
    buf = fm.quantize("mxfp4", _w(N, K, 12))
    codes, scales = qmoe.quantize_act_mxfp8(to_gpu(x))
    y = to_np(qmoe.gemm_mxfp4_mxfp8(to_gpu(buf), N, K, codes, scales))
    w = fm.dequantize("mxfp4", buf, N, K)
    exact = x.astype(np.float64) @ w.T
    rel = np.abs(y - exact) / (np.abs(x) @ np.abs(w).T)
    assert rel.max() < 2e-2 and np.median(rel) < 2e-3


# ------------------------------------------------ prefill, MXFP4 tier ----
from decode_moe_mul_amd.configs import Tier  # noqa: E402

def _h_slack(h, dbuf, H, F, rel=1e-6):
    """Slack for the MXFP8 decisions on h: the device's h = SiLU(g) u may
    differ from the oracle's by a few fp32 roundings (rel of |h|); an element
    whose interval |h| +- rel |h| holds more than one E4M3 code (or whose
    block's largest interval crosses a power of two, the scale decision) may
    take any of those values.  Returns, per output, sum_j |w_d[n, j]| times
    the spread of element j's valid dequantized values, and the fraction of
    elements with a choice."""
    R = h.shape[0]
    dh = rel * np.abs(h) + 1e-300
    lo_h, hi_h = np.maximum(np.abs(h) - dh, 0), np.abs(h) + dh
    spread = np.zeros_like(h)
    for r in range(R):
        for b in range(F // 32):
            sl = slice(32 * b, 32 * b + 32)
            ex = {int(np.clip(np.frexp(a)[1] - 9, -127, 127))
                  for a in (lo_h[r, sl].max(), hi_h[r, sl].max()) if a > 0}
            vals = [mx.e4m3_value(mx.e4m3_code_of_magnitude(m * 2.0 ** -E)) * 2.0 ** E
                    for E in ex for m in (lo_h[r, sl], hi_h[r, sl])]
            if vals:
                v = np.array(vals)
                spread[r, sl] = v.max(0) - v.min(0)
    wd = fm.dequantize("mxfp4", dbuf, H, F)
    return spread @ np.abs(wd).T, float((spread > 0).mean())


MX_SHAPES = [("mx_small", 256, 64), ("mx_ragged", 1088, 320)]
MX_TIERS = (Tier(0, 4, "q8_0", "q8_0"), Tier(4, 8, "q4_0", "q4_0"), Tier(8, 10, "mxfp4", "mxfp4"))


def _mx_bank(H, F, seed, exact_gate_up):
    """Tier banks of a 10-expert layer; the MXFP4 tier's gate/up either
    realistic (quantized normals) or on an exact grid: E2M1 codes with one
    shared scale 2^-6, so that against grid activations every partial sum of
    g and u is exact in fp32."""
    rng = np.random.default_rng(seed)
    host = []
    for t in MX_TIERS:
        n = t.e_end - t.e_begin
        gs, us, ds = [], [], []
        for _ in range(n):
            if t.fmt_gate_up == "mxfp4" and exact_gate_up:
                e = np.full((F, H // 32), 121, np.uint8)
                g = fm.pack("mxfp4", {"q": rng.integers(0, 16, (F, H)).astype(np.uint8), "e": e}, F, H)
                u = fm.pack("mxfp4", {"q": rng.integers(0, 16, (F, H)).astype(np.uint8), "e": e}, F, H)
            else:
                g = fm.quantize(t.fmt_gate_up, rng.normal(0, 0.02, (F, H)))
                u = fm.quantize(t.fmt_gate_up, rng.normal(0, 0.02, (F, H)))
            gs.append(g); us.append(u)
            ds.append(fm.quantize(t.fmt_down, rng.normal(0, 0.02, (H, F))))
        host.append((gs, us, ds))
    dev = [(t.e_begin, t.e_end, t.fmt_gate_up, t.fmt_down,
            to_gpu(np.concatenate(gs)), to_gpu(np.concatenate(us)), to_gpu(np.concatenate(ds)))
           for t, (gs, us, ds) in zip(MX_TIERS, host)]
    return host, dev


def _grid_x(T, H, seed):
    """Activations in {0, +-1, +-1.5, +-2, +-3} with a 2 or 3 leading every
    32-value block: the block scale is 2^-7 and every value is an E4M3 value
    times it, so quantizing x to MXFP8 changes nothing."""
    rng = np.random.default_rng(seed)
    x = rng.choice([0.0, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0, 3.0, -3.0], size=(T, H))
    x[:, ::32] = rng.choice([2.0, -2.0, 3.0, -3.0], size=(T, H // 32))
    return x.astype(np.float32)


def _run_mx_prefill(H, F, T, x, dev):
    E, k = 10, 3
    rng = np.random.default_rng(T + H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[: min(T, 4), 0] = E - 1  # the MXFP4 tier gets several rows of one expert
    offsets, perm, inv = qmoe.permute(to_gpu(ids), E)
    arr = qmoe.tiers_struct(dev)
    xg = to_gpu(x)
    o16 = to_np(qmoe.grouped_prefill(arr, E, H, F, xg, k, offsets, perm))
    omx = to_np(qmoe.grouped_prefill_mx(arr, E, H, F, xg, k, offsets, perm))
    return o16, omx, to_np(offsets), to_np(perm), k


@pytest.mark.parametrize("name,H,F", MX_SHAPES, ids=[m[0] for m in MX_SHAPES])
@pytest.mark.parametrize("T", [5, 150])
def test_prefill_mx_tier_exact_gate_up(name, H, F, T):
    """MXFP4/MXFP4 experts on the block-scaled path: with exact g and u the
    only open decisions are h's MXFP8 codes at fp32 rounding distance from a
    tie (slack below); the down projection must then be within 1e-3 of
    sum |w_d q(h)|.  Every other expert's rows equal qgemm_grouped_prefill
    bit for bit."""
    host, dev = _mx_bank(H, F, 7, exact_gate_up=True)
    x = _grid_x(T, H, T)
    o16, omx, off, pm, k = _run_mx_prefill(H, F, T, x, dev)
    checked = 0
    for e in range(10):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        if e < 8:
            assert_bitexact(omx[rows], o16[rows], f"{name} expert {e} (fp16 path)")
            continue
        gs, us, ds = host[2]
        gbuf, ubuf, dbuf = gs[e - 8], us[e - 8], ds[e - 8]
        X = x[pm[rows] // k].astype(np.float64)
        g, _ = mx.mx_gemm(gbuf, F, H, X)
        u, _ = mx.mx_gemm(ubuf, F, H, X)
        assert np.array_equal(mx.dequantize_mxfp8(*mx.quantize_mxfp8(X)), X)  # q(x) = x
        h = g / (1.0 + np.exp(-g)) * u
        ref, bound = mx.mx_gemm(dbuf, H, F, h)
        slack, frac = _h_slack(h, dbuf, H, F)
        assert frac < 1e-3, frac  # the decisions are almost all unique
        err = np.abs(omx[rows] - ref)
        lim = 1e-3 * bound + slack
        assert (err <= lim).all(), f"{name} mx expert {e}: worst ratio {(err / lim).max():.3g}"
        checked += rows.size
    assert checked > 0


def _silu_range(a, b):
    """Range of SiLU over [a, b] (elementwise): SiLU falls until its minimum
    at g* = -1.27846... and rises after it."""
    silu = lambda g: g / (1.0 + np.exp(-g))
    gstar = -1.2784645427610738
    lo = np.minimum(silu(a), silu(b))
    lo = np.where((a < gstar) & (b > gstar), silu(gstar), lo)
    return lo, np.maximum(silu(a), silu(b))


def _q_mxfp8_signed(h, E):
    """h quantized to E4M3 with the block exponent E (broadcast): monotone
    non-decreasing in h."""
    scale = np.ldexp(1.0, E)
    mag = mx.e4m3_value(mx.e4m3_code_of_magnitude(np.abs(h) / scale)) * scale
    return np.where(h < 0, -mag, mag)


def _h_decision_slack(g, u, bg, bu, dbuf, H, F, gamma=2.0 ** -18, rel_h=1e-6):
    """Computed slack for the MXFP8 decisions on h.  The device's g and u
    are fp32 sums of exact products on the matrix cores, rounded at most
    once per 32-value scale block (64 roundings at K = 2048), so they are
    within gamma * sum |w q(x)| of the oracle's (gamma = 64 * 2^-24), and its
    h = SiLU(g) u within rel_h |h| more.  So each h_j lies in an interval [lo_j, hi_j]; its block
    exponent may be any exponent of a block maximum in the interval of block
    maxima, and its quantized value anything between Q_E(lo_j) and Q_E(hi_j)
    over those exponents (quantization is monotone).  Returns per output
    sum_j |w_d[n, j]| * (that range's width), and the fraction of h elements
    with more than one possible value."""
    eg, eu = gamma * bg, gamma * bu
    s_lo, s_hi = _silu_range(g - eg, g + eg)
    c = np.stack([s_lo * (u - eu), s_lo * (u + eu), s_hi * (u - eu), s_hi * (u + eu)])
    h_lo, h_hi = c.min(0), c.max(0)
    h_lo = h_lo - rel_h * np.abs(h_lo)
    h_hi = h_hi + rel_h * np.abs(h_hi)
    R = g.shape[0]
    mag_lo = np.where(h_lo > 0, h_lo, np.where(h_hi < 0, -h_hi, 0.0))
    mag_hi = np.maximum(np.abs(h_lo), np.abs(h_hi))
    blo = mag_lo.reshape(R, F // 32, 32).max(-1)
    bhi = mag_hi.reshape(R, F // 32, 32).max(-1)

    def exp_of(a):  # the stored scale's exponent: floor(log2 a) - 8, clamped
        return np.clip(np.frexp(np.maximum(a, 1e-300))[1] - 1 - 8, -127, 127)

    e_lo, e_hi = exp_of(blo), exp_of(bhi)
    assert (e_hi - e_lo <= 1).all()
    vmin = np.full_like(h_lo, np.inf)
    vmax = np.full_like(h_lo, -np.inf)
    for e_b in (e_lo, e_hi):
        E = np.repeat(e_b, 32, axis=1)
        vmin = np.minimum(vmin, _q_mxfp8_signed(h_lo, E))
        vmax = np.maximum(vmax, _q_mxfp8_signed(h_hi, E))
    spread = vmax - vmin
    wd = fm.dequantize("mxfp4", dbuf, H, F)
    return spread @ np.abs(wd).T, float((spread > 0).mean())


MX_REAL_SHAPES = MX_SHAPES + [("mx_tail_tier", 2048, 640)]


@pytest.mark.parametrize("name,H,F", MX_REAL_SHAPES, ids=[m[0] for m in MX_REAL_SHAPES])
def test_prefill_mx_tier_realistic_elementwise(name, H, F):
    """MXFP4/MXFP4 experts on realistic weights and activations, up to the
    tail tier's real shape (hidden 2048, FFN 640): every output within 1e-3
    of sum |w_d q(h)| plus the computed slack of h's MXFP8 decisions near a
    rounding or scale boundary (_h_decision_slack); the other tiers equal
    qgemm_grouped_prefill bit for bit.  x's own MXFP8 codes are decided in
    fp32 on both sides, identically."""
    T = 150
    host, dev = _mx_bank(H, F, 9, exact_gate_up=False)
    x = synth.normal((T, H), 1.0, 3, synth.ACT, T)
    o16, omx, off, pm, k = _run_mx_prefill(H, F, T, x, dev)
    checked, choice = 0, []
    for e in range(10):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        if e < 8:
            assert_bitexact(omx[rows], o16[rows], f"{name} expert {e} (fp16 path)")
            continue
        gs, us, ds = host[2]
        gbuf, ubuf, dbuf = gs[e - 8], us[e - 8], ds[e - 8]
        X = x[pm[rows] // k].astype(np.float64)
        ref, bound = mx.mx_expert_ffn(gbuf, ubuf, dbuf, H, F, X)
        g, bg = mx.mx_gemm(gbuf, F, H, X)
        u, bu = mx.mx_gemm(ubuf, F, H, X)
        slack, frac = _h_decision_slack(g, u, bg, bu, dbuf, H, F)
        choice.append(frac)
        err = np.abs(omx[rows] - ref)
        lim = 1e-3 * bound + slack
        assert (err <= lim).all(), f"{name} mx expert {e}: worst ratio {(err / lim).max():.3g}"
        # the slack is not what carries the comparison: most outputs have none
        assert np.median(slack / bound) < 1e-3, np.median(slack / bound)
        checked += rows.size
    assert checked > 0
    assert max(choice) < 0.05, choice
