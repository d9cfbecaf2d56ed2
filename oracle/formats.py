"""Oracle block formats: quantize, pack, unpack, dequantize (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the formats this path streams but print no byte layout:
  * "RTX 3090 Llama 70B three-tier cache" page (bjdmk), section 一 "项目核心释义":
    GGUF Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K.
  * "Three RTX 3090 Qwen3.8-Flash-Next guide" page (n1n.ai), section
    "优化策略二" (tiers): Q6_K gate/up + Q8_0 down for hot experts, 4-bit
    middle tier, MXFP4 for the tail; down projection width 640 rules out
    256-value blocks for it.
The field widths and value formulas used here are the workload's statement of
those formats; the byte arrangement ("planes") is this project's own:

  A tensor W[N, K] quantized along K in blocks of B values (nb = K / B blocks
  per row) is stored as a sequence of planes.  Each plane holds one per-block
  field for all rows, row-major [N][nb][field bytes].  Every plane starts at a
  256-byte aligned offset from the tensor base; the tensor size is the end of
  the last plane rounded up to 256.

  Q8_0  B=32   plane 0: q  int8  x32           value d*q
               plane 1: d  fp16
  Q4_0  B=32   plane 0: q  4-bit x32 (16 B)    value d*(q-8)
               plane 1: d  fp16
  MXFP4 B=32   plane 0: q  E2M1 x32 (16 B)     value 2^(e-127) * E2M1(q)
               plane 1: e  uint8 (E8M0)
  Q4_K  B=256  plane 0: q  4-bit x256 (128 B)  value d*sc_j*q - dmin*m_j
               plane 1: meta 16 B: fp16 d, fp16 dmin, then a 96-bit
                        little-endian field with sc_j at bits 6j..6j+5 and
                        m_j at bits 48+6j..48+6j+5 (j = 0..7); sub-block j is
                        elements 32j..32j+31 of the block
  Q6_K  B=256  plane 0: ql low 4 bits x256 (128 B)   value d*sc_j*(q-32)
               plane 1: qh high 2 bits x256 (64 B)
               plane 2: sc int8 x16
               plane 3: d  fp16; sub-block j is elements 16j..16j+15

  T5    B=128  plane 0: 28-byte groups: bytes 0..25 base-3 codes, bytes 26..27
               fp16 d                  value d*t, t in {-1, 0, +1}
               (the "t5_g128_fp16" ternary format of the "RTX 4080 SUPER
               native Windows 27B: NInfer 80 SM port" page, section 九.2:
               base-3, five weights per byte, one FP16 scale per 128
               weights, 1.75 bits per weight.)  Weight i of a group is digit
               i mod 5 (least significant first) of code byte i div 5; a
               digit holds t + 1.  Byte 25 holds weights 125..127 in digits
               0..2 and t = 0 in digits 3..4.  26 + 2 bytes per 128 weights
               is exactly the page's 1.75 bits per weight.

  4-bit packing: element i of a row lives in byte i>>1 of the row's plane
  slice, low nibble for even i.  Q6_K high bits: element i lives in byte i>>2,
  bits 2*(i&3)..2*(i&3)+1.  E2M1 code: bit 3 sign, bits 2-1 exponent, bit 0
  mantissa; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} (OCP Microscaling
  Formats specification v1.0, FP4 E2M1 element type).  E8M0 code 255 is NaN.

Quantizer readings (the pages give none; the Q8_0 rule is the workload's):
  * T5: d = fp16(mean |w|) over the group, t = clamp(round(w/d), -1, 1)
    (the absolute-mean scale of ternary weight quantization);
  * all arithmetic in float64 on the float32 input values;
  * scales are rounded to fp16 round-to-nearest-even, and codes are computed
    against the *stored* fp16 scale;
  * code rounding is round-half-away-from-zero, then clamped;
  * a zero divisor gives a pre-offset code of 0.
"""
import numpy as np

FORMATS = ("q8_0", "q4_0", "mxfp4", "q4_k", "q6_k")
# the ternary format has its own tests (it is not a tier format of the layer)
TERNARY = ("t5",)
BLOCK = {"q8_0": 32, "q4_0": 32, "mxfp4": 32, "q4_k": 256, "q6_k": 256, "t5": 128}
# bits per weight of the densely packed form (planes add only alignment)
BITS_PER_WEIGHT = {"q8_0": 8.5, "q4_0": 4.5, "mxfp4": 4.25, "q4_k": 4.5,
                   "q6_k": 6.5625, "t5": 1.75}
T5_GROUP_BYTES = 28   # 26 code bytes + fp16 d
E2M1_MAGNITUDE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


# ---------------------------------------------------------------- layout ---

def _round_up(n, a=256):
    return (n + a - 1) // a * a


def plane_bytes(fmt, N, K):
    """Byte size of each plane of a [N, K] tensor, in storage order."""
    B = BLOCK[fmt]
    if K % B:
        raise ValueError(f"K={K} is not a multiple of the {fmt} block {B}")
    nb = K // B
    if fmt == "q8_0":
        return [N * K, N * nb * 2]
    if fmt == "q4_0":
        return [N * K // 2, N * nb * 2]
    if fmt == "mxfp4":
        return [N * K // 2, N * nb]
    if fmt == "q4_k":
        return [N * K // 2, N * nb * 16]
    if fmt == "q6_k":
        return [N * K // 2, N * K // 4, N * nb * 16, N * nb * 2]
    if fmt == "t5":
        return [N * nb * T5_GROUP_BYTES]
    raise ValueError(fmt)


def plane_offsets(fmt, N, K):
    offs, pos = [], 0
    for size in plane_bytes(fmt, N, K):
        offs.append(pos)
        pos = _round_up(pos + size)
    return offs, pos


def tensor_bytes(fmt, N, K):
    return plane_offsets(fmt, N, K)[1]


def _planes(fmt, buf, N, K):
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    offs, total = plane_offsets(fmt, N, K)
    if buf.size < total:
        raise ValueError("buffer smaller than the tensor")
    return [buf[o:o + s] for o, s in zip(offs, plane_bytes(fmt, N, K))]


# ------------------------------------------------------ scalar helpers -----

def fp16_rne(v):
    """Round float64 values to fp16, round-to-nearest-even (NumPy converts
    double -> half directly, with IEEE rounding, keeping subnormals)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def round_half_away(v):
    """Round float64 values to the nearest integer, halves away from zero."""
    v = np.asarray(v, dtype=np.float64)
    t = np.trunc(v)
    frac = np.abs(v - t)          # exact: v and t share sign and exponent range
    return t + np.where(frac >= 0.5, np.sign(v), 0.0)


def _safe_div(num, den):
    """num / den where den != 0, else 0 (the 'zero divisor' reading)."""
    num = np.asarray(num, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num.shape)
    out = np.zeros(num.shape, dtype=np.float64)
    np.divide(num, den, out=out, where=den != 0)
    return out


def _as_blocks(W, B):
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % B:
        raise ValueError("expected a [N, K] float32 matrix with K % block == 0")
    N, K = W.shape
    return W.astype(np.float64).reshape(N, K // B, B), N, K


# --------------------------------------------------------- quantizers ------
# Each returns the integer/fp16 fields; pack_<fmt> turns them into bytes.

def quantize_q8_0(W):
    """d = fp16(max|w| / 127); q = clamp(round(w / d), -127, 127)."""
    w, N, K = _as_blocks(W, 32)
    d16 = fp16_rne(np.abs(w).max(axis=-1) / 127.0)
    d = d16.astype(np.float64)
    q = np.clip(round_half_away(_safe_div(w, d[..., None])), -127, 127)
    return {"q": q.reshape(N, K).astype(np.int8), "d": d16}


def quantize_q4_0(W):
    """d = fp16(max|w| / 7); q = clamp(round(w / d) + 8, 0, 15)."""
    w, N, K = _as_blocks(W, 32)
    d16 = fp16_rne(np.abs(w).max(axis=-1) / 7.0)
    d = d16.astype(np.float64)
    q = np.clip(round_half_away(_safe_div(w, d[..., None])) + 8, 0, 15)
    return {"q": q.reshape(N, K).astype(np.uint8), "d": d16}


def _e2m1_code_of_magnitude(m):
    """Nearest E2M1 magnitude code for m >= 0, ties to the even code,
    saturating at 6 (the grid is 0, .5, 1, 1.5, 2, 3, 4, 6)."""
    m = np.asarray(m, dtype=np.float64)
    code = np.full(m.shape, 7, dtype=np.uint8)
    # thresholds are the midpoints; '<=' where the tie goes to the lower
    # (even) code, '<' where it goes to the upper (even) code
    code[m <= 5.0] = 6
    code[m < 3.5] = 5
    code[m <= 2.5] = 4
    code[m < 1.75] = 3
    code[m <= 1.25] = 2
    code[m < 0.75] = 1
    code[m <= 0.25] = 0
    return code


def quantize_mxfp4(W):
    """Shared exponent e = 127 + floor(log2 max|w|) - 2 (the E2M1 element's
    largest exponent is 2), clamped to [0, 254]; elements w / 2^(e-127) are
    rounded to the E2M1 grid, ties to even, saturating at +-6.  An all-zero
    block stores e = 0 and zero codes.  Sign bit = (w < 0)."""
    w, N, K = _as_blocks(W, 32)
    amax = np.abs(w).max(axis=-1)
    _, ex = np.frexp(amax)                     # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, np.clip(127 + (ex - 1) - 2, 0, 254), 0).astype(np.int64)
    scale = np.ldexp(1.0, e - 127)[..., None]
    code = _e2m1_code_of_magnitude(np.abs(w) / scale)
    code = code | np.where(w < 0, 8, 0).astype(np.uint8)
    return {"q": code.reshape(N, K).astype(np.uint8), "e": e.astype(np.uint8)}


def quantize_q4_k(W):
    """Per 32-value sub-block j: lo = min(0, min w), s_j = (max w - lo)/15,
    m'_j = 0 - lo.  d = fp16(max_j s_j / 63), dmin = fp16(max_j m'_j / 63),
    sc_j = clamp(round(s_j/d), 0, 63), m_j = clamp(round(m'_j/dmin), 0, 63),
    q = clamp(round((w + dmin*m_j) / (d*sc_j)), 0, 15).  Non-iterative."""
    w, N, K = _as_blocks(W, 256)
    w = w.reshape(N, K // 256, 8, 32)
    lo = np.minimum(0.0, w.min(axis=-1))
    s = (w.max(axis=-1) - lo) / 15.0
    mp = 0.0 - lo                # +0 (not -0) when lo is 0: the sign of a zero is not data
    d16 = fp16_rne(s.max(axis=-1) / 63.0)
    dmin16 = fp16_rne(mp.max(axis=-1) / 63.0)
    d = d16.astype(np.float64)[..., None]
    dmin = dmin16.astype(np.float64)[..., None]
    sc = np.clip(round_half_away(_safe_div(s, d)), 0, 63)
    m = np.clip(round_half_away(_safe_div(mp, dmin)), 0, 63)
    num = w + (dmin * m)[..., None]
    q = np.clip(round_half_away(_safe_div(num, (d * sc)[..., None])), 0, 15)
    return {"q": q.reshape(N, K).astype(np.uint8), "d": d16, "dmin": dmin16,
            "sc": sc.astype(np.uint8), "m": m.astype(np.uint8)}


def quantize_q6_k(W):
    """Per 16-value sub-block j: s_j = max|w| / 31.  d = fp16(max_j s_j / 127),
    sc_j = clamp(round(s_j/d), -128, 127), q = clamp(round(w/(d*sc_j)) + 32,
    0, 63)."""
    w, N, K = _as_blocks(W, 256)
    w = w.reshape(N, K // 256, 16, 16)
    s = np.abs(w).max(axis=-1) / 31.0
    d16 = fp16_rne(s.max(axis=-1) / 127.0)
    d = d16.astype(np.float64)[..., None]
    sc = np.clip(round_half_away(_safe_div(s, d)), -128, 127)
    q = np.clip(round_half_away(_safe_div(w, (d * sc)[..., None])) + 32, 0, 63)
    return {"q": q.reshape(N, K).astype(np.uint8), "d": d16,
            "sc": sc.astype(np.int8)}


def quantize_t5(W):
    """Ternary: per 128-group d = fp16(mean |w|), t = clamp(round(w/d), -1, 1)
    against the stored d (zero divisor: t = 0)."""
    b, N, K = _as_blocks(W, 128)
    d16 = fp16_rne(np.abs(b).mean(axis=2))
    t = np.clip(round_half_away(_safe_div(b, d16.astype(np.float64)[..., None])), -1, 1)
    return {"t": t.astype(np.int8).reshape(N, K), "d": d16}


QUANTIZE = {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0,
            "mxfp4": quantize_mxfp4, "q4_k": quantize_q4_k,
            "q6_k": quantize_q6_k, "t5": quantize_t5}


# ------------------------------------------------------------- packing -----

def _pack_nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8).reshape(codes.shape[0], -1)
    return (c[:, 0::2] & 15) | ((c[:, 1::2] & 15) << 4)


def _pack_q4k_meta(d16, dmin16, sc, m):
    """[N, nb] fp16 d, dmin and [N, nb, 8] 6-bit sc, m -> [N, nb, 16] bytes.
    The 96-bit field is assembled as a low 64-bit word (bits 0..63) and a high
    32-bit word (bits 64..95)."""
    N, nb = d16.shape
    out = np.zeros((N, nb, 16), dtype=np.uint8)
    out[..., 0:2] = d16.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    out[..., 2:4] = dmin16.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    lo = np.zeros((N, nb), dtype=np.uint64)
    hi = np.zeros((N, nb), dtype=np.uint64)
    fields = [(sc[..., j], 6 * j) for j in range(8)] + [(m[..., j], 48 + 6 * j) for j in range(8)]
    for val, pos in fields:
        v = val.astype(np.uint64) & np.uint64(63)
        if pos + 6 <= 64:
            lo |= v << np.uint64(pos)
        elif pos >= 64:
            hi |= v << np.uint64(pos - 64)
        else:                                   # straddles bit 64
            lo |= (v << np.uint64(pos)) & np.uint64(0xFFFFFFFFFFFFFFFF)
            hi |= v >> np.uint64(64 - pos)
    out[..., 4:12] = lo.astype("<u8").view(np.uint8).reshape(N, nb, 8)
    out[..., 12:16] = hi.astype("<u4").view(np.uint8).reshape(N, nb, 4)
    return out


def pack(fmt, fields, N, K):
    """Lay the fields out as the plane format described in the module doc."""
    planes = []
    if fmt == "q8_0":
        planes = [fields["q"].reshape(N, K).view(np.uint8),
                  fields["d"].astype("<f2").view(np.uint8)]
    elif fmt == "q4_0":
        planes = [_pack_nibbles(fields["q"].reshape(N, K)),
                  fields["d"].astype("<f2").view(np.uint8)]
    elif fmt == "mxfp4":
        planes = [_pack_nibbles(fields["q"].reshape(N, K)), fields["e"]]
    elif fmt == "q4_k":
        planes = [_pack_nibbles(fields["q"]),
                  _pack_q4k_meta(fields["d"], fields["dmin"], fields["sc"],
                                 fields["m"])]
    elif fmt == "t5":
        nb = K // 128
        c = fields["t"].astype(np.int64).reshape(N, nb, 128) + 1          # digits 0..2
        c = np.concatenate([c, np.ones((N, nb, 2), dtype=np.int64)], axis=2)  # pad t = 0
        c = c.reshape(N, nb, 26, 5)
        codes = (c * np.array([1, 3, 9, 27, 81], dtype=np.int64)).sum(axis=3)
        grp = np.zeros((N, nb, T5_GROUP_BYTES), dtype=np.uint8)
        grp[..., :26] = codes.astype(np.uint8)
        grp[..., 26:28] = fields["d"].astype("<f2").view(np.uint8).reshape(N, nb, 2)
        planes = [grp]
    elif fmt == "q6_k":
        q = fields["q"].reshape(N, K)
        hi = (q >> 4) & 3
        qh = (hi[:, 0::4] | (hi[:, 1::4] << 2) | (hi[:, 2::4] << 4)
              | (hi[:, 3::4] << 6)).astype(np.uint8)
        planes = [_pack_nibbles(q & 15), qh, fields["sc"].view(np.uint8),
                  fields["d"].astype("<f2").view(np.uint8)]
    else:
        raise ValueError(fmt)
    offs, total = plane_offsets(fmt, N, K)
    buf = np.zeros(total, dtype=np.uint8)
    for o, p in zip(offs, planes):
        p = np.ascontiguousarray(p).reshape(-1).view(np.uint8)
        buf[o:o + p.size] = p
    return buf


def quantize(fmt, W, rows_per_chunk=64):
    """float32 [N, K] -> packed bytes (uint8, tensor_bytes(fmt, N, K)).
    Blocks never span rows, so rows are quantized in chunks (for speed) and
    the fields concatenated."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    parts = [QUANTIZE[fmt](W[i:i + rows_per_chunk]) for i in range(0, max(N, 1), rows_per_chunk)]
    fields = {k: np.concatenate([p[k] for p in parts], axis=0) for k in parts[0]}
    return pack(fmt, fields, N, K)


# ----------------------------------------------------------- unpacking -----
# Written from the layout description, independently of the packers above.

def _nibble(plane, N, K):
    b = plane.reshape(N, K // 2)
    out = np.empty((N, K), dtype=np.int64)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def _f16(plane, shape):
    return plane.view("<f2").astype(np.float64).reshape(shape)


def unpack(fmt, buf, N, K):
    """Packed bytes -> integer / fp16 fields as float64 / int64 arrays, one
    entry per element where the field is per element."""
    p = _planes(fmt, buf, N, K)
    nb = K // BLOCK[fmt]
    if fmt == "q8_0":
        return {"q": p[0].view(np.int8).astype(np.int64).reshape(N, K),
                "d": _f16(p[1], (N, nb))}
    if fmt == "q4_0":
        return {"q": _nibble(p[0], N, K), "d": _f16(p[1], (N, nb))}
    if fmt == "mxfp4":
        return {"q": _nibble(p[0], N, K),
                "e": p[1].astype(np.int64).reshape(N, nb)}
    if fmt == "q4_k":
        meta = p[1].reshape(N, nb, 16)
        d = meta[..., 0:2].copy().view("<f2").astype(np.float64)[..., 0]
        dmin = meta[..., 2:4].copy().view("<f2").astype(np.float64)[..., 0]
        # the 96-bit field as integers: bit b of the field is bit b%8 of byte
        # 4 + b//8; field(pos) = the 6 bits starting at pos
        lo = meta[..., 4:12].copy().view("<u8")[..., 0].astype(np.uint64)
        hi = meta[..., 12:16].copy().view("<u4")[..., 0].astype(np.uint64)

        def field(pos):
            if pos + 6 <= 64:
                v = lo >> np.uint64(pos)
            elif pos >= 64:
                v = hi >> np.uint64(pos - 64)
            else:
                v = (lo >> np.uint64(pos)) | (hi << np.uint64(64 - pos))
            return (v & np.uint64(63)).astype(np.int64)

        sc = np.stack([field(6 * j) for j in range(8)], -1)
        m = np.stack([field(48 + 6 * j) for j in range(8)], -1)
        return {"q": _nibble(p[0], N, K), "d": d, "dmin": dmin,
                "sc": sc.astype(np.int64), "m": m.astype(np.int64)}
    if fmt == "t5":
        grp = p[0].reshape(N, nb, T5_GROUP_BYTES)
        code = grp[..., :26].astype(np.int64)
        digits = np.empty((N, nb, 26, 5), dtype=np.int64)
        for r in range(5):
            digits[..., r] = code % 3
            code = code // 3
        t = digits.reshape(N, nb, 130)[..., :128] - 1
        return {"t": t.reshape(N, K), "d": grp[..., 26:28].copy().view("<f2")[..., 0].astype(np.float64)}
    if fmt == "q6_k":
        lo = _nibble(p[0], N, K)
        qh = p[1].reshape(N, K // 4).astype(np.int64)
        hi = np.empty((N, K), dtype=np.int64)
        for r in range(4):
            hi[:, r::4] = (qh >> (2 * r)) & 3
        return {"q": lo | (hi << 4),
                "sc": p[2].view(np.int8).astype(np.int64).reshape(N, nb, 16),
                "d": _f16(p[3], (N, nb))}
    raise ValueError(fmt)


def e2m1_value(code):
    code = np.asarray(code, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDE, dtype=np.float64)[code & 7]
    return np.where(code & 8, -mag, mag)


def dequantize(fmt, buf, N, K):
    """Exact float64 value of every element.  Every value is exact in float64
    (at most ~50 significant bits are involved), so this is the format's value
    with no rounding at all."""
    f = unpack(fmt, buf, N, K)
    B = BLOCK[fmt]
    per_block = lambda a: np.repeat(a.reshape(N, -1), B, axis=1)
    if fmt == "q8_0":
        return per_block(f["d"]) * f["q"]
    if fmt == "q4_0":
        return per_block(f["d"]) * (f["q"] - 8)
    if fmt == "mxfp4":
        e = per_block(f["e"])
        scale = np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))
        return scale * e2m1_value(f["q"])
    if fmt == "q4_k":
        d = per_block(f["d"])
        dmin = per_block(f["dmin"])
        sc = np.repeat(f["sc"].reshape(N, -1), 32, axis=1)
        m = np.repeat(f["m"].reshape(N, -1), 32, axis=1)
        return d * sc * f["q"] - dmin * m
    if fmt == "q6_k":
        d = per_block(f["d"])
        sc = np.repeat(f["sc"].reshape(N, -1), 16, axis=1)
        return d * sc * (f["q"] - 32)
    if fmt == "t5":
        return per_block(f["d"]) * f["t"]
    raise ValueError(fmt)


def dequantize_f32(fmt, buf, N, K):
    """The fp32 value a decoder must produce: the exact value rounded to
    nearest-even float32 (bit-exact parity target for device dequant)."""
    return dequantize(fmt, buf, N, K).astype(np.float32)
