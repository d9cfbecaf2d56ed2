"""Pure-Python brute force for tiny cases (cross-checks the vectorised oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Element by element from the packed bytes with Python integers and floats (all
exact or float64), no NumPy arithmetic: a second reading of the same format
and layer definitions, kept deliberately naive.
"""
import itertools
import math
import struct

from . import formats as fm


def _f16(b0, b1):
    return struct.unpack("<e", bytes([b0, b1]))[0]


def element(fmt, buf, N, K, n, k):
    """Exact value of W[n, k] read straight from the packed bytes."""
    buf = bytes(buf)
    offs, _ = fm.plane_offsets(fmt, N, K)
    B = fm.BLOCK[fmt]
    nb = K // B
    blk = n * nb + k // B

    def nib(plane):
        byte = buf[offs[plane] + (n * K + k) // 2]
        return (byte >> 4) if k % 2 else (byte & 15)

    if fmt == "q8_0":
        q = buf[offs[0] + n * K + k]
        q = q - 256 if q > 127 else q
        return _f16(buf[offs[1] + 2 * blk], buf[offs[1] + 2 * blk + 1]) * q
    if fmt == "q4_0":
        return _f16(buf[offs[1] + 2 * blk], buf[offs[1] + 2 * blk + 1]) * (nib(0) - 8)
    if fmt == "mxfp4":
        e = buf[offs[1] + blk]
        c = nib(0)
        mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][c & 7]
        v = -mag if c & 8 else mag
        return float("nan") if e == 255 else math.ldexp(v, e - 127)
    if fmt == "q4_k":
        meta = buf[offs[1] + 16 * blk: offs[1] + 16 * blk + 16]
        d, dmin = _f16(meta[0], meta[1]), _f16(meta[2], meta[3])
        field = int.from_bytes(meta[4:16], "little")
        j = (k % 256) // 32
        sc = (field >> (6 * j)) & 63
        m = (field >> (48 + 6 * j)) & 63
        return d * sc * nib(0) - dmin * m
    if fmt == "q6_k":
        lo = nib(0)
        hbyte = buf[offs[1] + (n * K + k) // 4]
        hi = (hbyte >> (2 * (k % 4))) & 3
        j = (k % 256) // 16
        sc = buf[offs[2] + 16 * blk + j]
        sc = sc - 256 if sc > 127 else sc
        d = _f16(buf[offs[3] + 2 * blk], buf[offs[3] + 2 * blk + 1])
        return d * sc * ((lo | (hi << 4)) - 32)
    if fmt == "t5":
        g = offs[0] + fm.T5_GROUP_BYTES * blk
        i = k % 128
        code = buf[g + i // 5]
        digit = (code // 3 ** (i % 5)) % 3
        return _f16(buf[g + 26], buf[g + 27]) * (digit - 1)
    raise ValueError(fmt)


def gemv(fmt, buf, N, K, x):
    """[R][N] nested lists, summed left to right in float64."""
    return [[sum(element(fmt, buf, N, K, n, k) * float(xr[k]) for k in range(K))
             for n in range(N)] for xr in x]


def topk_by_enumeration(logits_row, k):
    """The k-subset with the largest logit sum; among equal sums the
    lexicographically smallest sorted id tuple (= ties to lower ids).
    Returned in descending-logit order, ties lower id first."""
    E = len(logits_row)
    best, best_sum = None, None
    for sub in itertools.combinations(range(E), k):
        s = sum(logits_row[i] for i in sub)
        if best is None or s > best_sum:
            best, best_sum = sub, s
    return sorted(best, key=lambda i: (-logits_row[i], i))


def expert_ffn(expert, H, F, xrow):
    fgu, gbuf, ubuf, fd, dbuf = expert
    g = gemv(fgu, gbuf, F, H, [xrow])[0]
    u = gemv(fgu, ubuf, F, H, [xrow])[0]
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return gemv(fd, dbuf, H, F, [h])[0]


def moe_layer(x, ids, p, get_expert, H, F, E):
    out = []
    for t, xrow in enumerate(x):
        y = [0.0] * H
        for i, e in enumerate(ids[t]):
            if 0 <= e < E:
                o = expert_ffn(get_expert(int(e)), H, F, [float(v) for v in xrow])
                y = [a + float(p[t][i]) * b for a, b in zip(y, o)]
        out.append(y)
    return out
