"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no arithmetic of the method (no quantization, dequant,
routing or FFN math): only random draws, the bf16 rounding of generated
activations, and the additive rank prior, all of which are *inputs*.

Every tensor is drawn from its own stream keyed by (seed, tag, index), so a
tensor can be regenerated alone (one expert of a 512-expert bank, say)
without drawing the others.  Two back ends:

* ``normal``        -- NumPy PCG64, float32 N(0, sigma) on the host;
* ``normal_device`` -- torch's Philox generator on a GPU, for banks too large
  to draw on the host (the same key always gives the same values on the same
  device type; it does not reproduce the NumPy stream).
"""
import numpy as np

# stream tags
ROUTER, GATE, UP, DOWN, ACT, SH_GATE, SH_UP, SH_DOWN, DENSE = range(1, 10)


def normal(shape, sigma, seed, tag, index=0):
    """float32 N(0, sigma): standard_normal(float32) * float32(sigma)."""
    rng = np.random.default_rng([int(seed), int(tag), int(index)])
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def _device_seed(seed, tag, index):
    return (int(seed) * 1_000_003 + int(tag) * 7_919 + int(index) * 104_729
            + 0x5EED) % (2 ** 63)


def normal_device(shape, sigma, seed, tag, index=0, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(seed, tag, index))
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return out.mul_(float(np.float32(sigma)))


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  Used to make activations that are exactly bf16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, b | 0x00400000, r)
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def bf16_bits(x_bf16_valued):
    """uint16 storage of float32 values that are exactly bfloat16."""
    b = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    return (b >> 16).astype(np.uint16)


def rank_prior(E, lam):
    """Additive router-logit bias b_e = -lam * ln(e + 1), float32: expert id
    = frequency rank - 1, so more frequent experts have smaller ids."""
    return (-float(lam) * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def random_ids(T, k, E, seed, distinct=True):
    """Routing ids [T, k] int32 drawn uniformly (distinct within a token when
    ``distinct``), for exercising permutation/FFN/combine in isolation."""
    rng = np.random.default_rng([int(seed), 77])
    if distinct:
        return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    return rng.integers(0, E, size=(T, k)).astype(np.int32)


def random_weights(T, k, seed):
    """Positive weights [T, k] float32 summing to ~1 per row."""
    rng = np.random.default_rng([int(seed), 78])
    w = rng.random((T, k)).astype(np.float64) + 0.05
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
