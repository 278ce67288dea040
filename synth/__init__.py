"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no convolution arithmetic. It only turns (seed, element index)
into a float, so the fp64 oracle and the HIP path can be fed the same tensors.

Generator: the i-th output (i = 0, 1, ...) of the SplitMix64 stream started at
``seed`` (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number Generators",
OOPSLA 2014; mixing constants of the public-domain ``splitmix64.c``):

    z   = seed + (i + 1) * 0x9E3779B97F4A7C15          (mod 2**64)
    z   = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
    z   = (z ^ (z >> 27)) * 0x94D049BB133111EB
    out = z ^ (z >> 31)

Kinds of element drawn from ``m = out >> 40`` (24 random bits):

* ``uniform01``  u = m * 2**-24, exactly representable in fp32, in [0, 1).
* ``symmetric``  fp32((2u - 1) * b) with b = fp32(1 / sqrt(fan_in)); ``2u - 1``
  is exact in fp32, so only the final product rounds (round to nearest even).
* ``int_range``  lo + ((m * span) >> 24), an integer in [lo, lo + span) stored
  as fp32. Sums of such products stay exact in fp32 while below 2**24, which
  lets a GPU result be compared bit for bit.

The same definition is implemented on the device by the library's fill entry
point, so inputs too large to build on the host (the 8.6 GB Conv1d input) are
generated in place and the host regenerates only the slice it checks.
"""
import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

KIND_UNIFORM01 = 0
KIND_SYMMETRIC = 1
KIND_INT = 2

_CHUNK = 1 << 22


def _bits24(seed, start, count):
    """24 random bits of outputs start .. start+count-1 as uint64."""
    i = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (i + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
        z = z ^ (z >> np.uint64(31))
    return z >> np.uint64(40)


def symmetric_bound(fan_in):
    """fp32(1/sqrt(fan_in)), the half-width of the weight distribution."""
    return float(np.float32(1.0 / math.sqrt(fan_in)))


def fill(kind, seed, count, start=0, bound=1.0, lo=0, span=1):
    """Return ``count`` fp32 values of element indices start .. start+count-1."""
    out = np.empty(count, dtype=np.float32)
    b32 = np.float32(bound)
    for c0 in range(0, count, _CHUNK):
        n = min(_CHUNK, count - c0)
        m = _bits24(seed, start + c0, n)
        if kind == KIND_UNIFORM01:
            out[c0:c0 + n] = m.astype(np.float32) * np.float32(2.0 ** -24)
        elif kind == KIND_SYMMETRIC:
            u = m.astype(np.float32) * np.float32(2.0 ** -24)
            out[c0:c0 + n] = (np.float32(2.0) * u - np.float32(1.0)) * b32
        elif kind == KIND_INT:
            v = (m * np.uint64(span)) >> np.uint64(24)
            out[c0:c0 + n] = (v.astype(np.int64) + lo).astype(np.float32)
        else:
            raise ValueError(f"unknown kind {kind}")
    return out


def uniform01(seed, shape, start=0):
    n = int(np.prod(shape)) if len(shape) else 1
    return fill(KIND_UNIFORM01, seed, n, start=start).reshape(shape)


def symmetric(seed, shape, fan_in, start=0):
    n = int(np.prod(shape)) if len(shape) else 1
    return fill(KIND_SYMMETRIC, seed, n, start=start, bound=symmetric_bound(fan_in)).reshape(shape)


def int_range(seed, shape, lo, hi, start=0):
    """Integers in [lo, hi] inclusive, as fp32."""
    n = int(np.prod(shape)) if len(shape) else 1
    return fill(KIND_INT, seed, n, start=start, lo=lo, span=hi - lo + 1).reshape(shape)


# ---------------------------------------------------------------------------
# The five workloads, with the seeds and distributions used everywhere.
# x ~ U[0,1); w and bias ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)) with
# fan_in = (C_in / groups) * prod(kernel).
# ---------------------------------------------------------------------------
WORKLOADS = {
    "tiny_conv3d": dict(
        nd=3, x=(2, 3, 16, 16, 16), w=(8, 3, 3, 3, 3), bias=True,
        stride=(1, 1, 1), padding=(0, 0, 0), dilation=(1, 1, 1), groups=1,
        seeds=(0xC1A, 0xC1B, 0xC1C), fused=False),
    "general_conv3d": dict(
        nd=3, x=(4, 16, 32, 32, 32), w=(32, 8, 3, 5, 7), bias=True,
        stride=(1, 2, 2), padding=(1, 2, 3), dilation=(1, 1, 2), groups=2,
        seeds=(0xC2A, 0xC2B, 0xC2C), fused=False),
    "conv3d_min_softmax": dict(
        nd=3, x=(128, 3, 24, 32, 32), w=(24, 3, 3, 3, 3), bias=True,
        stride=(1, 1, 1), padding=(0, 0, 0), dilation=(1, 1, 1), groups=1,
        seeds=(0xC3A, 0xC3B, 0xC3C), fused=True),
    "asym_conv3d": dict(
        nd=3, x=(16, 3, 64, 64, 64), w=(64, 3, 3, 5, 7), bias=False,
        stride=(1, 1, 1), padding=(0, 0, 0), dilation=(1, 1, 1), groups=1,
        seeds=(0xC4A, 0xC4B, None), fused=False),
    "long_conv1d": dict(
        nd=1, x=(64, 64, 524280), w=(128, 64, 3), bias=False,
        stride=(3,), padding=(0,), dilation=(4,), groups=1,
        seeds=(0xC5A, 0xC5B, None), fused=False),
}


# Shapes measured beside the five workloads: neighbours of three of them that
# are not among the build-time specialised geometries (a smaller asymmetric
# Conv3d input, a smaller general Conv3d input, the long Conv1d with 96 output
# channels and dilation 2), and the fused op with the minimum over H or W and
# with groups. Same distributions; each reuses its base workload's seeds.
VARIANTS = {
    "asym_conv3d_48": dict(WORKLOADS["asym_conv3d"], x=(16, 3, 48, 48, 48)),
    "general_conv3d_24": dict(WORKLOADS["general_conv3d"], x=(4, 16, 24, 24, 24)),
    "long_conv1d_c96_d2": dict(WORKLOADS["long_conv1d"], w=(96, 64, 3), dilation=(2,)),
    "conv3d_min_softmax_min_h": dict(WORKLOADS["conv3d_min_softmax"], min_dim=3),
    "conv3d_min_softmax_min_w": dict(WORKLOADS["conv3d_min_softmax"], min_dim=4),
    "conv3d_min_softmax_groups3": dict(WORKLOADS["conv3d_min_softmax"], w=(24, 1, 3, 3, 3), groups=3),
}


def config(name):
    """A workload or a variant by name."""
    return WORKLOADS[name] if name in WORKLOADS else VARIANTS[name]


def fan_in(w_shape):
    return int(np.prod(w_shape[1:]))


def make_inputs(name, n_samples=None, sample_start=0, integer=False):
    """Host tensors (numpy fp32) of a workload, optionally a contiguous batch slice.

    ``integer`` switches to the exact-arithmetic distribution: x in {0..3},
    w in {-2..2}, bias in {-4..4}.
    """
    cfg = config(name)
    xs = list(cfg["x"])
    per_sample = int(np.prod(xs[1:]))
    if n_samples is None:
        n_samples = xs[0] - sample_start
    xs_slice = [n_samples] + xs[1:]
    sx, sw, sb = cfg["seeds"]
    if integer:
        x = int_range(sx, xs_slice, 0, 3, start=sample_start * per_sample)
        w = int_range(sw, cfg["w"], -2, 2)
        b = int_range(sb if sb is not None else sw + 1, (cfg["w"][0],), -4, 4) if cfg["bias"] else None
    else:
        x = uniform01(sx, xs_slice, start=sample_start * per_sample)
        fi = fan_in(cfg["w"])
        w = symmetric(sw, cfg["w"], fi)
        b = symmetric(sb, (cfg["w"][0],), fi) if cfg["bias"] else None
    return x, w, b
