"""OCP 8-bit floating point, E4M3 ("FN") variant: decode and encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages only name "FP8/E4M3" KV caches ("大模型推理加速核心KV Cache 复用机制与内存布局
优化" §四; "苦猿的大模型日记 · Day45" PART 02, FP8 KV Cache).  The format used is
the OCP 8-bit floating point specification's E4M3, written from its
definition (no vendor conversion routine):

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 is subnormal: value = (m / 8) * 2^-6;
* otherwise value = 2^(e - 7) * (1 + m / 8);
* no infinities; S.1111.111 is NaN, so the largest finite magnitude is
  S.1111.110 = 448.

Encoding rounds to the nearest representable value, ties to the even
mantissa, and saturates to +-448 (it never produces NaN); the sign of zero is
kept.  It is done by a direct search over the 127 non-negative finite values
so it can be checked by eye.
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0


def decode(code: int) -> float:
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


# Non-negative finite codes 0x00 .. 0x7E in increasing value order.
_POS_CODES = list(range(0x7F))
_POS_VALUES = [decode(c) for c in _POS_CODES]

TABLE = np.array([decode(c) for c in range(256)], dtype=np.float64)


def encode(x: float) -> int:
    """Round a real number to E4M3FN (RNE, saturating)."""
    x = float(x)
    if math.isnan(x):
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a >= MAX_FINITE:
        return sign | 0x7E
    best = 0
    best_err = abs(a - _POS_VALUES[0])
    for c in _POS_CODES[1:]:
        err = abs(a - _POS_VALUES[c])
        if err < best_err or (err == best_err and (c & 1) == 0 and (best & 1) == 1):
            best, best_err = c, err
    return sign | best


def encode_array(x) -> np.ndarray:
    """Vectorised ``encode`` over an array of floats (same result elementwise)."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    vals = np.asarray(_POS_VALUES)
    a = np.abs(flat)
    # nearest by search; ties resolved toward the even code below
    idx = np.searchsorted(vals, a)                     # first value >= a
    idx = np.clip(idx, 1, len(vals) - 1)
    lo, hi = idx - 1, idx
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= MAX_FINITE, 0x7E, pick)
    pick = np.where(a == 0.0, 0, pick)
    sign = np.where(np.signbit(flat), 0x80, 0x00)
    return (pick | sign).astype(np.uint8).reshape(x.shape)


def decode_array(codes) -> np.ndarray:
    return TABLE[np.asarray(codes, dtype=np.uint8)]
