"""Scale rule for INT8 KV storage, one fp32 scale per (layer, block, KV head).

TEST INFRASTRUCTURE ONLY (see the package docstring).

PARITY UNPINNED BY THE PAGES.  They list INT8 beside FP8 and INT4 as KV
quantisation options ("LLM推理优化实战…" §6.1, the deployed engine supports FP8/INT4/INT8;
"LLM推理优化核心技术…" §1.2, one byte per element in the cache-size formula and
an INT8 column in its table) but fix no scheme.  The reading adopted mirrors
the fp8 rule (``fp8_policy``) with a symmetric integer code:

For each write of ``c`` new rows into one (block, KV head) that already holds
``n0`` valid rows with scale ``s``:

1. ``s_old = s`` if n0 > 0 else 0 (a fresh block starts with scale 0);
2. ``s_new = max(s_old, amax / 127)`` where amax is the largest magnitude of
   the new rows, all in float32 (IEEE division);
3. if ``s_new > s_old`` and n0 > 0, every held code c is re-encoded as
   ``enc((c * s_old) / s_new)`` (float32 multiply, then float32 divide);
4. each new value x is stored as ``enc(x / s_new)``; if s_new == 0 every new
   value is zero and is stored as code 0.

``enc`` rounds to the nearest integer, ties to even, and clamps to
[-127, 127]; the code is stored as a two's-complement byte.  The value of a
stored code is ``c * scale``.  The float32 steps use NumPy float32 scalars so
they round exactly as the device's IEEE float32 arithmetic does.

The rule is a reading; this code's rendering of it (with the store model's
split of a write into per-block runs) is pinned by codes and scales worked out
by hand from the steps above (tests/quant_literals.py).
"""
from __future__ import annotations

import numpy as np

F127 = np.float32(127.0)


def encode_array(x):
    """float32 values -> int8 codes (round half to even, clamp to +-127), as uint8 bytes."""
    q = np.rint(np.asarray(x, dtype=np.float32))
    return np.clip(q, -127, 127).astype(np.int8).view(np.uint8)


def decode_array(codes):
    """uint8 bytes holding int8 codes -> their integer values as fp64."""
    return np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


def write_rows(held_codes, scale_old, new_values):
    """Apply one write to a single (block, KV head).

    held_codes: uint8 [n0, D] codes already valid in the block (n0 may be 0)
    scale_old: the block's stored fp32 scale (ignored when n0 == 0)
    new_values: [c, D] new rows, exactly representable in float32
    returns (held_codes_after [n0, D] uint8, new_codes [c, D] uint8, scale_new float32)
    """
    held = np.asarray(held_codes, dtype=np.uint8)
    new = np.asarray(new_values, dtype=np.float32)
    n0 = held.shape[0]
    s_old = np.float32(scale_old) if n0 > 0 else np.float32(0.0)
    amax = np.float32(np.max(np.abs(new))) if new.size else np.float32(0.0)
    s_new = np.float32(max(s_old, np.float32(amax / F127)))
    if s_new > s_old and n0 > 0:
        dec = decode_array(held).astype(np.float32)
        held = encode_array(((dec * s_old).astype(np.float32) / s_new).astype(np.float32))
    if s_new > 0:
        new_codes = encode_array((new / s_new).astype(np.float32))
    else:
        new_codes = np.zeros(new.shape, dtype=np.uint8)
    return held, new_codes, s_new


def dequantize(codes, scale):
    """Real values represented by ``codes`` stored with ``scale`` (fp64)."""
    return decode_array(codes) * np.float64(np.float32(scale))
