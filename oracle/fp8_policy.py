"""Scale rule for fp8 (E4M3) KV storage, one fp32 scale per (layer, block, KV head).

TEST INFRASTRUCTURE ONLY (see the package docstring).

PARITY UNPINNED BY THE PAGES.  They say FP8/E4M3 KV halves storage and that
its error needs calibration ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §四/§五;
"苦猿的大模型日记 · Day45" PART 02) but give no scale rule.  The rule adopted
(the plainest one that never saturates the largest element and keeps every
block usable while it fills token by token):

For each write of ``c`` new rows into one (block, KV head) that already holds
``n0`` valid rows with scale ``s``:

1. ``s_old = s`` if n0 > 0 else 0 (a fresh block starts with scale 0);
2. ``s_new = max(s_old, amax / 448)`` where amax is the largest magnitude of
   the new rows, all in float32 (IEEE division);
3. if ``s_new > s_old`` and n0 > 0, every held code is re-encoded as
   ``enc((dec(code) * s_old) / s_new)`` (float32 multiply, then float32 divide);
4. each new value x is stored as ``enc(x / s_new)``; if s_new == 0 every new
   value is zero and is stored as ``enc(x)`` (the signed zero code).

The rule is a reading; this code's rendering of it (with the store model's
split of a write into per-block runs) is pinned by codes and scales worked out
by hand from the four steps above (tests/quant_literals.py).

``enc`` is E4M3FN round-to-nearest-even with saturation (``oracle.e4m3``).
The dequantised value of a stored code is ``dec(code) * scale``.  The float32
steps are written with NumPy float32 scalars so they round exactly as the
device's IEEE float32 arithmetic does.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

F448 = np.float32(448.0)


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
    s_new = max(s_old, np.float32(amax / F448))
    s_new = np.float32(s_new)
    if s_new > s_old and n0 > 0:
        dec = e4m3.decode_array(held).astype(np.float32)
        held = e4m3.encode_array(((dec * s_old).astype(np.float32) / s_new).astype(np.float32))
    if s_new > 0:
        new_codes = e4m3.encode_array((new / s_new).astype(np.float32))
    else:
        new_codes = e4m3.encode_array(new)
    return held, new_codes, s_new


def dequantize(codes, scale):
    """Real values represented by ``codes`` stored with ``scale`` (fp64)."""
    return e4m3.decode_array(codes) * np.float64(np.float32(scale))
