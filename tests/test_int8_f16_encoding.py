"""The identity behind the int8 cache's f16 scores (CPU only).

The decode walk and the row-split several-token kernel turn an int8 K code c
into the f16 value 1152 + c by flipping the code's sign bit and placing the
byte under 0x64 in a 16-bit lane (v_perm_b32 with the selectors 0x04010400 /
0x04030402 on the flipped dword and 0x64646464), then take 1152 times the
column's f16 query sum back out of each score.  This pins the identity for
every code and both byte pairs of a dword, and that the subtraction returns
the plain dot product exactly when the products and sums are exact.
"""
import numpy as np


def _perm(s0: int, s1: int, sel: int) -> int:
    """v_perm_b32: result byte i = byte sel_i of the 8-byte value {s0, s1}
    (selectors 0-3 pick s1's bytes, 4-7 s0's)."""
    pool = [(s1 >> (8 * k)) & 0xFF for k in range(4)] + [(s0 >> (8 * k)) & 0xFF for k in range(4)]
    out = 0
    for i in range(4):
        out |= pool[(sel >> (8 * i)) & 0xFF] << (8 * i)
    return out


def _f16_pair(word: int):
    return np.array([word & 0xFFFF, word >> 16], dtype=np.uint16).view(np.float16).astype(np.float64)


def test_every_code_becomes_1152_plus_code():
    codes = np.arange(-127, 128)
    for j in range(0, len(codes), 4):
        quad = list(codes[j:j + 4]) + [0] * (4 - len(codes[j:j + 4]))
        w = 0
        for k, c in enumerate(quad):
            w |= (int(c) & 0xFF) << (8 * k)
        x = w ^ 0x80808080
        lo = _f16_pair(_perm(0x64646464, x, 0x04010400))
        hi = _f16_pair(_perm(0x64646464, x, 0x04030402))
        got = np.concatenate([lo, hi])
        assert np.array_equal(got, 1152.0 + np.array(quad, dtype=np.float64)), (quad, got)


def test_bias_comes_back_out_exactly():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128).astype(np.float16).astype(np.float64)   # the f16 query the cores see
    codes = rng.integers(-127, 128, size=(16, 128))
    raw = (1152.0 + codes) @ q                                          # exact in float64
    kb = 1152.0 * q.sum()
    assert np.allclose(raw - kb, codes @ q, rtol=0, atol=1e-9)
