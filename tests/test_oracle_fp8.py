"""Pins for the oracle's E4M3 codec and fp8 scale rule (CPU only).

The codec is pinned to the OCP format table (golden fixture) and to torch's
float8_e4m3fn dtype, an independent implementation of the same format.  The
scale rule has no source on the pages ("parity unpinned" by them); here it is
checked against its own stated invariants, and test_oracle_quant_append.py pins
its rendering to codes and scales worked out by hand.
"""
import json
import math
import os

import numpy as np
import torch

from oracle import e4m3, fp8_policy


def test_codes_match_the_format_table(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_format.json")) as f:
        g = json.load(f)
    for code, val in g["values"].items():
        got = e4m3.decode(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(e4m3.decode(int(code, 16)))
    finite = [abs(e4m3.decode(c)) for c in range(256) if not math.isnan(e4m3.decode(c))]
    assert max(finite) == g["max_finite"]
    assert min(x for x in finite if x > 0) == g["min_subnormal"]


def test_all_256_codes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_encode_round_trips_every_finite_code():
    for c in range(256):
        v = e4m3.decode(c)
        if not math.isnan(v):
            assert e4m3.encode(v) == c, hex(c)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode_array(e4m3.decode_array(codes)), codes)


def test_encode_matches_torch_rne_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.uniform(-2 ** -5, 2 ** -5, 20000).astype(np.float32),     # subnormal range
        # exact midpoints between neighbouring codes (ties go to the even code)
        ((e4m3.TABLE[1:126] + e4m3.TABLE[2:127]) / 2).astype(np.float32),
        np.float32([0.0, -0.0, 448.0, -448.0, 2 ** -10, -(2 ** -10), 3 * 2 ** -11]),
    ])
    ref = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3.encode_array(x)
    assert np.array_equal(ours, ref)
    # the scalar and vector forms agree
    for v in x[::997]:
        assert e4m3.encode(float(v)) == e4m3.encode_array(np.float32(v)).item()


def test_encode_saturates_instead_of_nan():
    for v in (448.0, 449.0, 463.9, 464.0, 465.0, 1e6, math.inf):
        assert e4m3.encode(v) == 0x7E
        assert e4m3.encode(-v) == 0xFE
    assert e4m3.encode_array(np.float32([1e9, -1e9])).tolist() == [0x7E, 0xFE]


# -- scale rule (a reading, unpinned by the pages: invariants here; hand-worked
#    codes and scales in test_oracle_quant_append.py) --------------------------

def test_fresh_block_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    held, codes, s = fp8_policy.write_rows(np.zeros((0, 128), np.uint8), 123.0, x)
    assert held.shape == (0, 128)
    assert s == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
    deq = fp8_policy.dequantize(codes, s)
    # every element within half a step of the E4M3 grid (relative 2^-4, or the
    # subnormal spacing 2^-9 * s near zero)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the largest element is represented without saturating away from it
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert abs(deq[i] - x[i]) <= abs(x[i]) * 2.0 ** -4


def test_scale_is_monotone_and_reencodes_only_on_growth():
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((16, 64)).astype(np.float32)
    held = np.zeros((0, 64), np.uint8)
    s = np.float32(0)
    history, growths = [], []
    for t in range(16):
        new = rows[t:t + 1] * (3.0 if t == 9 else 1.0)
        prev_held, prev_s = held.copy(), s
        held_after, codes, s = fp8_policy.write_rows(held, prev_s, new)
        assert s >= prev_s
        if s == prev_s:
            assert np.array_equal(held_after, prev_held)
        elif t > 0:
            growths.append(t)
        held = np.concatenate([held_after, codes])
        history.append(new[0].astype(np.float64))
    deq = fp8_policy.dequantize(held, s)
    ref = np.array(history)
    # a row written at step t is rounded once, then once more per later growth
    for t in range(16):
        k = 1 + sum(1 for g in growths if g > t)
        bound = ((1 + 2.0 ** -4) ** k - 1) * np.abs(ref[t]) + k * 2.0 ** -10 * float(s)
        assert np.all(np.abs(deq[t] - ref[t]) <= bound * (1 + 1e-6) + 1e-12), t


def test_all_zero_rows_store_zero_codes():
    held, codes, s = fp8_policy.write_rows(np.zeros((0, 8), np.uint8), 0.0, np.zeros((2, 8), np.float32))
    assert s == 0 and np.all(codes == 0)
    neg = -np.zeros((1, 8), np.float32)
    _, codes, _ = fp8_policy.write_rows(np.zeros((0, 8), np.uint8), 0.0, neg)
    assert np.all(codes == 0x80)


# -- int8 scale rule (a reading, unpinned by the pages: invariants here; hand-worked
#    codes and scales in test_oracle_quant_append.py) --------------------------

from oracle import int8_policy  # noqa: E402


def test_int8_codec_is_twos_complement_rounding_half_even():
    x = np.array([0.0, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, 127.4, 200.0, -127.6, -300.0], dtype=np.float32)
    codes = int8_policy.encode_array(x)
    assert codes.dtype == np.uint8
    assert list(int8_policy.decode_array(codes)) == [0, 0, 2, 2, -0.0, -2, 126, 127, 127, -127, -127]
    # every code decodes to its own integer
    allc = np.arange(256, dtype=np.int32).astype(np.uint8)
    assert np.array_equal(int8_policy.decode_array(allc), allc.view(np.int8).astype(np.float64))


def test_int8_rule_invariants():
    rng = np.random.default_rng(17)
    for trial in range(200):
        d = 16
        held_vals = rng.standard_normal((rng.integers(0, 6), d)).astype(np.float32) * rng.choice([0.01, 1, 50])
        held, _, s0 = int8_policy.write_rows(np.zeros((0, d), np.uint8), 0, held_vals)
        new_vals = rng.standard_normal((rng.integers(1, 5), d)).astype(np.float32) * rng.choice([0.01, 1, 300])
        held2, new_codes, s1 = int8_policy.write_rows(held, s0, new_vals)
        assert s1.dtype == np.float32
        if held.shape[0]:
            assert s1 >= s0                                            # a filled block's scale never shrinks
        amax = float(np.max(np.abs(new_vals)))
        assert s1 >= np.float32(amax / np.float32(127))
        # the largest new element is not clipped, and every new value is
        # within half a step of its code
        deq = int8_policy.dequantize(new_codes, s1)
        assert np.all(np.abs(deq - new_vals.astype(np.float64)) <= 0.5 * float(s1) * (1 + 1e-6) + 1e-30)
        # held rows: unchanged when the scale did not move, else within one step
        if held.shape[0]:
            if s1 == s0:
                assert np.array_equal(held2, held)
            else:
                before = int8_policy.dequantize(held, s0)
                after = int8_policy.dequantize(held2, s1)
                assert np.all(np.abs(after - before) <= 0.5 * float(s1) * (1 + 1e-6) + 1e-30)


def test_int8_zero_rows_keep_scale_zero():
    held, new, s = int8_policy.write_rows(np.zeros((0, 8), np.uint8), 0, np.zeros((3, 8), np.float32))
    assert s == 0 and not new.any()
