"""Pins for the oracle's quantised append composition (CPU only).

``oracle.kvstore.KVStoreModel.append`` cuts a write into runs of rows that
land in one block and applies the one-byte scale rule to each run, re-encoding
held codes when a run grows the block's scale.  These tests run that
composition on the hand-worked scenario of ``quant_literals`` (a 20-row write
split over two blocks, scale growth with held codes re-encoded, an all-zero
run, E4M3 and int8 ties) and compare every code and scale with literals worked
out by hand from the rule's text -- not with ``fp8_policy`` or ``int8_policy``,
which these tests never call.  A planted mistake (held codes not re-encoded
when the scale grows) must fail the same comparison.
"""
import numpy as np
import pytest

import quant_literals as QL
from oracle import kvstore


def _bf16_bits(rows):
    """float rows (exact in bf16) -> [1, T, 1, D] uint16 bf16 bit patterns."""
    f = np.asarray(rows, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "input not exact in bf16"
    return (u >> 16).astype(np.uint16).reshape(1, len(rows), 1, QL.HEAD_DIM)


def _run(case):
    st = kvstore.KVStoreModel(1, QL.NUM_BLOCKS, 1, QL.HEAD_DIM, 16, case["dtype"], free_order=QL.FREE_ORDER,
                              in_dtype="bf16")
    assert st.allocate(0, 0) == 0
    scales = []
    for step in range(3):
        k, v = QL.step_rows(case, step)
        status, slots, cow = st.append([0], [QL.STEP_ROWS[step]], _bf16_bits(k), _bf16_bits(v))
        assert status == 0 and cow == []
        scales.append((st.k_scale[:, 0, 0].copy(), st.v_scale[:, 0, 0].copy()))
    return st, scales


def _check(st, scales, case):
    assert st.tables.tables[0] == [0, 1] and st.tables.lens[0] == 32
    for (blk, pool), per_step in case["scales"].items():
        for step, want in enumerate(per_step):
            got = scales[step][0 if pool == "k" else 1][blk]
            if want is None:
                assert got == 0.0
            else:
                assert got == np.float32(want), f"{case['dtype']} block {blk} {pool} scale after step {step + 1}"
    for (blk, pool), rows in case["blocks"].items():
        codes = (st.k if pool == "k" else st.v)[blk, 0, 0]          # [16 slots, D]
        want = np.array(rows, dtype=np.uint8)
        assert np.array_equal(codes[:, :2], want), (
            f"{case['dtype']} block {blk} {pool}: got\n{codes[:, :2].tolist()}\nwant\n{want.tolist()}")
        assert not codes[:, 2:].any(), "zero dims must hold the zero code"
    for blk in (2, 3):
        assert not st.k[blk].any() and not st.v[blk].any()


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_quantised_append_matches_hand_worked_codes(dtype):
    case = QL.CASES[dtype]
    st, scales = _run(case)
    _check(st, scales, case)


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_dequantised_values_are_code_times_scale(dtype):
    # gather() returns dec(code) * scale: spot values from the hand-worked table
    case = QL.CASES[dtype]
    st, _ = _run(case)
    k, v = st.gather(0)
    if dtype == "fp8":
        assert k[0, 0, :2].tolist() == [448.0, -1.0]        # 0x76 = 224 at scale 2; 0xB0 = -0.5 at 2
        assert k[16, 0, :2].tolist() == [28.0, -28.0]       # 0x7E = 448 at 1/16
        assert k[18, 0, :2].tolist() == [1.0, -1.0]         # 1.0625 stored as 16/16 (tie to even)
        assert k[19, 0, :2].tolist() == [1.25, -1.25]       # 1.1875 stored as 20/16
        assert v[30, 0, :2].tolist() == [7.0, 0.0]          # block 1 V after growth 0 -> 1/64
    else:
        assert k[0, 0, :2].tolist() == [128.0, 0.0]         # 127 halved to 64 (tie to even) at scale 2
        assert k[17, 0, :2].tolist() == [0.0, 0.0]          # 0.5 / 16 ties to 0
        assert v[9, 0, :2].tolist() == [2.5, -1.0]          # 10 * 0.25, -4 * 0.25
        assert v[30, 0, :2].tolist() == [63.5, -1.0]        # 127 * 0.5, -2 * 0.5


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_planted_missing_reencode_fails_the_literals(dtype, monkeypatch):
    # a rule that keeps held codes when the scale grows must not pass
    policy = kvstore.QUANTISED[dtype]
    real = policy.write_rows

    def no_reencode(held, scale_old, new_values):
        _, new_codes, s_new = real(held, scale_old, new_values)
        return np.asarray(held, dtype=np.uint8), new_codes, s_new

    monkeypatch.setattr(policy, "write_rows", no_reencode)
    case = QL.CASES[dtype]
    st, scales = _run(case)
    with pytest.raises(AssertionError):
        _check(st, scales, case)
