"""The shaped-score inputs reach the lazy-rescale branch, and the oracle's
answer on them (CPU only).

* For each planted profile (workloads.shape_scores) and cache dtype, replaying
  the decode's cut of the rows among waves on the stored values finds blocks
  whose scores move a finite reference max by more than 8 log2 units -- the
  premise the GPU rescale tests rely on.
* A key 32 log2 units above every other one takes all but 2^-32 of the weight:
  the oracle's decode output is that row's value (closed form) for every head
  of the group.
"""
import numpy as np
import pytest

from harness import oracle_decode, oracle_run, to_f64
from score_walk import decode_chunks, decode_grows, extend_grows, log2_scores
from workloads import custom_workload, make_values, shape_scores

LENS = [900, 130, 47, 400]


@pytest.mark.parametrize("pattern", [("ramp", 10.0), ("sink", 12.0), ("sink", 32.0), ("qscale", 30.0)])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_shaped_inputs_move_a_finite_reference(kv, pattern):
    wl = custom_workload(len(LENS), 8, 2, 64, kv, LENS, seed=9, name="premise")
    values = shape_scores(wl, make_values(wl, "cpu"), *pattern)
    st = oracle_run(wl, values)
    q64 = to_f64(values["q"])
    assert decode_grows(st, wl, q64, 1) > 0
    assert decode_grows(st, wl, q64, 7) > 0


def test_shaped_inputs_reach_the_branch_with_several_tokens():
    wl = custom_workload(3, 8, 2, 64, "bf16", [300, 64, 100], seed=10, name="premise extend",
                         query_lens=[5, 40, 70])
    values = shape_scores(wl, make_values(wl, "cpu"), "ramp", 10.0)
    st = oracle_run(wl, values)
    q64 = to_f64(values["q"])
    assert extend_grows(st, wl, q64, 16) > 0 and extend_grows(st, wl, q64, 32) > 0


def test_unshaped_inputs_rarely_reach_the_branch():
    # the reason for the shaped inputs: N(0, 1) draws barely move the reference
    # after the first block (scores ~ N(0, 1.44^2) in log2 units at D = 64)
    wl = custom_workload(len(LENS), 8, 2, 64, "bf16", LENS, seed=9, name="plain")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    assert decode_grows(st, wl, to_f64(values["q"]), 1) == 0


def test_dominant_key_gives_its_value_row():
    wl = custom_workload(len(LENS), 8, 2, 64, "bf16", LENS, seed=9, name="sink")
    values = shape_scores(wl, make_values(wl, "cpu"), "sink", 32.0)
    st = oracle_run(wl, values)
    out = oracle_decode(st, wl, values)
    q64 = to_f64(values["q"])
    G = wl.num_heads // wl.num_kv_heads
    for b in range(wl.batch):
        n = int(wl.attend_lens[b])
        p_s = min((int(0.7 * n) // 16) * 16 + 7, n - 1)
        _, v = st.gather(b)
        s = log2_scores(st, wl, q64, [b], b)[0]             # [Hq, n]
        for h in range(wl.num_heads):
            # every other row's weight relative to the sink's is 2^(s_t - s_sink)
            rest = np.delete(s[h], p_s) - s[h, p_s]
            assert rest.max() < -20
            bound = np.exp2(rest).sum() * 2 * np.abs(v).max()
            assert np.abs(out[b, h] - v[p_s, h // G]).max() <= bound


def test_decode_chunks_cover_every_block_once():
    lens = [17, 1, 300, 16, 33]
    for W in (1, 2, 5, 13, 40, 1000):
        chunks = decode_chunks(lens, W)
        seen = {}
        for b, j0, j1 in chunks:
            for j in range(j0, j1):
                assert (b, j) not in seen
                seen[(b, j)] = True
        assert len(seen) == sum((n + 15) // 16 for n in lens)
