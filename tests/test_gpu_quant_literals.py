"""The one-byte caches' append kernel against hand-worked codes (needs a GPU).

The scenario of ``quant_literals`` (a 20-row write split over two blocks,
scale growth with held codes re-encoded, an all-zero run, planted E4M3 and
int8 ties) written through libkvc's C ABI; every stored code and scale must
equal the literals worked out by hand from the rule's text, bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import quant_literals as QL
from conftest import gpu_available
from harness import read_pools

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_append_kernel_matches_hand_worked_codes(dtype):
    from paged_kv_cache_split_amd import KVCache
    print(f"[quant literals] {dtype}", file=sys.stderr, flush=True)
    case = QL.CASES[dtype]
    cache = KVCache(1, 1, QL.HEAD_DIM, QL.NUM_BLOCKS, dtype, device="cuda", free_order=QL.FREE_ORDER)
    cache.add_seq(0, 0)
    for step in range(3):
        k, v = QL.step_rows(case, step)
        T = QL.STEP_ROWS[step]
        kt = torch.tensor(k, dtype=torch.float32).to(torch.bfloat16).reshape(1, T, 1, QL.HEAD_DIM).cuda()
        vt = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).reshape(1, T, 1, QL.HEAD_DIM).cuda()
        cache.append([0], kt, vt, n_new=[T])
        torch.cuda.synchronize()
        pools = read_pools(cache)
        for (blk, pool), per_step in case["scales"].items():
            want = 0.0 if per_step[step] is None else per_step[step]
            got = pools["k_scale" if pool == "k" else "v_scale"][blk, 0, 0]
            assert np.float32(got).view(np.uint32) == np.float32(want).view(np.uint32), \
                f"{dtype} block {blk} {pool} scale after step {step + 1}: {got} != {want}"
    assert cache.get_table(0) == ([0, 1], 32)
    for (blk, pool), rows in case["blocks"].items():
        codes = pools[pool][blk, 0, 0]                                  # [16 slots, D]
        want = np.array(rows, dtype=np.uint8)
        assert np.array_equal(codes[:, :2], want), (
            f"{dtype} block {blk} {pool}: got\n{codes[:, :2].tolist()}\nwant\n{want.tolist()}")
        assert not codes[:, 2:].any(), "zero dims must hold the zero code"
