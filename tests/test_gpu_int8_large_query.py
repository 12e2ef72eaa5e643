"""int8 caches with query values beyond f16's comfortable range (needs a GPU).

The decode walk and the row-split several-token kernel take int8 scores on the
f16 matrix cores, converting each segment's query to f16; when some |q| of a
wave reaches 2^15 the query is scaled by 2^-e first and 2^e goes into the score
scale.  Queries scaled by 4e4 (|q| up to ~2e5, e = 3..4) and a batch where only
one sequence's query is that large (the small ones scaled down with it) must
still match the fp64 oracle at |gpu - ref| <= 2e-3 + 1e-2 |ref|, in the decode
(default launch and a work-item sweep) and in the several-token row split.
"""
import sys

import pytest
import torch

from conftest import gpu_available
from harness import (check_close, extend_poisoned, gpu_decode_again, gpu_setup, gpu_step, oracle_decode, oracle_extend,
                     oracle_run, query_start, to_f64)
from workloads import custom_workload, make_values, shape_scores

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)
LENS = [900, 40, 333, 17, 1200]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("only_one", [False, True])
def test_decode_large_queries(only_one):
    wl = custom_workload(len(LENS), 16, 4, 128, "int8", LENS, seed=71, name="int8 large q")
    _say(f"[int8 large q] decode only_one={only_one}")
    values = make_values(wl, "cpu")
    if only_one:
        values["q"][2] = (values["q"][2].float() * 4e4).to(values["q"].dtype)
    else:
        values = shape_scores(wl, values, "qscale", 4e4)
    assert float(values["q"].float().abs().max()) >= 2.0 ** 15
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    check_close(to_f64(out), ref, *TOL, f"int8 large q only_one={only_one}")
    for wi in (1, 5, 33):
        o = gpu_decode_again(cache, wl, values, bt, cl, kernel=2, work_items=wi)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"int8 large q only_one={only_one} work_items={wi}")


def test_extend_large_queries():
    qls = [3, 1, 5, 2, 4]
    wl = custom_workload(len(LENS), 16, 4, 128, "int8", LENS, seed=72, name="int8 large q extend", query_lens=qls)
    _say("[int8 large q] extend")
    values = shape_scores(wl, make_values(wl, "cpu"), "qscale", 4e4)
    assert float(values["q"].float().abs().max()) >= 2.0 ** 15
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    seqs = list(range(wl.batch))
    cache.append(seqs, values["k_new"].cuda().contiguous(), values["v_new"].cuda().contiguous(),
                 n_new=[int(x) for x in wl.q_lens])
    bt, cl = cache.export_tables(seqs)
    qs = torch.from_numpy(query_start(wl)).cuda()
    q = values["q"].cuda().contiguous()
    ref = oracle_extend(st, wl, values)
    for wi, tpw in ((0, 0), (3, 1), (7, 3)):
        o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, kernel=2,
                            work_items=wi, tiles_per_wave=tpw)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"int8 large q extend work_items={wi} tiles/wave={tpw}")
