"""GPU: the whole sequence lifecycle under the continuous-batching scheduler.

Requests of assorted prompt and output lengths go through a multi-layer cache
whose pool is too small to hold them all at once: chunked prefill, one row per
decoding request, finished requests freed, the newest running request
preempted and later recomputed.  Every iteration appends the planned rows
(each request's K/V and queries are fixed per token, so a recomputed request
writes the same rows), then runs the attention of every new token on every
layer.  A mirrored oracle store replays the same allocations, frees and
writes; the pools are compared bit-exactly with it, and every output of every
iteration is checked against the oracle's causal attention on its stored
values (|gpu - ref| <= 2e-3 + 1e-2 |ref|).
"""
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import check_close, extend_poisoned, read_pools, to_bits, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_scheduled_lifecycle_multi_layer(kv):
    import math

    import paged_kv_cache_split_amd as kvc
    from oracle.attention import extend_attention
    from oracle.kvstore import KVStoreModel
    from workloads import make_request_values

    L, Hq, Hkv, D, nblocks = 2, 8, 2, 64, 48
    q_dt = "bf16"
    in_dt = "bf16"
    scale = float(np.float32(1.0 / math.sqrt(D)))
    rng = np.random.default_rng(5)
    free_order = rng.permutation(nblocks).astype(np.int32)
    cache = kvc.KVCache(L, Hkv, D, nblocks, kv, device="cuda", free_order=free_order)
    st = KVStoreModel(L, nblocks, Hkv, D, 16, kv, free_order=free_order, in_dtype=in_dt)
    sched = kvc.Scheduler(cache, max_batch=5, chunk_tokens=48, max_tokens=120)
    reqs = {}
    for r in range(12):
        P, M = int(rng.integers(1, 260)), int(rng.integers(1, 40))
        reqs[r] = make_request_values(31, r, L, P + M, Hq, Hkv, D, q_dt, in_dt, "cpu")
        reqs[r]["P"], reqs[r]["M"] = P, M
        sched.submit(r, P, M)
    _say(f"[lifecycle] {kv}: 12 requests, pool {nblocks} blocks of 16")
    checked = 0
    for it in range(400):
        plan = sched.plan()
        for r in plan["preempted"]:
            assert st.free_seq(r) == 0
        ids, n_new, start = plan["ids"], plan["n_new"], plan["start"]
        if not ids:
            assert sched.stats()["finished"] == len(reqs)
            break
        for r, s0 in zip(ids, start):
            if s0 == 0:
                assert st.allocate(r, 0) == 0
        k_rows = torch.cat([reqs[r]["k"][:, s0:s0 + n] for r, s0, n in zip(ids, start, n_new)], dim=1).contiguous()
        v_rows = torch.cat([reqs[r]["v"][:, s0:s0 + n] for r, s0, n in zip(ids, start, n_new)], dim=1).contiguous()
        q_rows = torch.cat([reqs[r]["q"][s0:s0 + n] for r, s0, n in zip(ids, start, n_new)]).contiguous()
        cache.append(ids, k_rows.cuda(), v_rows.cuda(), n_new=n_new)
        assert st.append(ids, n_new, to_bits(k_rows, in_dt), to_bits(v_rows, in_dt))[0] == 0
        bt, cl = cache.export_tables(ids)
        qs = torch.tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32), device="cuda")
        qd = q_rows.cuda()
        outs = [extend_poisoned(cache, qd, qs, max(n_new), bt, cl, int(cl.max().item()), scale, layer=layer)
                for layer in range(L)]
        torch.cuda.synchronize()
        for layer in range(L):
            got = to_f64(outs[layer])
            q64 = to_f64(q_rows)
            row = 0
            for r, n in zip(ids, n_new):
                k, v = st.gather(r, layer)
                ref = extend_attention(q64[row:row + n], k, v, scale)
                check_close(got[row:row + n], ref, 2e-3, 1e-2, f"iteration {it} layer {layer} request {r}")
                row += n
                checked += n
        if it % 4 == 0:
            pools = read_pools(cache)
            assert np.array_equal(pools["k"], st.k) and np.array_equal(pools["v"], st.v), f"pools at iteration {it}"
        for r in sched.commit():
            assert st.free_seq(r) == 0
    else:
        raise AssertionError("the requests did not finish")
    stats = sched.stats()
    _say(f"  {stats['iterations']} iterations, {stats['preemptions']} preemptions, {checked} outputs checked")
    assert stats["preemptions"] >= 1, "the pool was meant to force a preemption"
    assert cache.stats()["free_blocks"] == nblocks
