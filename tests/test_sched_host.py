"""The continuous-batching scheduler (kvc_sched_*) on a bookkeeping-only cache.

Expected plans in the first two tests are worked out by hand from the rules
stated in include/kvc.h (every decoding request gets one row, prefill chunks
follow within the row budget, the newest running request is preempted when
the iteration's blocks do not fit, waiting requests are admitted in order).
The stress test checks invariants over random workloads: the plan always fits
the free list (the reservation never fails), budgets hold, admission is in
submission order, every request emits exactly its token count, and no block
leaks.
"""
import random

import numpy as np
import pytest

import paged_kv_cache_split_amd as kvc


def _cache(num_blocks, block_size=4):
    return kvc.KVCache(1, 2, 64, num_blocks, "bf16", block_size=block_size, device=None)


def _run_iteration(cache, sched):
    p = sched.plan()
    if p["ids"]:
        cache.reserve_host(p["ids"], p["n_new"])   # the plan must fit: no KVC_E_NO_BLOCKS
    return p, sched.commit()


def test_hand_worked_plans():
    # pool 10 blocks of 4 tokens; chunk 8, budget 16, batch 4
    cache = _cache(10)
    s = kvc.Scheduler(cache, 4, 8, 16)
    s.submit(1, 10, 3)        # prompt 10, 3 tokens
    s.submit(2, 5, 2)
    p, fin = _run_iteration(cache, s)
    assert p == dict(ids=[1, 2], n_new=[8, 5], start=[0, 0], emits=[0, 1], preempted=[]) and fin == []
    p, fin = _run_iteration(cache, s)      # 1 ends its prompt (emits), 2 writes its 1st token's row (emits, done)
    assert p == dict(ids=[1, 2], n_new=[2, 1], start=[8, 5], emits=[1, 1], preempted=[]) and fin == [2]
    assert cache.stats()["free_blocks"] == 7
    p, fin = _run_iteration(cache, s)
    assert p["ids"] == [1] and p["start"] == [10] and fin == []
    p, fin = _run_iteration(cache, s)
    assert p["ids"] == [1] and p["start"] == [11] and fin == [1]
    assert cache.stats()["free_blocks"] == 10
    st = s.stats()
    assert st["finished"] == 2 and st["tokens_scheduled"] == (10 + 3 - 1) + (5 + 2 - 1) and st["preemptions"] == 0


def test_hand_worked_preemption_and_recompute():
    # pool 4 blocks of 4 tokens: two requests of prompt 6 fill it after three
    # decode rows each; the fourth needs a block each, so the newer one (B) is
    # preempted, A runs to the end, then B re-prefills 6 + 3 tokens and goes on.
    cache = _cache(4)
    s = kvc.Scheduler(cache, 4, 8, 16)
    s.submit(10, 6, 8)        # A
    s.submit(11, 6, 8)        # B
    plans = []
    for _ in range(30):
        p, fin = _run_iteration(cache, s)
        plans.append((p, fin))
        if s.stats()["finished"] == 2:
            break
    p0 = plans[0][0]
    assert p0["ids"] == [10, 11] and p0["n_new"] == [6, 6] and p0["emits"] == [1, 1]
    for it in (1, 2):
        assert plans[it][0]["ids"] == [10, 11] and plans[it][0]["n_new"] == [1, 1]
    p3 = plans[3][0]
    assert p3["preempted"] == [11] and p3["ids"] == [10] and p3["start"] == [8]
    # A alone until it has emitted its 8 tokens (rows up to position 12)
    for it in range(4, 8):
        assert plans[it][0]["ids"] == [10]
    assert plans[7][1] == [10]
    # B re-prefills its prompt and its 3 emitted tokens: 8 rows, then 1 row that emits
    p8 = plans[8][0]
    assert p8["ids"] == [11] and p8["n_new"] == [8] and p8["start"] == [0] and p8["emits"] == [0]
    p9 = plans[9][0]
    assert p9["ids"] == [11] and p9["n_new"] == [1] and p9["start"] == [8] and p9["emits"] == [1]
    st = s.stats()
    assert st["preemptions"] == 1 and st["finished"] == 2
    assert cache.stats()["free_blocks"] == 4


@pytest.mark.parametrize("trial", range(6))
def test_random_workloads_keep_the_invariants(trial):
    rng = random.Random(100 + trial)
    bs = rng.choice([4, 16])
    nblocks = rng.randint(12, 60)
    max_batch, chunk, budget = rng.randint(1, 8), rng.randint(1, 40), rng.randint(8, 120)
    cache = _cache(nblocks, bs)
    s = kvc.Scheduler(cache, max_batch, chunk, budget)
    reqs = {}
    # every request must fit the pool alone, or the run could not finish
    cap_tokens = nblocks * bs
    for i in range(rng.randint(5, 30)):
        P = rng.randint(1, min(200, cap_tokens // 2))
        M = rng.randint(1, min(60, cap_tokens - P))
        reqs[i] = dict(P=P, M=M, emitted=0, cached=0, rows=0)
        s.submit(i, P, M)
    first_admit = []
    for it in range(20000):
        p = s.plan()
        assert len(p["ids"]) <= max_batch and len(set(p["ids"])) == len(p["ids"])
        for r in p["preempted"]:
            reqs[r]["cached"] = 0
        decode_rows = sum(1 for r, n in zip(p["ids"], p["n_new"]) if reqs[r]["cached"] >= reqs[r]["P"])
        prefill_rows = sum(p["n_new"]) - decode_rows
        assert prefill_rows <= max(0, budget - decode_rows)
        for r, n, st, em in zip(p["ids"], p["n_new"], p["start"], p["emits"]):
            q = reqs[r]
            if q["cached"] == 0 and r not in first_admit:
                first_admit.append(r)
            assert st == q["cached"] and n >= 1
            known = q["P"] + q["emitted"]
            assert q["cached"] + n <= known
            assert em == (1 if q["cached"] + n == known else 0)
        if p["ids"]:
            cache.reserve_host(p["ids"], p["n_new"])
        fin = s.commit()
        for r, n, em in zip(p["ids"], p["n_new"], p["emits"]):
            reqs[r]["cached"] += n
            reqs[r]["rows"] += n
            reqs[r]["emitted"] += em
        for r in fin:
            assert reqs[r]["emitted"] == reqs[r]["M"]
        if s.stats()["finished"] == len(reqs):
            break
    else:
        raise AssertionError("the workload did not finish")
    assert first_admit == sorted(first_admit), "admission overtook an earlier request"
    st = s.stats()
    for q in reqs.values():
        assert q["emitted"] == q["M"]
        assert q["rows"] >= q["P"] + q["M"] - 1
    assert st["tokens_scheduled"] == sum(q["rows"] for q in reqs.values())
    assert cache.stats()["free_blocks"] == nblocks and cache.stats()["num_seqs"] == 0


def test_scheduler_errors():
    cache = _cache(3)
    with pytest.raises(kvc.KvcError):
        kvc.Scheduler(cache, 0, 8, 8)
    s = kvc.Scheduler(cache, 2, 8, 16)
    s.submit(1, 5, 2)
    with pytest.raises(kvc.KvcError) as e:
        s.submit(1, 5, 2)
    assert e.value.status == 5                 # KVC_E_SEQ_EXISTS
    with pytest.raises(kvc.KvcError):
        s.submit(2, 0, 2)
    s.plan()
    with pytest.raises(kvc.KvcError) as e:
        s.plan()                               # previous plan not committed
    assert e.value.status == 1
    with pytest.raises(kvc.KvcError) as e:
        s.commit()                             # planned rows not appended
    assert e.value.status == 1
    # a request whose first chunk cannot fit an empty pool
    s2 = kvc.Scheduler(_cache(1), 2, 8, 16)
    s2.submit(7, 6, 1)
    with pytest.raises(kvc.KvcError) as e:
        s2.plan()
    assert e.value.status == 3                 # KVC_E_NO_BLOCKS
    # a request that outgrows the whole pool on its own
    c3 = _cache(2)
    s3 = kvc.Scheduler(c3, 2, 8, 16)
    s3.submit(9, 6, 20)
    for _ in range(3):                         # rows 0..5, then 6 and 7: 8 tokens, 2 blocks
        _run_iteration(c3, s3)
    with pytest.raises(kvc.KvcError) as e:
        s3.plan()
    assert e.value.status == 3
