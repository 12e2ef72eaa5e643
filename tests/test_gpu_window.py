"""GPU parity under a sliding window with KV eviction.

The history is written in chunks, and after each chunk the blocks that the
step's tokens will no longer see are released (kvc_evict) and reused by later
appends.  Checked against the oracle:

* block tables (with released entries) and the whole pools, bit-exact;
* decode (both kernels) and several new tokens per sequence under the window,
  per element within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle's
  windowed attention on the stored values;
* a window of one row, a window longer than the history (bitwise equal to no
  window), forced splits, and the full-size windowed workload on sampled
  sequences.
"""
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import (check_close, decode_poisoned, extend_poisoned, gpu_decode_again, gpu_extend_step, gpu_setup,
                     gpu_step, oracle_decode, oracle_extend, oracle_run, read_pools, to_f64)
from workloads import custom_workload, make_values, make_window_workload, setup_ops

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_state(cache, st, wl, bt, cl):
    pools = read_pools(cache)
    assert np.array_equal(pools["k"], st.k), "K pool differs from the oracle's store"
    assert np.array_equal(pools["v"], st.v), "V pool differs from the oracle's store"
    if wl.kv_dtype in ("fp8", "int8"):
        assert np.array_equal(pools["k_scale"].view(np.uint32), st.k_scale.view(np.uint32))
        assert np.array_equal(pools["v_scale"].view(np.uint32), st.v_scale.view(np.uint32))
    rows, lens = st.tables.export(list(range(wl.batch)), bt.shape[1])
    assert np.array_equal(bt.cpu().numpy(), np.array(rows, dtype=np.int32)), "block tables differ"
    assert np.array_equal(cl.cpu().numpy(), np.array(lens, dtype=np.int32))
    assert (bt.cpu().numpy() == -1).any(), "no block was released"


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8", "f32"])
def test_window_decode_after_eviction(kv):
    wl = make_window_workload(small=True, kv_dtype=kv)
    _say(f"[window] decode {kv}: {wl.name}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values, partition_tokens=64)
    torch.cuda.synchronize()
    _check_state(cache, st, wl, bt, cl)
    assert cache.stats()["used_blocks"] <= wl.batch * ((wl.window + 15) // 16 + 1)
    ref = oracle_decode(st, wl, values)
    for kernel in ([1] if kv == "f32" else [1, 2]):
        for wi in (0, 3):
            o = gpu_decode_again(cache, wl, values, bt, cl, kernel=kernel, partition_tokens=64, work_items=wi)
            torch.cuda.synchronize()
            check_close(to_f64(o), ref, *TOL, f"window decode {kv} kernel {kernel} work_items {wi}")


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8"])
def test_window_several_new_tokens(kv):
    wl = make_window_workload(small=True, kv_dtype=kv, query_lens=[3, 1, 40, 17], seed=9)
    _say(f"[window] several tokens {kv}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl, qs = gpu_extend_step(cache, wl, values)
    torch.cuda.synchronize()
    ref = oracle_extend(st, wl, values)
    check_close(to_f64(out), ref, *TOL, f"window extend {kv}")
    q = values["q"].cuda().contiguous()
    for wi, tpw in ((2, 0), (9, 0), (4, 1), (3, 2), (6, 3)):
        o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, work_items=wi,
                         window=wl.window, tiles_per_wave=tpw, kernel=2)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"window extend {kv} work_items {wi}")
    o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, window=wl.window, kernel=3)
    torch.cuda.synchronize()
    check_close(to_f64(o), ref, *TOL, f"window extend {kv} kernel 3")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_window_limits(kv):
    lens = [100, 33, 257, 1, 40]
    wl = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=31, name="window limits")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    full, bt, cl = gpu_step(cache, wl, values)
    q = values["q"].cuda().contiguous()
    # a window longer than every history changes nothing, bit for bit
    for kernel in (1, 2):
        ref_k = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=32)
        o = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=32, window=258)
        torch.cuda.synchronize()
        assert torch.equal(ref_k.view(torch.int16), o.view(torch.int16)), f"kernel {kernel}"
    # a window of one row: each token returns its own value row (dequantised)
    wl.window = 1
    ref = oracle_decode(st, wl, values)
    for kernel in (1, 2):
        o = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=32, window=1)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"window 1 kernel {kernel}")
    # assorted windows, including one ending inside a block
    for w in (5, 16, 17, 100):
        wl.window = w
        ref = oracle_decode(st, wl, values)
        for kernel in (1, 2):
            o = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=32, window=w,
                             work_items=4)
            torch.cuda.synchronize()
            check_close(to_f64(o), ref, *TOL, f"window {w} kernel {kernel}")


def test_full_size_window_decode_sampled():
    from oracle.attention import extend_attention
    from oracle.kvstore import KVStoreModel
    wl = make_window_workload()
    _say(f"[window full] {wl.name}; {wl.num_blocks} blocks")
    values = make_values(wl, "cuda")
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    got = to_f64(out)
    q = to_f64(values["q"])
    rows = bt.cpu().numpy()
    pools = read_pools(cache)
    from harness import _history_rows, to_bits
    for b in sorted({0, wl.batch // 2, wl.batch - 1}):
        # the window's rows of b straight from the workload tensors, checked
        # against the pool through b's exported table, then the oracle on them
        L = int(wl.context_lens[b])
        n = L + 1
        lo = n - wl.window
        st = KVStoreModel(1, (n + 15) // 16, wl.num_kv_heads, wl.head_dim, 16, wl.kv_dtype, in_dtype=wl.new_dtype)
        st.allocate(0, 0)
        hr = _history_rows(wl, b).to(values["k_hist"].device)
        kb = to_bits(values["k_hist"][:, hr], wl.new_dtype)
        vb = to_bits(values["v_hist"][:, hr], wl.new_dtype)
        assert st.append([0], [L], kb, vb)[0] == 0
        assert st.append([0], [1], to_bits(values["k_new"][:, b:b + 1], wl.new_dtype),
                         to_bits(values["v_new"][:, b:b + 1], wl.new_dtype))[0] == 0
        for j in range(lo // 16, (n + 15) // 16):
            assert rows[b][j] >= 0, f"seq {b}: block {j} inside the window was released"
            assert np.array_equal(pools["k"][rows[b][j]], st.k[st.tables.tables[0][j]]), f"seq {b} block {j} K"
            assert np.array_equal(pools["v"][rows[b][j]], st.v[st.tables.tables[0][j]]), f"seq {b} block {j} V"
        # everything before the oldest needed position was released
        assert all(rows[b][j] == -1 for j in range((L - wl.window + 1) // 16)), f"seq {b}: not evicted"
        k, v = st.gather(0, start=lo)
        ref = extend_attention(q[b:b + 1], k, v, wl.scale, window=wl.window)[0]
        ma, mr = check_close(got[b], ref, *TOL, f"window full seq {b}")
        _say(f"  seq {b}: max_abs {ma:.2e} max_rel {mr:.2e}")
