"""GPU parity of the multi-token call (several new tokens per sequence, causal
among them: the verify pass of speculative decoding, a prefill chunk) against
the oracle's ``extend_attention`` on the stored values.

* the pools after the step's append, bit-exact against the oracle's store;
* outputs per element within |gpu - ref| <= 2e-3 + 1e-2 |ref| for f16 / bf16
  caches and for fp8 against the dequantised stored values;
* ragged query counts (0, 1, one tile, many tiles per sequence), head
  groupings, forced splits of every sequence over many chunks (partials that
  see none of a chunk's rows), one token per sequence bitwise equal to the
  decode kernel, and pools whose unused slots hold NaN bit patterns; both
  several-token kernels (rows split over waves and merged, and one wave per
  32 columns over all their rows);
* the three multi-token workloads at full size on sampled sequences.
"""
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import (check_close, decode_poisoned, extend_poisoned, gpu_extend_step, gpu_setup, gpu_step, oracle_decode,
                     oracle_extend, oracle_run, query_start, read_pools, to_bits, to_f64, _history_rows)
from workloads import custom_workload, make_extend_workload, make_values

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_pools(cache, st, wl):
    pools = read_pools(cache)
    assert np.array_equal(pools["k"], st.k), "K pool differs from the oracle's store"
    assert np.array_equal(pools["v"], st.v), "V pool differs from the oracle's store"
    if wl.kv_dtype in ("fp8", "int8"):
        assert np.array_equal(pools["k_scale"].view(np.uint32), st.k_scale.view(np.uint32))
        assert np.array_equal(pools["v_scale"].view(np.uint32), st.v_scale.view(np.uint32))


@pytest.mark.parametrize("kind", ["verify", "prefill", "chunk"])
def test_small_extend_workloads(kind):
    wl = make_extend_workload(kind, small=True)
    _say(f"[extend] {kind} (small): {wl.name}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl, qs = gpu_extend_step(cache, wl, values)
    torch.cuda.synchronize()
    _check_pools(cache, st, wl)
    assert np.array_equal(cl.cpu().numpy(), wl.attend_lens)
    ref = oracle_extend(st, wl, values)
    check_close(to_f64(out), ref, *TOL, f"extend {kind}")
    q = values["q"].cuda().contiguous()
    for kernel in (2, 3):
        o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, kernel=kernel)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"extend {kind} kernel {kernel}")


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8"])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (16, 16, 64), (16, 1, 128), (12, 3, 64), (64, 8, 128)])
def test_ragged_query_counts(kv, hq, hkv, d):
    # history lengths and new tokens per sequence: none, one, within a tile,
    # across several tiles and blocks, a whole uncached prompt
    lens = [0, 5, 40, 300, 129, 16, 1, 77]
    qls = [3, 1, 0, 17, 2, 40, 6, 33]
    wl = custom_workload(len(lens), hq, hkv, d, kv, lens, seed=hq + 5 * hkv + d, name="ragged extend",
                         query_lens=qls)
    _say(f"[extend] ragged heads {hq}/{hkv} D={d} kv={kv}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl, qs = gpu_extend_step(cache, wl, values)
    torch.cuda.synchronize()
    _check_pools(cache, st, wl)
    ref = oracle_extend(st, wl, values)
    check_close(to_f64(out), ref, *TOL, f"ragged {hq}/{hkv} D{d} {kv}")
    # many chunks per sequence: tiles whose tokens see none of a chunk's rows
    # leave empty partials that the merge must skip
    q = values["q"].cuda().contiguous()
    for wi, tpw in ((2, 0), (7, 0), (64, 0), (0, 1), (5, 2), (3, 3), (9, 4)):
        o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, work_items=wi,
                         tiles_per_wave=tpw, kernel=2)
        torch.cuda.synchronize()
        check_close(to_f64(o), ref, *TOL, f"ragged {hq}/{hkv} D{d} {kv} work_items {wi} tiles/wave {tpw}")
    # one wave per 32 (token, head) columns over all their rows: tiles with
    # padding columns, tokens of one column tile in several sequences' worth of
    # heads, an odd number of blocks
    o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, kernel=3)
    torch.cuda.synchronize()
    check_close(to_f64(o), ref, *TOL, f"ragged {hq}/{hkv} D{d} {kv} kernel 3")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_one_token_per_sequence_matches_decode_bitwise(kv):
    lens = [100, 33, 257, 1, 4000]
    wl = custom_workload(len(lens), 32, 8, 128, kv, lens, seed=17, name="extend = decode")
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    dec, bt, cl = gpu_step(cache, wl, values, work_items=100)
    qs = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    ext = extend_poisoned(cache, values["q"].cuda().contiguous(), qs, 1, bt, cl, wl.max_context_len, wl.scale, work_items=100)
    torch.cuda.synchronize()
    assert torch.equal(dec.view(torch.int16), ext.view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8", "f32"])
def test_unwritten_slots_holding_nan(kv):
    # Pools whose every byte is 0xFF (a NaN in each dtype) before anything is
    # written: the slots past each sequence's end in its last block are read
    # but must not reach the result.
    lens = [20, 3, 130, 47]
    qls = [2, 5, 1, 9]
    wl = custom_workload(len(lens), 16, 4, 128 if kv != "f32" else 64, kv, lens, seed=23, name="nan slots")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values, pool_fill=255)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    for kernel in ([1] if kv == "f32" else [1, 2]):
        o = decode_poisoned(cache, values["q"].cuda().contiguous(), bt, cl, wl.max_context_len, wl.scale, kernel=kernel,
                         partition_tokens=32)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all(), f"kernel {kernel}: NaN from unused slots"
        check_close(to_f64(o), ref, *TOL, f"nan slots {kv} kernel {kernel}")
    if kv == "f32":
        return
    # several new tokens per sequence on a fresh NaN-filled cache
    wl2 = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=29, name="nan slots extend", query_lens=qls)
    values2 = make_values(wl2, "cpu")
    st2 = oracle_run(wl2, values2)
    cache2 = gpu_setup(wl2, values2, pool_fill=255)
    out2, bt2, cl2, qs2 = gpu_extend_step(cache2, wl2, values2)
    torch.cuda.synchronize()
    assert torch.isfinite(out2.float()).all()
    ref2 = oracle_extend(st2, wl2, values2)
    check_close(to_f64(out2), ref2, *TOL, f"nan slots extend {kv}")
    o3 = cache2.extend(values2["q"].cuda().contiguous(), qs2, wl2.max_query_len, bt2, cl2, wl2.max_context_len,
                       wl2.scale, kernel=3)
    torch.cuda.synchronize()
    assert torch.isfinite(o3.float()).all(), "kernel 3: NaN from unused slots"
    check_close(to_f64(o3), ref2, *TOL, f"nan slots extend {kv} kernel 3")


def _oracle_single(wl, values, b):
    """Oracle store holding sequence b alone, written the way the GPU wrote it
    (history in one append, then the step's new tokens)."""
    from oracle.kvstore import KVStoreModel
    L = int(wl.context_lens[b])
    ql = int(wl.q_lens[b])
    st = KVStoreModel(1, (L + ql + 15) // 16, wl.num_kv_heads, wl.head_dim, 16, wl.kv_dtype, in_dtype=wl.new_dtype)
    st.allocate(0, 0)
    if L:
        rows = _history_rows(wl, b)
        kb = to_bits(values["k_hist"][:, rows.to(values["k_hist"].device)], wl.new_dtype)
        vb = to_bits(values["v_hist"][:, rows.to(values["v_hist"].device)], wl.new_dtype)
        assert st.append([0], [L], kb, vb)[0] == 0
    qs = query_start(wl)
    assert st.append([0], [ql], to_bits(values["k_new"][:, qs[b]:qs[b + 1]], wl.new_dtype),
                     to_bits(values["v_new"][:, qs[b]:qs[b + 1]], wl.new_dtype))[0] == 0
    return st


@pytest.mark.parametrize("kind", ["verify", "prefill", "chunk"])
def test_full_size_extend_sampled(kind):
    from oracle.attention import extend_attention
    wl = make_extend_workload(kind)
    _say(f"[extend full] {kind}: {wl.name}; {wl.total_queries} queries, {wl.num_blocks} blocks")
    values = make_values(wl, "cuda")
    cache = gpu_setup(wl, values)
    out, bt, cl, qs = gpu_extend_step(cache, wl, values)
    torch.cuda.synchronize()
    assert np.array_equal(cl.cpu().numpy(), wl.attend_lens)
    L = wl.context_lens
    sample = sorted({0, wl.batch - 1, int(np.argmin(L)), int(np.argmax(L))})
    qsn = query_start(wl)
    q = to_f64(values["q"])
    got = to_f64(out)
    pools = read_pools(cache)
    rows = bt.cpu().numpy()
    for b in sample:
        st = _oracle_single(wl, values, b)
        for i, blk in enumerate(st.tables.tables[0]):
            assert np.array_equal(pools["k"][rows[b][i]], st.k[blk]), f"seq {b} block {i} K"
            assert np.array_equal(pools["v"][rows[b][i]], st.v[blk]), f"seq {b} block {i} V"
        k, v = st.gather(0)
        ref = extend_attention(q[qsn[b]:qsn[b + 1]], k, v, wl.scale)
        ma, mr = check_close(got[qsn[b]:qsn[b + 1]], ref, *TOL, f"{kind} seq {b}")
        _say(f"  seq {b} (L={int(L[b])}, {int(wl.q_lens[b])} new): max_abs {ma:.2e} max_rel {mr:.2e}")
