"""GPU parity of the decode step with its append folded in (needs a GPU).

kvc_append without rows reserves the step's slots (and copies shared blocks);
kvc_decode_attention with opts.k_new / v_new then writes each sequence's
newest row -- inside the matrix-core walk for 16-bit caches with the static
split (the wave that reads a sequence's last block writes it first), through
an append kernel driven by the block table otherwise -- and attends.

* the pools afterwards, bit-exact against the oracle's store after the same
  append (every layer of a multi-layer pool, fp8 / int8 scales included);
* the outputs within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the fp64 oracle and
  bit-identical to the two-call step (append with rows, then decode) in the
  same launch configuration;
* work-item sweeps, the dynamic pool and the fp32 FMA kernel (append kernel
  first), a sliding window, a shared prefix, copy-on-write into a forked
  half-full block, and a bad table entry that must not be written.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import (check_close, decode_poisoned, gpu_setup, oracle_decode, oracle_run, read_pools, to_f64)
from workloads import custom_workload, make_values, make_window_workload, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _same_pools(cache, st, wl):
    pools = read_pools(cache)
    assert np.array_equal(pools["k"], st.k), "K pool differs from the oracle's store"
    assert np.array_equal(pools["v"], st.v), "V pool differs from the oracle's store"
    if wl.kv_dtype in ("fp8", "int8"):
        assert np.array_equal(pools["k_scale"].view(np.uint32), st.k_scale.view(np.uint32))
        assert np.array_equal(pools["v_scale"].view(np.uint32), st.v_scale.view(np.uint32))


def _fused_step(cache, wl, values, layer=0, **opts):
    """Reserve without rows, export tables, decode layer `layer` writing its rows."""
    seqs = list(range(wl.batch))
    cache.append(seqs, None, None)
    bt, cl = cache.export_tables(seqs)
    q = values["q"].cuda().contiguous()
    kn = values["k_new"][layer].cuda().contiguous()
    vn = values["v_new"][layer].cuda().contiguous()
    o = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, layer=layer, window=wl.window,
                        k_new=kn, v_new=vn, **opts)
    return o, bt, cl


def _two_call_out(wl, values, **opts):
    """The same step as append-with-rows then decode, on a fresh cache."""
    cache = gpu_setup(wl, values)
    seqs = list(range(wl.batch))
    cache.append(seqs, values["k_new"].cuda().contiguous(), values["v_new"].cuda().contiguous())
    bt, cl = cache.export_tables(seqs)
    q = values["q"].cuda().contiguous()
    return decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, window=wl.window, **opts)


def _case(wl, label, **opts):
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = _fused_step(cache, wl, values, **opts)
    torch.cuda.synchronize()
    _same_pools(cache, st, wl)
    ref = oracle_decode(st, wl, values)
    ma, _ = check_close(to_f64(out), ref, *TOL, f"{label} folded append")
    two = _two_call_out(wl, values, **opts)
    torch.cuda.synchronize()
    bits = torch.int32 if wl.kv_dtype == "f32" else torch.int16
    assert torch.equal(out.view(bits), two.view(bits)), f"{label}: folded step differs from append + decode"
    _say(f"  {label}: max_abs {ma:.2e}")


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, "5-int8"])
def test_small_configs(cid):
    wl = make_workload(5, small=True, kv_dtype="int8") if cid == "5-int8" else make_workload(cid, small=True)
    _say(f"[folded append] config {cid} (small): {wl.name}")
    _case(wl, f"config {cid}")


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8"])
def test_splits_pool_and_fma(kv):
    lens = [0, 14, 15, 16, 300, 31, 1, 129, 47, 16 * 40 - 1]
    wl = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=61, name="folded append splits")
    _say(f"[folded append] splits kv={kv}")
    for opts in (dict(kernel=2, work_items=1), dict(kernel=2, work_items=3), dict(kernel=2, work_items=17),
                 dict(kernel=2, work_items=1000), dict(kernel=2, work_items=3, pool_pieces=2, pool_shift=1),
                 dict(kernel=1, partition_tokens=64)):
        _case(wl, f"{kv} {opts}", **opts)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_window_and_shared_prefix(kv):
    wl = make_window_workload(small=True, kv_dtype=kv)
    _say(f"[folded append] window kv={kv}")
    _case(wl, f"window {kv}")
    lens = [128 + x for x in (0, 3, 300, 16, 33, 1)]
    wl = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=62, shared_prefix=128, name="folded prefix")
    _case(wl, f"shared prefix {kv}", kernel=2, shared_prefix=128)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_copy_on_write_and_layers(kv):
    # a 21-token prefix (block 1 half full) forked three ways: the reserve-only
    # append copies that block for every writer, then each layer's decode
    # writes its own rows into the copies
    wl = custom_workload(3, 8, 2, 128, kv, [21, 21, 21], seed=63, shared_prefix=21, name="folded cow")
    wl = dataclasses.replace(wl, num_layers=3, num_blocks=wl.num_blocks + 6)
    wl.free_order = np.random.default_rng(4).permutation(wl.num_blocks).astype(np.int32)
    _say(f"[folded append] copy-on-write, {wl.num_layers} layers, kv={kv}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    seqs = list(range(wl.batch))
    cache.append(seqs, None, None)
    assert cache.stats()["cow_copies"] == st.tables.cow_copies >= 2
    bt, cl = cache.export_tables(seqs)
    q = values["q"].cuda().contiguous()
    outs = []
    for layer in range(wl.num_layers):
        outs.append(decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, layer=layer,
                                    k_new=values["k_new"][layer].cuda().contiguous(),
                                    v_new=values["v_new"][layer].cuda().contiguous()))
    torch.cuda.synchronize()
    _same_pools(cache, st, wl)
    for layer, o in enumerate(outs):
        check_close(to_f64(o), oracle_decode(st, wl, values, layer=layer), *TOL, f"cow {kv} layer {layer}")


def test_bad_table_entry_is_not_written():
    # a table entry outside [0, num_blocks) for the newest row: no write
    # anywhere (the pool is unchanged but for the good sequences' rows)
    lens = [40, 17]
    wl = custom_workload(len(lens), 8, 2, 128, "bf16", lens, seed=64, name="folded bad entry")
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    seqs = list(range(wl.batch))
    cache.append(seqs, None, None)
    bt, cl = cache.export_tables(seqs)
    before = read_pools(cache)
    bt[1, (int(cl[1]) - 1) // 16] = wl.num_blocks + 5
    q = values["q"].cuda().contiguous()
    decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=2,
                    k_new=values["k_new"][0].cuda().contiguous(), v_new=values["v_new"][0].cuda().contiguous())
    torch.cuda.synchronize()
    after = read_pools(cache)
    changed = np.argwhere(np.any(before["k"] != after["k"], axis=(1, 2, 3, 4)))[:, 0].tolist()
    good = bt[0, (int(cl[0]) - 1) // 16].item()
    assert changed == [good], changed
