"""GPU parity: libkvc's HIP path against the oracle (needs an MI355X).

* append: the whole pool (and fp8 scales) bit-exact against the oracle's store,
  block tables and lengths bit-exact against the oracle's allocator model;
* decode: per element |gpu - ref| <= atol + rtol * |ref| with (2e-3, 1e-2) for
  f32 / f16 / bf16 caches and for fp8 against the oracle fed the stored
  (dequantised) values, and (5e-2, 1e-2) for fp8 against the unquantised rows;
* placement invariance and run-to-run determinism bitwise; partition-boundary
  sweeps; both decode kernels (fp32 FMA and MFMA).
"""
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import (check_close, decode_poisoned, gpu_decode_again, gpu_setup, gpu_step, logical_history,
                     oracle_decode, oracle_run, read_pools, to_f64)
from workloads import custom_workload, make_values, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"f32": (2e-3, 1e-2), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "fp8": (2e-3, 1e-2), "int8": (2e-3, 1e-2)}
FP8_UNQUANT_TOL = (5e-2, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _kernels_for(wl):
    return [1] if wl.kv_dtype == "f32" else [1, 2]


def _check_append(cache, st, wl, bt, cl):
    pools = read_pools(cache)
    assert np.array_equal(pools["k"], st.k), "K pool differs from the oracle's store"
    assert np.array_equal(pools["v"], st.v), "V pool differs from the oracle's store"
    if wl.kv_dtype in ("fp8", "int8"):
        assert np.array_equal(pools["k_scale"].view(np.uint32), st.k_scale.view(np.uint32))
        assert np.array_equal(pools["v_scale"].view(np.uint32), st.v_scale.view(np.uint32))
    rows, lens = st.tables.export(list(range(wl.batch)), bt.shape[1])
    assert np.array_equal(bt.cpu().numpy(), np.array(rows, dtype=np.int32))
    assert np.array_equal(cl.cpu().numpy(), np.array(lens, dtype=np.int32))
    assert np.array_equal(cl.cpu().numpy(), wl.attend_lens)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, "5-int8"])
def test_small_configs_append_and_decode(cid):
    # "5-int8": the fp8 mixed batch with an int8 cache instead
    wl = make_workload(5, small=True, kv_dtype="int8") if cid == "5-int8" else make_workload(cid, small=True)
    _say(f"[parity] config {cid} (small): {wl.name}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    _check_append(cache, st, wl, bt, cl)
    ref = oracle_decode(st, wl, values)
    atol, rtol = TOL[wl.kv_dtype]
    for kernel in _kernels_for(wl):
        o = out if kernel == _kernels_for(wl)[-1] else gpu_decode_again(cache, wl, values, bt, cl, kernel=kernel)
        got = to_f64(o)
        ma, mr = check_close(got, ref, atol, rtol, f"config {cid} kernel {kernel}")
        _say(f"  kernel {kernel}: max_abs {ma:.2e} max_rel {mr:.2e}")
    if wl.kv_dtype in ("fp8", "int8"):
        # end to end, quantisation error included: against the unquantised rows
        # (the lengths here start at 256, as in the full fp8 workload)
        from oracle.attention import decode_attention
        q = to_f64(values["q"])
        worst = 0.0
        for b in range(wl.batch):
            k, v = logical_history(wl, values, b)
            r = decode_attention(q[b], k, v, wl.scale)
            ma, _ = check_close(to_f64(out[b]), r, *FP8_UNQUANT_TOL, f"config {cid} seq {b} vs unquantised rows")
            worst = max(worst, ma)
        _say(f"  {wl.kv_dtype} vs unquantised rows: max_abs {worst:.2e}")


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "fp8", "int8"])
@pytest.mark.parametrize("pt", [16, 64])
def test_partition_boundaries(kv, pt):
    # Lengths around block and partition edges.  The FMA kernel cuts each
    # sequence into pt-token partitions; the MFMA kernel cuts the batch's
    # concatenated blocks into work_items runs, swept from one wave holding
    # everything to more waves than blocks.
    lens = [0, 14, 15, 16, pt - 2, pt - 1, pt, pt + 15, 2 * pt, 3 * pt + 5]
    wl = custom_workload(len(lens), 8, 2, 64 if kv == "f32" else 128, kv, lens, seed=11, name=f"boundary {kv} {pt}")
    _say(f"[parity] partition boundaries kv={kv} partition_tokens={pt}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values, partition_tokens=pt)
    torch.cuda.synchronize()
    _check_append(cache, st, wl, bt, cl)
    ref = oracle_decode(st, wl, values)
    o = gpu_decode_again(cache, wl, values, bt, cl, kernel=1, partition_tokens=pt)
    check_close(to_f64(o), ref, *TOL[kv], f"{kv} P={pt} FMA kernel")
    if kv != "f32":
        for wi in (1, 2, 3, 7, 13, 64, 1000):
            o = gpu_decode_again(cache, wl, values, bt, cl, kernel=2, work_items=wi)
            check_close(to_f64(o), ref, *TOL[kv], f"{kv} MFMA kernel work_items={wi}")


def test_long_segments_cross_the_block_id_window():
    # one sequence of 300 blocks held by one wave: the wave walks its block ids
    # 64 at a time while prefetching across the window edge
    lens = [300 * 16 - 5, 7, 130 * 16]
    for kv in ("bf16", "fp8"):
        wl = custom_workload(len(lens), 8, 2, 128, kv, lens, seed=21, name="long segments")
        values = make_values(wl, "cpu")
        st = oracle_run(wl, values)
        cache = gpu_setup(wl, values)
        out, bt, cl = gpu_step(cache, wl, values, kernel=2, work_items=1)
        torch.cuda.synchronize()
        ref = oracle_decode(st, wl, values)
        check_close(to_f64(out), ref, *TOL[kv], f"{kv} one wave")
        for wi in (2, 5):
            o = gpu_decode_again(cache, wl, values, bt, cl, kernel=2, work_items=wi)
            check_close(to_f64(o), ref, *TOL[kv], f"{kv} work_items={wi}")


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8"])
def test_dynamic_pool_pieces(kv):
    # The MFMA decode hands the last 1/2^shift of every wave's run out at run
    # time in `pieces` pieces, each at least two turns of the prefetch ring
    # long (10 blocks for 16-bit caches, 8 for one-byte codes; 346 blocks per
    # head here).  Cases: one wave taking its own pool, several waves
    # competing for pieces that cut across sequence boundaries, and pools too
    # small for their piece count (pool unused).  Every result matches the
    # oracle and repeats bit for bit, whichever wave took which piece.
    lens = [16 * 90 + 3, 1, 17, 16 * 41, 5, 16 * 200 - 1, 33, 16 * 7]
    wl = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=41, name="dynamic pool")
    _say(f"[parity] dynamic pool kv={kv}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values, kernel=2, work_items=3, pool_pieces=-1)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    check_close(to_f64(out), ref, *TOL[kv], f"{kv} static split")
    for wi, pieces, shift in [(1, 1, 1), (2, 1, 1), (3, 2, 1), (3, 4, 1), (4, 2, 2), (5, 3, 1), (8, 1, 2),
                              (16, 1, 1), (3, 2, 3), (3, 8, 1), (7, 64, 6), (40, 2, 3), (2, 5, 4), (64, 1, 1)]:
        split = dict(kernel=2, work_items=wi, pool_pieces=pieces, pool_shift=shift)
        o = gpu_decode_again(cache, wl, values, bt, cl, **split)
        check_close(to_f64(o), ref, *TOL[kv], f"{kv} work_items={wi} pieces={pieces} shift={shift}")
        again = gpu_decode_again(cache, wl, values, bt, cl, **split)
        torch.cuda.synchronize()
        check_close(to_f64(again), ref, *TOL[kv], f"{kv} repeat of work_items={wi} pieces={pieces} shift={shift}")
        assert_same_bits(o, again, f"not deterministic: {split}")


def assert_same_bits(a, b, what):
    """a and b bit for bit; else name the (sequence, head) pairs that differ."""
    same = a.view(torch.int16) == b.view(torch.int16)
    if bool(same.all()):
        return
    bad = (~same).nonzero().cpu().tolist()
    pairs = sorted({(s, h) for s, h, _ in bad})
    diff = (a.float() - b.float()).abs().max().item()
    raise AssertionError(f"{what}: {len(bad)} elements differ, max |diff| {diff:.3g}, "
                         f"(sequence, head) pairs {pairs[:24]}")


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 4, 128), (16, 4, 64), (16, 1, 128), (32, 2, 128), (12, 3, 64)])
@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8"])
def test_head_groupings(hq, hkv, d, kv):
    lens = [5, 40, 300, 129]
    wl = custom_workload(len(lens), hq, hkv, d, kv, lens, seed=hq * 7 + hkv, name="groupings")
    _say(f"[parity] heads {hq}/{hkv} D={d} kv={kv}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values, partition_tokens=128)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    for kernel in (1, 2):
        o = gpu_decode_again(cache, wl, values, bt, cl, kernel=kernel, partition_tokens=128)
        check_close(to_f64(o), ref, *TOL[kv], f"{hq}/{hkv} D{d} {kv} kernel {kernel}")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_placement_invariance_and_determinism(kv):
    lens = [100, 33, 257, 1]
    outs = []
    for seed_order in (None, 5):
        wl = custom_workload(len(lens), 16, 4, 128, kv, lens, seed=3, name="placement")
        if seed_order is None:
            wl.free_order = np.arange(wl.num_blocks, dtype=np.int32)[::-1].copy()   # pops 0, 1, 2, ...: contiguous
        else:
            wl.free_order = np.random.default_rng(seed_order).permutation(wl.num_blocks).astype(np.int32)
        values = make_values(wl, "cpu")
        cache = gpu_setup(wl, values)
        out, bt, cl = gpu_step(cache, wl, values, partition_tokens=64, work_items=5)
        again = gpu_decode_again(cache, wl, values, bt, cl, partition_tokens=64, work_items=5)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "decode not deterministic"
        outs.append(out.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "result depends on placement"


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_fork_mid_block_copy_on_write(kv):
    # prefix of 21 tokens (block 1 half full) shared by 3 sequences; each then
    # appends its own rows: the first write into the shared half block copies it.
    wl = custom_workload(3, 8, 2, 128, kv, [21 + 9, 21 + 2, 21 + 30], seed=4, shared_prefix=21, name="cow")
    wl.num_blocks += 4
    wl.free_order = np.random.default_rng(1).permutation(wl.num_blocks).astype(np.int32)
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values, partition_tokens=32, work_items=3)
    torch.cuda.synchronize()
    assert cache.stats()["cow_copies"] == st.tables.cow_copies >= 2
    _check_append(cache, st, wl, bt, cl)
    ref = oracle_decode(st, wl, values)
    check_close(to_f64(out), ref, *TOL[kv], f"cow {kv}")


def test_stream_copy_calibration_kernel():
    from paged_kv_cache_split_amd import stream_copy
    src = torch.randint(0, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_stream_read_calibration_kernel():
    # every 16-byte chunk read once: the xor of what the waves store equals
    # the xor of every word of the source (no two waves share a sink word here)
    from paged_kv_cache_split_amd import stream_read
    for n in (1 << 20, (1 << 22) + 48):
        src = torch.randint(0, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
        sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
        stream_read(src, sink)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8", "f32"])
def test_multi_layer_pool_and_cow(kv):
    # three layers share one block id space: appends write every layer, a
    # copy-on-write copies every layer (and fp8 scales), decode reads one layer
    wl = custom_workload(3, 8, 2, 64, kv, [21 + 9, 21 + 2, 40], seed=6, shared_prefix=21, name="layers")
    wl.num_layers = 3
    wl.num_blocks += 4
    wl.free_order = np.random.default_rng(2).permutation(wl.num_blocks).astype(np.int32)
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out0, bt, cl = gpu_step(cache, wl, values, partition_tokens=32, work_items=3)
    torch.cuda.synchronize()
    assert cache.stats()["cow_copies"] == st.tables.cow_copies >= 2
    _check_append(cache, st, wl, bt, cl)
    for layer in range(3):
        ref = oracle_decode(st, wl, values, layer=layer)
        for kernel in _kernels_for(wl):
            q = values["q"].to("cuda").contiguous()
            o = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, layer=layer, kernel=kernel,
                             partition_tokens=32, work_items=3)
            check_close(to_f64(o), ref, *TOL[kv], f"{kv} layer {layer} kernel {kernel}")


def test_decode_rejects_negative_or_infinite_scale():
    from paged_kv_cache_split_amd import KvcError
    lens = [20, 3]
    wl = custom_workload(len(lens), 8, 2, 128, "bf16", lens, seed=11, name="scale checks")
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    q = values["q"].to("cuda").contiguous()
    for bad in (-0.125, float("inf"), float("nan")):
        with pytest.raises(KvcError):
            decode_poisoned(cache, q, bt, cl, wl.max_context_len, bad)
    # scale 0 is allowed: every weight is equal, the output is the mean of V
    z = decode_poisoned(cache, q, bt, cl, wl.max_context_len, 0.0)
    torch.cuda.synchronize()
    start = 0
    for b, n in enumerate(lens):
        v = torch.cat([values["v_hist"][0, start:start + n], values["v_new"][0, b:b + 1]]).to(torch.float64)
        start += n
        mean = v.mean(0)                                   # [Hkv, D]
        ref = mean.repeat_interleave(wl.num_heads // wl.num_kv_heads, 0).numpy()
        check_close(to_f64(z[b]), ref, *TOL["bf16"], f"scale 0 seq {b}")
