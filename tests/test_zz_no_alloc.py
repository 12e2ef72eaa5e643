"""The allocation-free decode entry point (kvc_decode_attention_static).

Called through the C ABI, it must give the same bits as kvc_decode_attention
with a workspace of its own (poisoned with 0xFF bytes here) on the same
inputs, and match the fp64 oracle within |gpu - ref| <= 2e-3 + 1e-2 |ref|:
on two calls in a row, the second with a smaller input (fewer sequences,
shorter contexts), so partials the first call left in the shared static array
must not reach the second one's results.  Also the dynamic pool (whose ticket
counters the call zeroes itself), the shared-prefix decode, a one-byte cache,
and a shape beyond the static array's size (refused, nothing launched).
"""
import sys

import pytest
import torch

import paged_kv_cache_split_amd as kvc
from conftest import gpu_available
from harness import check_close, decode_poisoned, gpu_setup, gpu_step, oracle_decode, oracle_run, to_f64
from workloads import custom_workload, make_values, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_static_entry_point_two_calls_second_smaller(kv):
    wl = make_workload(3, small=True, kv_dtype=kv) if kv != "bf16" else make_workload(3, small=True)
    _say(f"[no-alloc] {wl.name}")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    q = values["q"].cuda().contiguous()
    for opts in (dict(), dict(kernel=2, work_items=7), dict(kernel=2, work_items=3, pool_pieces=2, pool_shift=1),
                 dict(kernel=1, partition_tokens=64)):
        # first call: the whole batch
        a = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, **opts)
        s = cache.decode_static(q, bt, cl, wl.max_context_len, wl.scale, **opts)
        torch.cuda.synchronize()
        _same_bits(s, a, f"{kv} {opts}: static entry point differs from the workspace one")
        check_close(to_f64(s), ref, *TOL, f"{kv} {opts} static")
        # second call right after: a smaller input, the first half of the
        # sequences with their tables cut to the blocks they hold
        half = wl.batch // 2
        lens = cl[:half].cpu().numpy()
        mb = int((lens.max() + 15) // 16)
        bt2, cl2 = bt[:half, :mb].contiguous(), cl[:half].contiguous()
        q2 = q[:half].contiguous()
        s2 = cache.decode_static(q2, bt2, cl2, int(lens.max()), wl.scale, **opts)
        a2 = decode_poisoned(cache, q2, bt2, cl2, int(lens.max()), wl.scale, **opts)
        torch.cuda.synchronize()
        _same_bits(s2, a2, f"{kv} {opts}: smaller second call differs")
        check_close(to_f64(s2), ref[:half], *TOL, f"{kv} {opts} static, smaller second call")


def test_static_entry_point_shared_prefix():
    lens = [128 + x for x in (0, 3, 300, 16, 33, 1)]
    wl = custom_workload(len(lens), 16, 4, 128, "bf16", lens, seed=71, shared_prefix=128, name="no-alloc prefix")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    _, bt, cl = gpu_step(cache, wl, values)
    q = values["q"].cuda().contiguous()
    a = decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, kernel=2, shared_prefix=128)
    s = cache.decode_static(q, bt, cl, wl.max_context_len, wl.scale, kernel=2, shared_prefix=128)
    torch.cuda.synchronize()
    _same_bits(s, a, "shared prefix: static entry point differs")
    check_close(to_f64(s), oracle_decode(st, wl, values), *TOL, "shared prefix static")


def test_static_entry_point_refuses_shapes_beyond_its_array():
    wl = make_workload(3, small=True)
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    _, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    # 8192 sequences of 64 query heads need ~280 MB of partials: refused
    # before any launch (the arguments are sized for the shape all the same,
    # every sequence empty)
    B, Hq = 8192, 64
    need = kvc.decode_workspace_bytes(B, Hq, wl.num_kv_heads, wl.head_dim, 4096)
    assert need > kvc._binding.STATIC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    bt0 = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    cl0 = torch.zeros((B,), dtype=torch.int32, device="cuda")
    lib = kvc.lib()
    import ctypes
    st = lib.kvc_decode_attention_static(cache.handle, 0, ctypes.c_void_p(q.data_ptr()), kvc.BF16,
                                         ctypes.c_void_p(bt0.data_ptr()), 1, ctypes.c_void_p(cl0.data_ptr()), 16, B,
                                         Hq, wl.num_kv_heads, wl.head_dim, 16, float(wl.scale),
                                         ctypes.c_void_p(out.data_ptr()), None, None)
    assert st == kvc._binding.E_WORKSPACE
    assert b"static workspace" in lib.kvc_last_error()
    torch.cuda.synchronize()
    # and the entry point still works afterwards
    s = cache.decode_static(values["q"].cuda().contiguous(), bt, cl, wl.max_context_len, wl.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(s.float()).all()
