"""GPU parity of the shared-prefix (cascade) decode: kvc_decode_attention with
opts.shared_prefix = P (every sequence forked from one P-token prefix) against
the oracle's decode attention over all rows, per element within
|gpu - ref| <= 2e-3 + 1e-2 |ref| (fp8 / int8 against the stored values), and
close to the plain decode of the same step.

Cases: the scaled-down shared-prefix workload in every cache dtype; head
groupings from MHA to 16 query heads per KV head; batches whose queries fill
one, several and a partial prefix work-group (32-column tiles of (sequence,
head) pairs, four per group); prefixes of one block and of many (the prefix
pass cut into pieces); own rows of one token, within a block, across blocks;
forced splits of the own rows over many waves; and the options the mode
rejects.
"""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_split_amd as kvc
from conftest import gpu_available
from harness import (check_close, decode_poisoned, gpu_decode_again, gpu_setup, gpu_step, oracle_decode, oracle_run,
                     to_f64)
from workloads import custom_workload, make_values, make_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = (2e-3, 1e-2)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(wl, **split):
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    plain, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    ref = oracle_decode(st, wl, values)
    o = gpu_decode_again(cache, wl, values, bt, cl, kernel=2, shared_prefix=wl.shared_prefix, **split)
    torch.cuda.synchronize()
    return o, plain, ref


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8", "int8"])
def test_shared_prefix_workload(kv):
    wl = make_workload(4, small=True, kv_dtype=kv)
    _say(f"[cascade] {wl.name}")
    o, plain, ref = _run(wl)
    check_close(to_f64(o), ref, *TOL, f"cascade {kv}")
    check_close(to_f64(o), to_f64(plain), 4e-3, 2e-2, f"cascade vs plain decode {kv}")


@pytest.mark.parametrize("hq,hkv,d,B,P", [(8, 2, 128, 40, 16), (16, 1, 64, 3, 512), (32, 8, 128, 9, 64),
                                          (12, 3, 64, 70, 256), (4, 4, 128, 5, 1024), (16, 16, 64, 33, 48)])
def test_shapes(hq, hkv, d, B, P):
    rng = np.random.default_rng(hq * 31 + B)
    own = rng.choice([0, 1, 5, 15, 16, 17, 40, 200], size=B)   # rows past the prefix before the step
    lens = P + own
    wl = custom_workload(B, hq, hkv, d, "bf16", lens, seed=B + P, shared_prefix=P, name="cascade shapes")
    _say(f"[cascade] heads {hq}/{hkv} D{d} B{B} prefix {P}")
    o, plain, ref = _run(wl)
    check_close(to_f64(o), ref, *TOL, f"cascade {hq}/{hkv} D{d} B{B} P{P}")


@pytest.mark.parametrize("wi", [1, 3, 100])
def test_own_rows_split_over_waves(wi):
    lens = [128 + x for x in (0, 3, 300, 16, 33, 1)]
    wl = custom_workload(len(lens), 16, 4, 128, "fp8", lens, seed=7, shared_prefix=128, name="cascade splits")
    o, plain, ref = _run(wl, work_items=wi)
    check_close(to_f64(o), ref, *TOL, f"cascade work_items {wi}")


def test_options_the_mode_rejects():
    lens = [64 + 5, 64 + 20]
    wl = custom_workload(len(lens), 8, 2, 128, "bf16", lens, seed=3, shared_prefix=64, name="cascade options")
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    _, bt, cl = gpu_step(cache, wl, values)
    q = values["q"].cuda().contiguous()
    for bad in (dict(shared_prefix=40), dict(shared_prefix=-16), dict(shared_prefix=64, window=32),
                dict(shared_prefix=64, kernel=1), dict(shared_prefix=64, pool_pieces=2),
                dict(shared_prefix=16 * bt.shape[1])):
        with pytest.raises(kvc.KvcError):
            decode_poisoned(cache, q, bt, cl, wl.max_context_len, wl.scale, **bad)
    assert kvc.decode_workspace_bytes(2, 8, 2, 128, 100, shared_prefix=40) == 0
    assert kvc.decode_workspace_bytes(2, 8, 2, 128, 100, shared_prefix=64) > \
        kvc.decode_workspace_bytes(2, 8, 2, 128, 100)


def test_layers_of_a_multi_layer_pool():
    # the prefix pass and the own-rows decode read the requested layer's tiles
    import dataclasses
    lens = [96 + x for x in (1, 17, 40, 0, 65)]
    wl = dataclasses.replace(custom_workload(len(lens), 16, 4, 128, "bf16", lens, seed=41, shared_prefix=96,
                                             name="cascade layers"), num_layers=3)
    _say(f"[cascade] {wl.num_layers} layers")
    values = make_values(wl, "cpu")
    st = oracle_run(wl, values)
    cache = gpu_setup(wl, values)
    _, bt, cl = gpu_step(cache, wl, values)
    for layer in (0, 2):
        o = gpu_decode_again(cache, wl, values, bt, cl, kernel=2, shared_prefix=96, layer=layer)
        torch.cuda.synchronize()
        check_close(to_f64(o), oracle_decode(st, wl, values, layer=layer), *TOL, f"cascade layer {layer}")


def test_batch_breaking_the_prefix_conditions():
    # sequences 0-2 share a 64-token prefix; sequence 10 has its own blocks.
    # Decoding [0, 1, 10] with shared_prefix = 64 gives sequence 10 NaN rows
    # (its table does not start with the prefix blocks) and the others their
    # plain decode; with seq_ids the library refuses the batch before launch.
    lens = [64 + 5, 64 + 20, 64 + 30]
    wl = custom_workload(len(lens), 8, 2, 128, "bf16", lens, seed=12, shared_prefix=64, name="cascade misuse")
    wl.num_blocks += 8
    wl.free_order = np.random.default_rng(3).permutation(wl.num_blocks).astype(np.int32)
    values = make_values(wl, "cpu")
    cache = gpu_setup(wl, values)
    gen = torch.Generator().manual_seed(5)
    rows = torch.randn((1, 100, 2, 128), generator=gen).to(torch.bfloat16).cuda()
    cache.add_seq(10, 0)
    cache.append([10], rows, rows.flip(1).contiguous(), n_new=[100])
    seqs = [0, 1, 10]
    new = torch.randn((1, 3, 2, 128), generator=gen).to(torch.bfloat16).cuda()
    cache.append(seqs, new, new.neg().contiguous())
    bt, cl = cache.export_tables(seqs)
    q = torch.randn((3, 8, 128), generator=gen).to(torch.bfloat16).cuda()
    plain = decode_poisoned(cache, q, bt, cl, int(cl.max()), wl.scale, kernel=2)
    casc = decode_poisoned(cache, q, bt, cl, int(cl.max()), wl.scale, kernel=2, shared_prefix=64)
    torch.cuda.synchronize()
    check_close(to_f64(casc[:2]), to_f64(plain[:2]), 4e-3, 2e-2, "sequences that share the prefix")
    assert torch.isnan(casc[2].float()).all(), "a sequence outside the prefix must get NaN rows"
    with pytest.raises(kvc.KvcError) as e:
        decode_poisoned(cache, q, bt, cl, int(cl.max()), wl.scale, kernel=2, shared_prefix=64, seq_ids=seqs)
    assert "does not share" in str(e.value)
    ok = decode_poisoned(cache, q[:2].contiguous(), bt[:2].contiguous(), cl[:2].contiguous(), int(cl.max()),
                         wl.scale, kernel=2, shared_prefix=64, seq_ids=[0, 1])
    torch.cuda.synchronize()
    check_close(to_f64(ok), to_f64(plain[:2]), 4e-3, 2e-2, "checked batch")
