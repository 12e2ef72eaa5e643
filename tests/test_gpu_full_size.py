"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (automatic partition size and kernel choice).

The whole batch runs on the GPU; the oracle checks every sequence of
configs 2-4 and 16 sequences of config 5 (first, last, shortest, longest and
twelve spread over the batch; most of them straddle a boundary between two
waves' chunks in the launch the benchmark times) one by one: its own
single-sequence store replays that sequence's writes (history in one append,
then the new token) and the fp64 decode runs on the stored values.  Block
tables of every sequence are checked bit-exactly against the oracle's
allocator model.  The workload with a shared prefix is also decoded with the
prefix attended once for the batch and checked on the same sequences.
"""
import sys

import numpy as np
import pytest
import torch

from conftest import gpu_available
from harness import (check_close, decode_poisoned, gpu_setup, gpu_step, logical_history, read_pools, to_bits, to_f64,
                     _history_rows)
from workloads import make_values, make_workload, setup_ops

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _oracle_single(wl, values, b):
    """Oracle store holding sequence b alone, written the way the GPU wrote it."""
    from oracle.kvstore import KVStoreModel
    L = int(wl.context_lens[b])
    nblk = (L + 1 + 15) // 16
    st = KVStoreModel(1, nblk, wl.num_kv_heads, wl.head_dim, 16, wl.kv_dtype, in_dtype=wl.new_dtype)
    st.allocate(0, 0)
    rows = _history_rows(wl, b)
    kb = to_bits(values["k_hist"][:, rows.to(values["k_hist"].device)], wl.new_dtype)
    vb = to_bits(values["v_hist"][:, rows.to(values["v_hist"].device)], wl.new_dtype)
    splits = [wl.shared_prefix, L - wl.shared_prefix] if wl.shared_prefix else [L]
    r0 = 0
    for n in splits:
        assert st.append([0], [n], kb[:, r0:r0 + n], vb[:, r0:r0 + n])[0] == 0
        r0 += n
    assert st.append([0], [1], to_bits(values["k_new"][:, b:b + 1], wl.new_dtype),
                     to_bits(values["v_new"][:, b:b + 1], wl.new_dtype))[0] == 0
    return st


def _straddlers(wl, W):
    """Sequences whose blocks fall in more than one chunk of the even split of
    the batch's blocks over W waves per KV head."""
    from score_walk import decode_chunks
    seen = {}
    for b, _, _ in decode_chunks(wl.attend_lens, W):
        seen[b] = seen.get(b, 0) + 1
    return {b for b, c in seen.items() if c > 1}


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_every_sequence(cid):
    from oracle.attention import decode_attention
    from oracle.blocktable import BlockTableModel
    wl = make_workload(cid)
    _say(f"[full] config {cid}: {wl.name}; {int(wl.attend_lens.sum())} tokens, {wl.num_blocks} blocks")
    values = make_values(wl, "cuda")
    cache = gpu_setup(wl, values)
    out, bt, cl = gpu_step(cache, wl, values)
    torch.cuda.synchronize()
    # tables of every sequence, bit-exact
    model = BlockTableModel(wl.num_blocks, 16, wl.free_order)
    row = 0
    for op in setup_ops(wl):
        if op[0] == "add":
            model.allocate(op[1], op[2])
        elif op[0] == "fork":
            model.fork(op[1], op[2])
        else:
            assert model.append(op[1], op[2])[0] == 0
    assert model.append(list(range(wl.batch)))[0] == 0
    rows, lens = model.export(list(range(wl.batch)), bt.shape[1])
    assert np.array_equal(bt.cpu().numpy(), np.array(rows, dtype=np.int32))
    assert np.array_equal(cl.cpu().numpy(), np.array(lens, dtype=np.int32))
    # every sequence (config 5: 16 of them)
    L = wl.context_lens
    if cid == 5:
        spread = np.linspace(1, wl.batch - 2, 12).astype(int).tolist()
        sample = sorted({0, wl.batch - 1, int(np.argmin(L)), int(np.argmax(L))} | set(spread))
    else:
        sample = list(range(wl.batch))
    straddle = _straddlers(wl, 1024 // wl.num_kv_heads) & set(sample)
    _say(f"  checking {len(sample)} sequences, {len(straddle)} of them across a chunk boundary")
    if cid in (3, 5):
        assert len(straddle) >= 8
    pools = read_pools(cache)
    q = to_f64(values["q"])
    got_all = to_f64(out)
    got_sp = None
    if wl.shared_prefix:   # the same step with the shared prefix attended once for the batch
        o_sp = decode_poisoned(cache, values["q"].contiguous(), bt, cl, wl.max_context_len, wl.scale, kernel=2,
                            shared_prefix=wl.shared_prefix)
        torch.cuda.synchronize()
        got_sp = to_f64(o_sp)
    for b in sample:
        st = _oracle_single(wl, values, b)
        # stored rows of b, bit-exact, through its exported table
        tab = rows[b]
        for i, blk in enumerate(st.tables.tables[0]):
            assert np.array_equal(pools["k"][tab[i]], st.k[blk]), f"seq {b} block {i} K"
            assert np.array_equal(pools["v"][tab[i]], st.v[blk]), f"seq {b} block {i} V"
            if wl.kv_dtype in ("fp8", "int8"):
                assert np.array_equal(pools["k_scale"][tab[i]].view(np.uint32), st.k_scale[blk].view(np.uint32))
                assert np.array_equal(pools["v_scale"][tab[i]].view(np.uint32), st.v_scale[blk].view(np.uint32))
        k, v = st.gather(0)
        ref = decode_attention(q[b], k, v, wl.scale)
        ma, mr = check_close(got_all[b], ref, 2e-3, 1e-2, f"config {cid} seq {b}")
        msg = f"  seq {b} (L={int(L[b])}): max_abs {ma:.2e} max_rel {mr:.2e}"
        if got_sp is not None:
            ma3, _ = check_close(got_sp[b], ref, 2e-3, 1e-2, f"config {cid} seq {b} shared prefix")
            msg += f"; shared prefix max_abs {ma3:.2e}"
        if wl.kv_dtype in ("fp8", "int8"):
            ku, vu = logical_history(wl, values, b)
            ma2, _ = check_close(got_all[b], decode_attention(q[b], ku, vu, wl.scale), 5e-2, 1e-2,
                                 f"config {cid} seq {b} vs unquantised rows")
            msg += f"; vs unquantised rows max_abs {ma2:.2e}"
        _say(msg)
