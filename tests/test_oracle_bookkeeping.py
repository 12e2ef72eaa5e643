"""Pins for the oracle's sizing, block-table and KV-store models (CPU only)."""
import json
import os
import random

import numpy as np
import pytest

from oracle import blocktable, kvstore, sizing
from oracle.blocktable import BlockTableModel


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# -- sizing: values printed on the pages --------------------------------------

def test_bytes_per_token_page5(golden_dir):
    g = _load(golden_dir, "kv_bytes.json")["per_token_formula"]
    b = sizing.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"], g["dtype"])
    assert b == g["bytes_per_token"] == 147456
    assert b == g["kib_per_token"] * 1024
    one = g["request_tokens"] * b
    assert one == int(g["request_gib"] * 2 ** 30)
    assert g["concurrent_requests"] * one == g["concurrent_gib"] * 2 ** 30
    # the same request held as 16-token blocks needs exactly ceil(8192/16) blocks
    blocks = sizing.blocks_for_tokens(g["request_tokens"], 16)
    assert blocks == 512
    pool = 2 * sizing.pool_bytes(g["num_layers"], blocks, g["num_kv_heads"], g["head_dim"], 16, g["dtype"])
    assert pool == one


def test_bytes_per_token_page3_table(golden_dir):
    g = _load(golden_dir, "kv_bytes.json")["seventy_b_table"]
    per_layer = sizing.kv_bytes_per_token(1, g["num_kv_heads"], g["head_dim"], g["dtype"])
    assert per_layer == g["bytes_per_token_per_layer"] == 32768
    all_layers = sizing.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"], g["dtype"])
    assert all_layers == g["mib_per_token_all_layers"] * 2 ** 20
    assert 4096 * all_layers == g["gib_at_4k"] * 2 ** 30
    assert 32768 * all_layers == g["gib_at_32k"] * 2 ** 30


def test_fp8_halves_bytes():
    assert sizing.kv_bytes_per_token(36, 8, 128, "fp8") * 2 == sizing.kv_bytes_per_token(36, 8, 128, "bf16")


# -- block table: the pages' figures ------------------------------------------

def test_alan_turing_figure(golden_dir):
    g = _load(golden_dir, "paged_figures.json")["alan_turing"]
    bs = g["block_size"]
    bt = BlockTableModel(8, bs, free_order=[5, 1, 7, 0, 3, 6, 2, 4])
    assert bt.allocate(0, 0) == blocktable.OK
    st, slots, cow = bt.append([0], [len(g["tokens"])])
    assert st == blocktable.OK and cow == []
    table = bt.tables[0]
    assert len(table) == len(g["blocks"]) == 3
    # tokens land in logical block p // bs at offset p % bs; the last block is 2/4 full
    words_by_block = [[g["tokens"][p] for p in range(len(g["tokens"])) if p // bs == i] for i in range(3)]
    assert words_by_block == g["blocks"]
    assert bt.lens[0] - (len(table) - 1) * bs == 2
    # physical blocks are non-contiguous and come off the end of the free list
    assert table == [4, 2, 6]
    for p, s in enumerate(slots):
        assert s == table[p // bs] * bs + p % bs
    bt.check_invariants()


def test_shared_prompt_figure_copy_on_write(golden_dir):
    g = _load(golden_dir, "paged_figures.json")["shared_prompt"]
    bs = g["block_size"]
    bt = BlockTableModel(8, bs)
    bt.allocate("A", 0)
    bt.append(["A"], [len(g["prompt"])])
    assert bt.fork("A", "B") == blocktable.OK
    assert bt.tables["A"] == bt.tables["B"]
    assert len(bt.tables["A"]) == len(g["physical_blocks"]) == 2
    assert all(bt.ref[b] == 2 for b in bt.tables["A"])
    bt.check_invariants()
    shared_full, shared_half = bt.tables["A"]
    # first writer into the half-full shared block copies it ...
    st, slots, cow = bt.append(["A"], [1])
    assert st == blocktable.OK
    assert len(cow) == 1 and cow[0][0] == shared_half
    new_blk = cow[0][1]
    assert bt.tables["A"] == [shared_full, new_blk]
    assert slots == [new_blk * bs + 2]
    assert bt.ref[shared_half] == 1 and bt.ref[shared_full] == 2
    # ... and the other sequence then writes in place
    st, slots, cow = bt.append(["B"], [1])
    assert cow == [] and slots == [shared_half * bs + 2]
    bt.check_invariants()


# -- block table: rules restored from page 2's garbled listing -----------------

def test_allocate_oom_is_all_or_nothing():
    bt = BlockTableModel(4, 16)
    assert bt.allocate(1, 40) == blocktable.OK        # 3 blocks
    free_before = list(bt.free)
    assert bt.allocate(2, 17) == blocktable.E_NO_BLOCKS
    assert bt.free == free_before and 2 not in bt.tables
    assert bt.allocate(1, 1) == blocktable.E_SEQ_EXISTS
    assert bt.fork(9, 10) == blocktable.E_NO_SEQ


def test_append_oom_is_atomic_across_the_batch():
    bt = BlockTableModel(3, 4)
    for s in (0, 1):
        bt.allocate(s, 0)
    bt.append([0, 1], [4, 4])                          # 2 blocks used, 1 free
    snap = (dict(bt.lens), {k: list(v) for k, v in bt.tables.items()}, list(bt.free), list(bt.ref))
    st, slots, cow = bt.append([0, 1], [1, 1])         # needs 2 fresh blocks
    assert st == blocktable.E_NO_BLOCKS and slots == [] and cow == []
    assert snap == (dict(bt.lens), {k: list(v) for k, v in bt.tables.items()}, list(bt.free), list(bt.ref))
    st, slots, _ = bt.append([0], [1])                 # exactly exhausts the pool
    assert st == blocktable.OK and bt.free == []


def test_free_returns_blocks_only_at_refcount_zero():
    bt = BlockTableModel(6, 4)
    bt.allocate(0, 0)
    bt.append([0], [6])
    bt.fork(0, 1)
    blocks = list(bt.tables[0])
    bt.free_seq(0)
    assert all(b not in bt.free for b in blocks)
    bt.free_seq(1)
    assert bt.free[-2:] == blocks                      # returned in table order
    bt.check_invariants()
    assert bt.free_seq(1) == blocktable.E_NO_SEQ


def test_truncate_then_reappend_reuses_the_same_slots():
    bt = BlockTableModel(10, 16, free_order=list(np.random.default_rng(0).permutation(10)))
    bt.allocate(0, 0)
    bt.append([0], [32])
    _, s1, _ = bt.append([0], [1])                     # opens a third block
    assert bt.truncate(0, 32) == blocktable.OK
    _, s2, _ = bt.append([0], [1])
    assert s1 == s2
    assert bt.truncate(0, 33) == blocktable.OK and bt.lens[0] == 33
    assert bt.truncate(0, 34) == blocktable.E_INVALID


def test_randomised_operation_sequences_keep_invariants():
    rng = random.Random(1234)
    for trial in range(30):
        bs = rng.choice([1, 4, 16])
        nb = rng.randint(1, 40)
        order = None if trial % 2 else list(np.random.default_rng(trial).permutation(nb))
        bt = BlockTableModel(nb, bs, free_order=order)
        live, nxt = [], 0
        for _ in range(200):
            op = rng.random()
            if op < 0.2 or not live:
                st = bt.allocate(nxt, rng.randint(0, 40))
                if st == blocktable.OK:
                    live.append(nxt)
                nxt += 1
            elif op < 0.35:
                st = bt.fork(rng.choice(live), nxt)
                assert st == blocktable.OK
                live.append(nxt)
                nxt += 1
            elif op < 0.5:
                s = rng.choice(live)
                assert bt.free_seq(s) == blocktable.OK
                live.remove(s)
            elif op < 0.55:
                s = rng.choice(live)
                bt.truncate(s, rng.randint(0, bt.lens[s]))
            elif op < 0.6:
                s = rng.choice(live)
                before = list(bt.tables[s])
                k = rng.randint(0, bt.lens[s])
                assert bt.evict(s, k) == blocktable.OK
                # exactly the blocks wholly before k are gone; the rest are untouched
                for j, b in enumerate(bt.tables[s]):
                    assert b == (-1 if (j + 1) * bs <= k else before[j])
            else:
                k = rng.randint(1, len(live))
                seqs = rng.sample(live, k)
                n_new = [rng.randint(0, 2 * bs + 1) for _ in seqs]
                before = {s: bt.lens[s] for s in seqs}
                st, slots, cow = bt.append(seqs, n_new)
                if st == blocktable.OK:
                    assert len(slots) == sum(n_new)
                    # every written slot is private to its writer after the call
                    for b in {x // bs for x in slots}:
                        assert bt.ref[b] == 1
                    assert len(set(slots)) == len(slots)
                    for s, n in zip(seqs, n_new):
                        assert bt.lens[s] == before[s] + n
                else:
                    assert st == blocktable.E_NO_BLOCKS
                    assert all(bt.lens[s] == before[s] for s in seqs)
            bt.check_invariants()


# -- KV store model -------------------------------------------------------------

def test_kvstore_append_and_gather_are_exact_copies():
    rng = np.random.default_rng(0)
    st = kvstore.KVStoreModel(1, 12, 2, 8, 4, "bf16", free_order=list(rng.permutation(12)))
    for s in range(3):
        st.allocate(s, 0)
    n = [5, 1, 9]
    k = rng.integers(0, 2 ** 16, size=(1, sum(n), 2, 8), dtype=np.uint16) & 0x7F7F
    v = rng.integers(0, 2 ** 16, size=(1, sum(n), 2, 8), dtype=np.uint16) & 0x7F7F
    status, slots, _ = st.append([0, 1, 2], n, k, v)
    assert status == blocktable.OK
    off = 0
    for s, cnt in enumerate(n):
        ks, vs = st.gather(s)
        np.testing.assert_array_equal(ks, kvstore.bits_to_f64(k[0, off:off + cnt], "bf16"))
        np.testing.assert_array_equal(vs, kvstore.bits_to_f64(v[0, off:off + cnt], "bf16"))
        off += cnt


def test_kvstore_cow_keeps_both_histories():
    rng = np.random.default_rng(1)
    st = kvstore.KVStoreModel(2, 8, 1, 4, 4, "f16")
    st.allocate("A", 0)
    base = rng.integers(0, 0x3C00, size=(2, 6, 1, 4), dtype=np.uint16)
    st.append(["A"], [6], base, base)
    st.fork("A", "B")
    ka = rng.integers(0, 0x3C00, size=(2, 1, 1, 4), dtype=np.uint16)
    kb = rng.integers(0, 0x3C00, size=(2, 1, 1, 4), dtype=np.uint16)
    _, _, cow = st.append(["A"], [1], ka, ka)
    assert len(cow) == 1
    st.append(["B"], [1], kb, kb)
    for seq, last in (("A", ka), ("B", kb)):
        for layer in range(2):
            ks, _ = st.gather(seq, layer)
            np.testing.assert_array_equal(ks[:6], kvstore.bits_to_f64(base[layer], "f16"))
            np.testing.assert_array_equal(ks[6], kvstore.bits_to_f64(last[layer, 0], "f16"))


def test_paged_history_is_placement_invariant():
    # The same token rows written under two different physical placements
    # gather back to identical histories (paged == contiguous through the model).
    rng = np.random.default_rng(2)
    k = rng.integers(0, 0x3C00, size=(1, 40, 2, 8), dtype=np.uint16)
    outs = []
    for order in (list(range(16)), list(rng.permutation(16))):
        st = kvstore.KVStoreModel(1, 16, 2, 8, 4, "f16", free_order=order)
        st.allocate(0, 0)
        st.append([0], [40], k, k)
        outs.append(st.gather(0)[0])
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], kvstore.bits_to_f64(k[0], "f16"))


# -- sliding-window eviction ----------------------------------------------------

def test_eviction_keeps_the_cache_bounded():
    # A sequence that keeps generating under a window of w tokens, releasing
    # what leaves the window after every step, never holds more than
    # ceil(w / bs) + 1 blocks, and the blocks it releases serve other sequences.
    bs, w = 4, 10
    bt = BlockTableModel(8, bs)
    assert bt.allocate(0, 0) == blocktable.OK
    for step in range(200):
        assert bt.append([0], [1])[0] == blocktable.OK
        n = bt.lens[0]                                   # the next token sits at position n
        assert bt.evict(0, max(0, n - w + 1)) == blocktable.OK   # it sees positions n - w + 1 .. n
        live = [b for b in bt.tables[0] if b >= 0]
        assert len(live) <= -(-w // bs) + 1
        bt.check_invariants()
    assert len(bt.tables[0]) == -(-200 // bs)             # logical indexing unchanged
    # the released blocks are back on the free list
    assert len(bt.free) == 8 - len([b for b in bt.tables[0] if b >= 0])


def test_evict_fork_and_free_respect_released_entries():
    bs = 4
    bt = BlockTableModel(10, bs)
    bt.allocate(0, 0)
    bt.append([0], [14])                                  # blocks 0..3, last one half full
    assert bt.evict(0, 9) == blocktable.OK                # positions 0..7 gone: blocks 0, 1
    assert bt.tables[0][:2] == [-1, -1]
    assert bt.fork(0, 1) == blocktable.OK                 # shares the two live blocks only
    for b in bt.tables[0][2:]:
        assert bt.ref[b] == 2
    bt.check_invariants()
    assert bt.truncate(1, 6) == blocktable.E_INVALID      # would end inside a released block
    assert bt.truncate(1, 8) == blocktable.OK             # a block boundary is fine
    assert bt.append([1], [1])[0] == blocktable.OK        # position 8: a fresh block after two released
    bt.check_invariants()
    assert bt.free_seq(0) == blocktable.OK and bt.free_seq(1) == blocktable.OK
    assert sorted(bt.free) == list(range(10))
    assert bt.evict(5, 0) == blocktable.E_NO_SEQ
    bt.allocate(2, 0)
    bt.append([2], [3])
    assert bt.evict(2, 4) == blocktable.E_INVALID          # beyond the length
