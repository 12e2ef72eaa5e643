"""Logical model of the stored KV cache: what every physical block must hold.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A ``KVStoreModel`` owns a ``BlockTableModel`` and, per physical block, the
stored rows of every (layer, KV head, slot) -- raw bit patterns for the 16/32-
bit dtypes (writes are plain copies, so the expected contents are the input
bits), E4M3 codes plus one fp32 scale per (layer, KV head) for fp8 (written
with ``fp8_policy``), int8 codes plus the same scales for int8 (``int8_policy``).  It knows nothing about how the device lays blocks out in
memory; tests map device memory onto (block, layer, head, slot, dim) through
the pool layout the library's header documents.

Append = reserve slots (``BlockTableModel.append``), do the copy-on-write
copies it lists (whole blocks, all layers, scales included), then write each
new row into its slot ("苦猿的大模型日记 · Day45" PART 02: compute only the new
token's K/V and add it to the cache; "大模型推理加速——KV Cache篇" §3: the cache is
written at [start_pos : start_pos + seqlen] and read back over
[: start_pos + seqlen]).
"""
from __future__ import annotations

import numpy as np

from . import blocktable, e4m3, fp8_policy, int8_policy

QUANTISED = {"fp8": fp8_policy, "int8": int8_policy}

BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8, "int8": np.uint8}


def bits_to_f64(bits, dtype: str) -> np.ndarray:
    """Real values of raw storage bits (exact)."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


class KVStoreModel:
    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, block_size,
                 kv_dtype, free_order=None, in_dtype=None):
        self.L, self.N, self.H, self.D, self.bs = num_layers, num_blocks, num_kv_heads, head_dim, block_size
        self.kv_dtype = kv_dtype
        self.in_dtype = in_dtype or (kv_dtype if kv_dtype not in QUANTISED else "bf16")
        self.tables = blocktable.BlockTableModel(num_blocks, block_size, free_order)
        shape = (num_blocks, num_layers, num_kv_heads, block_size, head_dim)
        self.k = np.zeros(shape, dtype=BITS_DTYPE[kv_dtype])
        self.v = np.zeros(shape, dtype=BITS_DTYPE[kv_dtype])
        self.written = np.zeros((num_blocks, block_size), dtype=bool)
        if kv_dtype in QUANTISED:
            self.k_scale = np.zeros((num_blocks, num_layers, num_kv_heads), dtype=np.float32)
            self.v_scale = np.zeros((num_blocks, num_layers, num_kv_heads), dtype=np.float32)

    # bookkeeping pass-throughs
    def allocate(self, seq, n):
        return self.tables.allocate(seq, n)

    def fork(self, parent, child):
        return self.tables.fork(parent, child)

    def free_seq(self, seq):
        return self.tables.free_seq(seq)

    def evict(self, seq, keep_from):
        return self.tables.evict(seq, keep_from)

    def truncate(self, seq, n):
        return self.tables.truncate(seq, n)

    def append(self, seqs, n_new, k_new_bits, v_new_bits):
        """k_new_bits/v_new_bits: [L, T, Hkv, D] raw input bits (in_dtype),
        rows ordered sequence by sequence, positions ascending."""
        lens_before = {s: self.tables.lens.get(s) for s in seqs}
        status, slots, cow = self.tables.append(seqs, n_new)
        if status != blocktable.OK:
            return status, [], []
        for src, dst in cow:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]
            self.written[dst] = self.written[src]
            if self.kv_dtype in QUANTISED:
                self.k_scale[dst] = self.k_scale[src]
                self.v_scale[dst] = self.v_scale[src]
        k_new_bits = np.asarray(k_new_bits)
        v_new_bits = np.asarray(v_new_bits)
        if self.kv_dtype not in QUANTISED:
            for t, slot in enumerate(slots):
                blk, off = divmod(slot, self.bs)
                self.k[blk, :, :, off, :] = k_new_bits[:, t]
                self.v[blk, :, :, off, :] = v_new_bits[:, t]
                self.written[blk, off] = True
            return status, slots, cow
        # fp8 / int8: one scale update per (block, layer, head) per run of rows in a block
        policy = QUANTISED[self.kv_dtype]
        kx = bits_to_f64(k_new_bits, self.in_dtype).astype(np.float32)
        vx = bits_to_f64(v_new_bits, self.in_dtype).astype(np.float32)
        t = 0
        for s, n in zip(seqs, n_new if n_new is not None else [1] * len(seqs)):
            p0 = lens_before[s]
            i = 0
            while i < n:
                slot = slots[t + i]
                blk, off = divmod(slot, self.bs)
                run = min(n - i, self.bs - off)
                for layer in range(self.L):
                    for h in range(self.H):
                        for pool, scales, x in ((self.k, self.k_scale, kx), (self.v, self.v_scale, vx)):
                            held = pool[blk, layer, h, :off, :]
                            held2, new_codes, s_new = policy.write_rows(
                                held, scales[blk, layer, h], x[layer, t + i:t + i + run, h, :])
                            pool[blk, layer, h, :off, :] = held2
                            pool[blk, layer, h, off:off + run, :] = new_codes
                            scales[blk, layer, h] = s_new
                self.written[blk, off:off + run] = True
                i += run
            t += n
            assert p0 is not None
        return status, slots, cow

    # logical views
    def gather(self, seq, layer=0, start=0):
        """Stored K/V of one sequence in position order, as fp64 values
        (dequantised for fp8 and int8): ([n, Hkv, D], [n, Hkv, D]).  Positions before
        ``start`` (released by eviction, say) are returned as zeros."""
        n = self.tables.lens[seq]
        table = np.asarray(self.tables.tables[seq], dtype=np.int64)
        ks = np.zeros((n, self.H, self.D))
        vs = np.zeros((n, self.H, self.D))
        pos = np.arange(start, n)
        blk, off = table[pos // self.bs], pos % self.bs      # the slot of every position
        assert np.all(blk >= 0), "position inside a released block"
        if self.kv_dtype in QUANTISED:
            dec = e4m3.decode_array if self.kv_dtype == "fp8" else int8_policy.decode_array
            ks[start:] = dec(self.k[blk, layer, :, off, :]) * self.k_scale[blk, layer, :, None].astype(np.float64)
            vs[start:] = dec(self.v[blk, layer, :, off, :]) * self.v_scale[blk, layer, :, None].astype(np.float64)
        else:
            ks[start:] = bits_to_f64(self.k[blk, layer, :, off, :], self.kv_dtype)
            vs[start:] = bits_to_f64(self.v[blk, layer, :, off, :], self.kv_dtype)
        return ks, vs
