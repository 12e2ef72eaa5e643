"""Block allocator model: free list, per-sequence block tables, refcounts, CoW.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the ``BlockTable`` class of "大模型推理加速核心KV Cache 复用机制与内存布局优化"
§三 and the ``RequestBlockTable`` of "LLM推理优化实战：从KV-Cache到Continuous
Batching…" §2.2.  The first page's code lost its operators in extraction; the
reading restored here (plainest one the rest of the code supports):

* ``allocate(seq, n)``: needed = ceil(n / block_size); if fewer free blocks
  than needed, fail with nothing taken (the page's "OOM triggers preemption");
  otherwise pop ``needed`` blocks from the END of the free list (``pop()``),
  each with refcount 1.  The page allocates for new sequences; growth of an
  existing one goes through ``append``.
* ``fork(parent, child)``: the child gets a copy of the parent's table (and
  length) and every block's refcount goes up by one; no data moves.  A missing
  parent fails.
* ``free(seq)``: every block of the table, in table order, loses one
  reference; a block whose count reaches 0 is appended to the free list.
* ``append``: position p of a sequence lives in logical block p // block_size
  at offset p % block_size (page 3: ``logical_block_id = num_tokens //
  BLOCK_SIZE``).  The slot written is table[p // bs] * bs + p % bs.  Writing
  into a block that other sequences still reference (refcount > 1) first
  gives this sequence a private block (copy-on-write, page 2 ``fork`` and
  "大模型推理加速——KV Cache篇" §6.1, "copy only when it must be modified"); the
  old block's valid rows are copied only if this sequence has rows in it
  (p % bs > 0).  A position past the last block takes a fresh block.

* ``evict(seq, keep_from)``: the sliding-window / KV-eviction item of
  "苦猿的大模型日记 · Day45" PART 02 (a fixed cache bound bought with the history
  that leaves the window).  Every block of the sequence whose positions all
  lie before ``keep_from`` loses this sequence's reference (freed at 0); its
  table entry becomes -1 so logical indexing is unchanged.  Not on the pages
  as code; released in table order.

Ordering rules (so that physical ids are reproducible bit for bit): sequences
are processed in call order, positions ascending; every new block comes from
``free.pop()`` at the moment it is needed.  ``truncate`` (not on the pages; the
rollback a speculative-decoding verifier or a benchmark needs) releases the
dropped blocks from the last one backwards, so re-appending the same number of
tokens takes the same physical blocks back.  Every failing call leaves the
state exactly as it was.
"""
from __future__ import annotations

import copy

OK = 0
E_INVALID = 1
E_NO_BLOCKS = 3
E_NO_SEQ = 4
E_SEQ_EXISTS = 5


class BlockTableModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if free_order is None:
            self.free = list(range(num_blocks))
        else:
            self.free = [int(x) for x in free_order]
            if sorted(self.free) != list(range(num_blocks)):
                raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.ref = [0] * num_blocks
        self.cow_copies = 0

    # -- page 2 BlockTable -------------------------------------------------
    def allocate(self, seq: int, num_tokens: int) -> int:
        if seq in self.tables:
            return E_SEQ_EXISTS
        if num_tokens < 0:
            return E_INVALID
        needed = (num_tokens + self.block_size - 1) // self.block_size
        if len(self.free) < needed:
            return E_NO_BLOCKS
        blocks = [self.free.pop() for _ in range(needed)]
        for b in blocks:
            self.ref[b] = 1
        self.tables[seq] = blocks
        self.lens[seq] = 0
        return OK

    def fork(self, parent: int, child: int) -> int:
        if parent not in self.tables:
            return E_NO_SEQ
        if child in self.tables:
            return E_SEQ_EXISTS
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            if b >= 0:
                self.ref[b] += 1
        return OK

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return E_NO_SEQ
        for b in self.tables[seq]:
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lens[seq]
        return OK

    # -- growth ------------------------------------------------------------
    def append(self, seqs, n_new=None):
        """Reserve slots for n_new[i] new tokens of seqs[i].

        Returns (status, slots, cow_pairs).  ``slots`` lists the slot of every
        new token, sequence by sequence in call order, positions ascending;
        ``cow_pairs`` lists (src_block, dst_block) copies in the order issued.
        On failure the state is unchanged and slots/cow_pairs are empty.
        """
        seqs = list(seqs)
        if n_new is None:
            n_new = [1] * len(seqs)
        n_new = [int(x) for x in n_new]
        if len(n_new) != len(seqs) or any(x < 0 for x in n_new):
            return E_INVALID, [], []
        if len(set(seqs)) != len(seqs):
            return E_INVALID, [], []
        for s in seqs:
            if s not in self.tables:
                return E_NO_SEQ, [], []
        saved = (copy.deepcopy(self.tables), dict(self.lens), list(self.free),
                 list(self.ref), self.cow_copies)
        bs = self.block_size
        slots, cow = [], []
        for s, n in zip(seqs, n_new):
            table = self.tables[s]
            for p in range(self.lens[s], self.lens[s] + n):
                idx, off = divmod(p, bs)
                if idx == len(table):
                    if not self.free:
                        self._restore(saved)
                        return E_NO_BLOCKS, [], []
                    b = self.free.pop()
                    self.ref[b] = 1
                    table.append(b)
                elif table[idx] < 0:
                    self._restore(saved)
                    return E_INVALID, [], []
                elif self.ref[table[idx]] > 1:
                    if not self.free:
                        self._restore(saved)
                        return E_NO_BLOCKS, [], []
                    old = table[idx]
                    b = self.free.pop()
                    self.ref[b] = 1
                    self.ref[old] -= 1
                    table[idx] = b
                    if off > 0:
                        cow.append((old, b))
                        self.cow_copies += 1
                slots.append(table[idx] * bs + off)
            self.lens[s] += n
        return OK, slots, cow

    def truncate(self, seq: int, num_tokens: int) -> int:
        if seq not in self.tables:
            return E_NO_SEQ
        if num_tokens < 0 or num_tokens > self.lens[seq]:
            return E_INVALID
        table = self.tables[seq]
        if num_tokens % self.block_size and table[num_tokens // self.block_size] < 0:
            return E_INVALID                            # the next write would land in a released block
        keep = (num_tokens + self.block_size - 1) // self.block_size
        for b in reversed(table[keep:]):
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del table[keep:]
        self.lens[seq] = num_tokens
        return OK

    def evict(self, seq: int, keep_from: int) -> int:
        """Release the blocks of ``seq`` that hold only positions < keep_from."""
        if seq not in self.tables:
            return E_NO_SEQ
        if keep_from < 0 or keep_from > self.lens[seq]:
            return E_INVALID
        table = self.tables[seq]
        for j in range(keep_from // self.block_size):
            b = table[j]
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            table[j] = -1
        return OK

    def _restore(self, saved):
        self.tables, self.lens, self.free, self.ref, self.cow_copies = saved

    # -- queries -----------------------------------------------------------
    def export(self, seqs, max_blocks: int):
        """Block-table rows padded with -1, and the lengths, for ``seqs``."""
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def check_invariants(self):
        """Raise AssertionError if the bookkeeping is inconsistent."""
        count = [0] * self.num_blocks
        for s, t in self.tables.items():
            live = [b for b in t if b >= 0]
            assert len(set(live)) == len(live), "block repeated inside one table"
            assert self.lens[s] <= len(t) * self.block_size, "length beyond capacity"
            first_live = next((j for j, b in enumerate(t) if b >= 0), len(t))
            assert all(b >= 0 for b in t[first_live:]), "released entry after a live one"
            for b in live:
                count[b] += 1
        assert count == self.ref, "refcount != number of tables holding the block"
        assert len(set(self.free)) == len(self.free), "block twice in the free list"
        for b in self.free:
            assert self.ref[b] == 0, "free block still referenced"
        used = {b for b in range(self.num_blocks) if self.ref[b] > 0}
        assert used.isdisjoint(self.free)
        assert len(used) + len(self.free) == self.num_blocks, "block leaked"
