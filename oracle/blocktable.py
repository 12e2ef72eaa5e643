"""Block allocator model: free list, per-sequence block tables, refcounts, CoW.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it models.  "大模型推理加速核心KV Cache 复用机制与内存布局优化" §三 (a block
table over a shared pool: whole blocks per sequence, a free list, reference
counts so forks share blocks) and "LLM推理优化实战：从KV-Cache到Continuous
Batching…" §2.2 (the per-request table that maps a position to its block).
The first page's listing lost its operators in extraction; the plainest
reading its surrounding text supports is taken, and written here as state
transitions of our own:

State: ``free`` (a stack: new blocks come off its end, released ones go on its
end), ``ref`` (references per physical block), ``tables`` (sequence -> list of
physical ids, -1 for a released entry) and ``lens`` (tokens per sequence).

Every operation is a sequence of three primitive moves, each logged in a
journal so that a failing operation is rolled back to the exact prior state:

* TAKE: pop a block off the free stack with one reference (fails with
  E_NO_BLOCKS on an empty stack);
* SHARE: one more reference to a live block;
* DROP: one reference less; at zero the block goes back on the free stack.

The operations, as sequences of moves:

* ``allocate(seq, n)``: a new sequence with ceil(n / block_size) TAKEs; the
  count is checked first, so a pool that cannot hold the sequence leaves
  everything untouched (the page's out-of-blocks case is left to the caller,
  a scheduler that preempts).  Its length starts at 0: rows arrive through
  ``append``.
* ``fork(parent, child)``: the child's table is a copy of the parent's, with a
  SHARE of every live entry in table order; the length is copied; no data
  moves.
* ``free_seq(seq)``: a DROP of every live entry in table order.
* ``append(seqs, n_new)``: position p of a sequence is slot p % block_size of
  its logical block p // block_size.  Sequences in call order, positions
  ascending: a position one past the table's end TAKEs a block; a position in
  a block other tables still hold (ref > 1) first TAKEs a private block for
  this sequence and DROPs the shared one (copy-on-write, the first page's
  sharing and "大模型推理加速——KV Cache篇" §6.1); the rows already there are copied
  only when the sequence has some in that block (p % block_size > 0).
* ``evict(seq, keep_from)``: a DROP of every block whose positions all lie
  before keep_from, in table order, its entry set to -1 so logical indexing
  does not move (the sliding-window bound of "苦猿的大模型日记 · Day45" PART 02).
* ``truncate(seq, n)``: DROPs of the blocks past the first ceil(n /
  block_size), last one first, so appending the same tokens again takes the
  same physical blocks back (the rollback a speculative verifier needs; not on
  the pages).

The order of moves fixes every physical id, so the library's tables can be
compared with these bit for bit.
"""
from __future__ import annotations

OK = 0
E_INVALID = 1
E_NO_BLOCKS = 3
E_NO_SEQ = 4
E_SEQ_EXISTS = 5


class _Abort(Exception):
    def __init__(self, status):
        super().__init__(status)
        self.status = status


class BlockTableModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(self.free) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.ref = [0] * num_blocks
        self.cow_copies = 0
        self._log = None          # the running operation's journal of undo actions

    # -- moves (each logs how to undo itself) ------------------------------
    def _take(self) -> int:
        if not self.free:
            raise _Abort(E_NO_BLOCKS)
        b = self.free.pop()
        self.ref[b] = 1

        def undo():
            self.ref[b] = 0
            self.free.append(b)
        self._log.append(undo)
        return b

    def _share(self, b: int):
        self.ref[b] += 1
        self._log.append(lambda: self.ref.__setitem__(b, self.ref[b] - 1))

    def _drop(self, b: int):
        self.ref[b] -= 1
        released = self.ref[b] == 0
        if released:
            self.free.append(b)

        def undo():
            if released:
                self.free.pop()
            self.ref[b] += 1
        self._log.append(undo)

    def _set(self, store: dict, key, value):
        """Assign store[key] (a missing key is removed again on undo)."""
        had, old = key in store, store.get(key)
        store[key] = value

        def undo():
            if had:
                store[key] = old
            else:
                del store[key]
        self._log.append(undo)

    def _forget(self, store: dict, key):
        old = store.pop(key)
        self._log.append(lambda: store.__setitem__(key, old))

    def _entry(self, table: list, idx: int, value: int):
        """table[idx] = value, or a push when idx is one past the end."""
        if idx == len(table):
            table.append(value)
            self._log.append(table.pop)
        else:
            old = table[idx]
            table[idx] = value
            self._log.append(lambda: table.__setitem__(idx, old))

    def _count_copy(self):
        self.cow_copies += 1
        self._log.append(lambda: setattr(self, "cow_copies", self.cow_copies - 1))

    def _run(self, body):
        """Run one operation; on failure undo its moves in reverse order."""
        self._log = []
        try:
            return body()
        except _Abort as a:
            for undo in reversed(self._log):
                undo()
            return a.status
        finally:
            self._log = None

    def _live(self, seq):
        if seq not in self.tables:
            raise _Abort(E_NO_SEQ)
        return self.tables[seq]

    # -- operations --------------------------------------------------------
    def allocate(self, seq: int, num_tokens: int) -> int:
        def body():
            if seq in self.tables:
                raise _Abort(E_SEQ_EXISTS)
            if num_tokens < 0:
                raise _Abort(E_INVALID)
            count = -(-num_tokens // self.block_size)
            if count > len(self.free):
                raise _Abort(E_NO_BLOCKS)
            self._set(self.tables, seq, [])
            self._set(self.lens, seq, 0)
            for j in range(count):
                self._entry(self.tables[seq], j, self._take())
            return OK
        return self._run(body)

    def fork(self, parent: int, child: int) -> int:
        def body():
            src = self._live(parent)
            if child in self.tables:
                raise _Abort(E_SEQ_EXISTS)
            self._set(self.tables, child, src[:])
            self._set(self.lens, child, self.lens[parent])
            for b in src:
                if b >= 0:
                    self._share(b)
            return OK
        return self._run(body)

    def free_seq(self, seq: int) -> int:
        def body():
            for b in self._live(seq):
                if b >= 0:
                    self._drop(b)
            self._forget(self.tables, seq)
            self._forget(self.lens, seq)
            return OK
        return self._run(body)

    def append(self, seqs, n_new=None):
        """Reserve slots for n_new[i] new tokens of seqs[i].

        Returns (status, slots, cow_pairs).  ``slots`` lists the slot of every
        new token, sequence by sequence in call order, positions ascending;
        ``cow_pairs`` lists (src_block, dst_block) copies in the order issued.
        On failure the state is unchanged and slots/cow_pairs are empty.
        """
        seqs = list(seqs)
        counts = [1] * len(seqs) if n_new is None else [int(x) for x in n_new]
        slots, pairs = [], []

        def body():
            if len(counts) != len(seqs) or min(counts, default=0) < 0 or len(set(seqs)) != len(seqs):
                raise _Abort(E_INVALID)
            for s in seqs:
                self._live(s)
            bs = self.block_size
            for s, n in zip(seqs, counts):
                table = self.tables[s]
                start = self.lens[s]
                for p in range(start, start + n):
                    j, off = p // bs, p % bs
                    if j == len(table):
                        self._entry(table, j, self._take())
                    elif table[j] < 0:
                        raise _Abort(E_INVALID)          # a released block cannot take rows
                    elif self.ref[table[j]] > 1:
                        shared = table[j]
                        own = self._take()
                        self._drop(shared)
                        self._entry(table, j, own)
                        if off:
                            pairs.append((shared, own))
                            self._count_copy()
                    slots.append(table[j] * bs + off)
                self._set(self.lens, s, start + n)
            return OK
        st = self._run(body)
        return (st, slots, pairs) if st == OK else (st, [], [])

    def truncate(self, seq: int, num_tokens: int) -> int:
        def body():
            table = self._live(seq)
            if not 0 <= num_tokens <= self.lens[seq]:
                raise _Abort(E_INVALID)
            bs = self.block_size
            if num_tokens % bs and table[num_tokens // bs] < 0:
                raise _Abort(E_INVALID)                  # the next write would land in a released block
            keep = -(-num_tokens // bs)
            while len(table) > keep:
                b = table[-1]
                if b >= 0:
                    self._drop(b)
                table.pop()
                self._log.append(lambda b=b, t=table: t.append(b))
            self._set(self.lens, seq, num_tokens)
            return OK
        return self._run(body)

    def evict(self, seq: int, keep_from: int) -> int:
        """Release the blocks of ``seq`` that hold only positions < keep_from."""
        def body():
            table = self._live(seq)
            if not 0 <= keep_from <= self.lens[seq]:
                raise _Abort(E_INVALID)
            for j in range(keep_from // self.block_size):
                if table[j] >= 0:
                    self._drop(table[j])
                    self._entry(table, j, -1)
            return OK
        return self._run(body)

    # -- queries -----------------------------------------------------------
    def export(self, seqs, max_blocks: int):
        """Block-table rows padded with -1, and the lengths, for ``seqs``."""
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def check_invariants(self):
        """Raise AssertionError if the bookkeeping is inconsistent."""
        held = [0] * self.num_blocks
        for s, t in self.tables.items():
            live = [b for b in t if b >= 0]
            assert len(set(live)) == len(live), "block repeated inside one table"
            assert self.lens[s] <= len(t) * self.block_size, "length beyond capacity"
            first_live = next((j for j, b in enumerate(t) if b >= 0), len(t))
            assert all(b >= 0 for b in t[first_live:]), "released entry after a live one"
            for b in live:
                held[b] += 1
        assert held == self.ref, "refcount != number of tables holding the block"
        assert len(set(self.free)) == len(self.free), "block twice in the free list"
        assert all(self.ref[b] == 0 for b in self.free), "free block still referenced"
        in_use = sum(1 for r in self.ref if r > 0)
        assert in_use + len(self.free) == self.num_blocks, "block leaked"
