"""CPU oracle for paged GQA decode attention and its KV-cache bookkeeping.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no common kernels, headers, helpers, tables or generators).

The oracle is deliberately plain and slow: fp64 NumPy for the floating-point
results, plain Python for the bookkeeping, and float32 NumPy only where the
method's fp8 storage step is itself defined in float32 (see ``fp8_policy``).

Modules and the passages each follows (pages are cited by title and section):

* ``attention`` -- decode attention softmax(q K^T * scale) V per query head over
  a contiguously gathered history, GQA head grouping, the multi-token causal
  form (several new tokens per sequence), and a brute-force full causal
  attention used to pin them.
* ``blocktable`` -- the block allocator: free list, per-sequence tables,
  refcounts, copy-on-write fork, slot mapping for appends.
* ``e4m3`` -- the OCP 8-bit float E4M3 ("FN") format, decode and round-to-
  nearest-even encode, written from the format definition.
* ``fp8_policy`` -- the per-(block, KV head) scale rule used when fp8 KV is
  written.  Parity unpinned by the pages (they name FP8/E4M3 KV but give no
  scale rule): the rule is a reading, whose rendering here is pinned by
  invariants and by hand-worked codes and scales.
* ``int8_policy`` -- the same kind of scale rule for a symmetric int8 code
  (round half to even, clamp to +-127).  Parity unpinned by the pages (they
  list INT8 KV quantisation but give no scheme): a reading, pinned like fp8's.
* ``sizing`` -- the KV bytes-per-token formula and pool sizes.
"""
