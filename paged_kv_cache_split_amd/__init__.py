"""Paged KV cache and split-K paged GQA decode attention for MI355X (gfx950).

The work is done by libkvc (C ABI in include/kvc.h): a host block allocator
with refcounted copy-on-write and hand-written HIP kernels for the append,
the split-K decode (one new token per sequence, or several with a causal
mask among them) and the merge.  This package is its ctypes binding; torch
provides device memory and streams.  Importing it fails if libkvc.so has not
been built (``python paged_kv_cache_split_amd/build.py``).
"""
from ._binding import (BF16, F16, F32, FP8, INT8, KVCache, KvcError, Scheduler, bytes_per_token,  # noqa: F401
                       decode_workspace_bytes, extend_workspace_bytes, lib, pool_bytes, scale_bytes,
                       scratch_bytes, stream_copy, stream_read)
from ._binding import LIB_PATH, SYMBOLS  # noqa: F401
