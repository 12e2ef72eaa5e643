"""ctypes binding of libkvc (include/kvc.h).

Argument marshalling only: every step of the decode path runs in libkvc's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built this module raises ImportError -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libkvc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libkvc.so not found at {LIB_PATH}; build it with `python paged_kv_cache_split_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

# status codes (kvc_status)
OK, E_INVALID, E_UNSUPPORTED, E_NO_BLOCKS, E_NO_SEQ, E_SEQ_EXISTS, E_HIP, E_WORKSPACE = range(8)
STATUS_NAMES = {0: "OK", 1: "E_INVALID", 2: "E_UNSUPPORTED", 3: "E_NO_BLOCKS", 4: "E_NO_SEQ",
                5: "E_SEQ_EXISTS", 6: "E_HIP", 7: "E_WORKSPACE"}
STATIC_SCRATCH_BYTES = 32 << 20   # KVC_STATIC_SCRATCH_BYTES
# dtypes (kvc_dtype)
F32, F16, BF16, FP8, INT8 = 0, 1, 2, 3, 4
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "fp8": FP8, "int8": INT8}

SYMBOLS = [
    "kvc_bytes_per_token", "kvc_pool_bytes", "kvc_scale_bytes", "kvc_scratch_bytes", "kvc_create", "kvc_destroy",
    "kvc_set_scratch", "kvc_add_seq", "kvc_fork", "kvc_free_seq", "kvc_truncate", "kvc_truncate_many", "kvc_evict",
    "kvc_reserve_host",
    "kvc_get_table", "kvc_stats", "kvc_check_shared_prefix", "kvc_append", "kvc_export_tables", "kvc_decode_workspace_bytes",
    "kvc_decode_attention", "kvc_decode_attention_static", "kvc_extend_workspace_bytes", "kvc_extend_attention", "kvc_sched_create",
    "kvc_sched_destroy", "kvc_sched_submit", "kvc_sched_plan", "kvc_sched_commit", "kvc_sched_get_stats",
    "kvc_stream_copy", "kvc_stream_read", "kvc_last_error",
]


class KvcConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("kv_dtype", ctypes.c_int),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("dev_scratch", ctypes.c_void_p), ("dev_scratch_bytes", ctypes.c_size_t),
        ("free_order", ctypes.POINTER(ctypes.c_int32)),
    ]


class KvcStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("total_blocks", "free_blocks", "used_blocks", "shared_blocks",
                                               "peak_used_blocks", "cow_copies", "num_seqs")]


class KvcSchedConfig(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32), ("max_tokens", ctypes.c_int32)]


class KvcSchedStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("submitted", "running", "waiting", "finished", "preemptions",
                                              "iterations", "tokens_scheduled")]


class KvcDecodeOpts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32), ("work_items", ctypes.c_int32),
                ("pool_pieces", ctypes.c_int32), ("pool_shift", ctypes.c_int32),
                ("split_start", ctypes.c_void_p), ("split_end", ctypes.c_void_p), ("window", ctypes.c_int32),
                ("tiles_per_wave", ctypes.c_int32), ("shared_prefix", ctypes.c_int32),
                ("seq_ids", ctypes.POINTER(ctypes.c_int64)), ("k_new", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p)]


_i32, _i64, _sz, _vp, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_P32, _P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)

_sig = {
    "kvc_bytes_per_token": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "kvc_pool_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, ctypes.c_int]),
    "kvc_scale_bytes": (_sz, [_i32, _i32, _i32]),
    "kvc_scratch_bytes": (_sz, [_i32, _i64]),
    "kvc_create": (ctypes.c_int, [ctypes.POINTER(KvcConfig), ctypes.POINTER(_vp)]),
    "kvc_destroy": (None, [_vp]),
    "kvc_set_scratch": (ctypes.c_int, [_vp, _vp, _sz]),
    "kvc_add_seq": (ctypes.c_int, [_vp, _i64, _i32]),
    "kvc_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "kvc_free_seq": (ctypes.c_int, [_vp, _i64]),
    "kvc_truncate": (ctypes.c_int, [_vp, _i64, _i32]),
    "kvc_truncate_many": (ctypes.c_int, [_vp, _i32, _P64, _P32]),
    "kvc_evict": (ctypes.c_int, [_vp, _i64, _i32]),
    "kvc_reserve_host": (ctypes.c_int, [_vp, _i32, _P64, _P32, _P32, _P32, _P32, _i32, _P32]),
    "kvc_get_table": (ctypes.c_int, [_vp, _i64, _P32, _i32, _P32, _P32]),
    "kvc_stats": (ctypes.c_int, [_vp, ctypes.POINTER(KvcStats)]),
    "kvc_check_shared_prefix": (ctypes.c_int, [_vp, _i32, _P64, _i32]),
    "kvc_append": (ctypes.c_int, [_vp, _i32, _P64, _P32, _vp, _vp, ctypes.c_int, _vp]),
    "kvc_export_tables": (ctypes.c_int, [_vp, _i32, _P64, _vp, _i32, _vp, _vp]),
    "kvc_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(KvcDecodeOpts)]),
    "kvc_decode_attention": (ctypes.c_int, [_vp, _i32, _vp, ctypes.c_int, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f, _vp, _vp, _sz, ctypes.POINTER(KvcDecodeOpts), _vp]),
    "kvc_decode_attention_static": (ctypes.c_int, [_vp, _i32, _vp, ctypes.c_int, _vp, _i32, _vp, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _f, _vp, ctypes.POINTER(KvcDecodeOpts), _vp]),
    "kvc_extend_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(KvcDecodeOpts)]),
    "kvc_extend_attention": (ctypes.c_int, [_vp, _i32, _vp, ctypes.c_int, _vp, _i32, _i32, _vp, _i32, _vp, _i32,
                                            _i32, _i32, _i32, _i32, _i32, _f, _vp, _vp, _sz,
                                            ctypes.POINTER(KvcDecodeOpts), _vp]),
    "kvc_sched_create": (ctypes.c_int, [_vp, ctypes.POINTER(KvcSchedConfig), ctypes.POINTER(_vp)]),
    "kvc_sched_destroy": (None, [_vp]),
    "kvc_sched_submit": (ctypes.c_int, [_vp, _i64, _i32, _i32]),
    "kvc_sched_plan": (ctypes.c_int, [_vp, _i32, _P64, _P32, _P32, _P32, _P32, _P64, _i32, _P32]),
    "kvc_sched_commit": (ctypes.c_int, [_vp, _P64, _i32, _P32]),
    "kvc_sched_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(KvcSchedStats)]),
    "kvc_stream_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "kvc_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _sz, _vp]),
    "kvc_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.kvc_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status: int, where: str):
    if status != OK:
        raise KvcError(status, where)


def lib():
    return _lib


def _i64_array(xs):
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int64))
    return a, a.ctypes.data_as(_P64)


def _i32_array(xs):
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int32))
    return a, a.ctypes.data_as(_P32)


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    if isinstance(t, str):
        return DTYPE_CODES[t]
    import torch
    return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t]


# -- sizing -----------------------------------------------------------------

def bytes_per_token(num_layers, num_kv_heads, head_dim, dtype) -> int:
    return _lib.kvc_bytes_per_token(num_layers, num_kv_heads, head_dim, DTYPE_CODES[dtype])


def pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, block_size, dtype) -> int:
    return _lib.kvc_pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, block_size, DTYPE_CODES[dtype])


def scale_bytes(num_layers, num_blocks, num_kv_heads) -> int:
    return _lib.kvc_scale_bytes(num_layers, num_blocks, num_kv_heads)


def scratch_bytes(max_batch, max_tokens) -> int:
    return _lib.kvc_scratch_bytes(max_batch, max_tokens)


def decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_context_len, partition_tokens=0,
                           kernel=0, work_items=0, pool_pieces=0, pool_shift=0, shared_prefix=0) -> int:
    opts = KvcDecodeOpts(partition_tokens, kernel, work_items, pool_pieces, pool_shift, None, None, 0, 0,
                         shared_prefix)
    return _lib.kvc_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_context_len,
                                           ctypes.byref(opts))


def extend_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_query_len, max_context_len, work_items=0,
                           tiles_per_wave=0, kernel=0) -> int:
    opts = KvcDecodeOpts(0, kernel, work_items, 0, 0, None, None, 0, tiles_per_wave)
    return _lib.kvc_extend_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_query_len, max_context_len,
                                           ctypes.byref(opts))


def stream_copy(dst, src, nbytes=None, stream=None):
    """Plain device copy of ``nbytes`` (default: all of src) -- the calibration kernel."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(_lib.kvc_stream_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), nbytes,
                                _stream_ptr(stream)), "kvc_stream_copy")


def stream_read(src, sink, nbytes=None, stream=None):
    """Plain streaming read of ``nbytes`` (default: all of src) -- the read-rate
    calibration kernel; sink: a device int32/uint32 tensor the waves write to."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(_lib.kvc_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                sink.numel(), _stream_ptr(stream)), "kvc_stream_read")


# -- the cache ----------------------------------------------------------------

class KVCache:
    """A paged KV cache: host bookkeeping in libkvc, pools in torch device memory.

    ``device=None`` builds a bookkeeping-only cache (no pools, no device work).
    """

    def __init__(self, num_layers, num_kv_heads, head_dim, num_blocks, kv_dtype, block_size=16,
                 device="cuda", free_order=None):
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.num_blocks, self.block_size, self.kv_dtype = num_blocks, block_size, kv_dtype
        self.device = device
        self.k_pool = self.v_pool = self.k_scale = self.v_scale = self.scratch = None
        cfg = KvcConfig()
        cfg.num_layers, cfg.num_kv_heads, cfg.head_dim = num_layers, num_kv_heads, head_dim
        cfg.block_size, cfg.num_blocks, cfg.kv_dtype = block_size, num_blocks, DTYPE_CODES[kv_dtype]
        if device is not None:
            import torch
            nbytes = pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, block_size, kv_dtype)
            self.k_pool = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.v_pool = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            cfg.k_pool, cfg.v_pool = self.k_pool.data_ptr(), self.v_pool.data_ptr()
            if kv_dtype in ("fp8", "int8"):
                n = scale_bytes(num_layers, num_blocks, num_kv_heads) // 4
                self.k_scale = torch.zeros(n, dtype=torch.float32, device=device)
                self.v_scale = torch.zeros(n, dtype=torch.float32, device=device)
                cfg.k_scale, cfg.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
        self._order = None
        if free_order is not None:
            self._order, cfg.free_order = _i32_array(free_order)
        handle = ctypes.c_void_p()
        _check(_lib.kvc_create(ctypes.byref(cfg), ctypes.byref(handle)), "kvc_create")
        self._h = handle
        self._order = None

    def close(self):
        if getattr(self, "_h", None):
            _lib.kvc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # bookkeeping
    def add_seq(self, seq_id, num_tokens=0):
        _check(_lib.kvc_add_seq(self._h, int(seq_id), int(num_tokens)), "kvc_add_seq")

    def fork(self, parent_id, child_id):
        _check(_lib.kvc_fork(self._h, int(parent_id), int(child_id)), "kvc_fork")

    def free_seq(self, seq_id):
        _check(_lib.kvc_free_seq(self._h, int(seq_id)), "kvc_free_seq")

    def evict(self, seq_id, keep_from):
        """Release the blocks of seq_id holding only positions < keep_from."""
        _check(_lib.kvc_evict(self._h, int(seq_id), int(keep_from)), "kvc_evict")

    def truncate(self, seq_id, num_tokens):
        _check(_lib.kvc_truncate(self._h, int(seq_id), int(num_tokens)), "kvc_truncate")

    def truncate_many(self, seq_ids, num_tokens):
        """truncate of every (seq_ids[i], num_tokens[i]) in one call, last entry
        first, all or nothing."""
        ids, pids = _i64_array(seq_ids)
        nt, pnt = _i32_array(num_tokens)
        if len(ids) != len(nt):
            raise ValueError("seq_ids and num_tokens differ in length")
        _check(_lib.kvc_truncate_many(self._h, len(ids), pids, pnt), "kvc_truncate_many")

    def reserve_host(self, seq_ids, n_new=None):
        ids, pids = _i64_array(seq_ids)
        nn, pnn = (None, None) if n_new is None else _i32_array(n_new)
        total = len(ids) if n_new is None else int(np.sum(nn))
        slots = np.zeros(max(total, 1), dtype=np.int32)
        cap = len(ids) + total // max(self.block_size, 1) + 1
        src = np.zeros(cap, dtype=np.int32)
        dst = np.zeros(cap, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.kvc_reserve_host(self._h, len(ids), pids, pnn, slots.ctypes.data_as(_P32),
                                     src.ctypes.data_as(_P32), dst.ctypes.data_as(_P32), cap,
                                     ctypes.byref(ncow)), "kvc_reserve_host")
        n = ncow.value
        return slots[:total].tolist(), list(zip(src[:n].tolist(), dst[:n].tolist()))

    def get_table(self, seq_id):
        nb, ln = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_lib.kvc_get_table(self._h, int(seq_id), None, 0, ctypes.byref(nb), ctypes.byref(ln)),
               "kvc_get_table")
        out = np.zeros(max(nb.value, 1), dtype=np.int32)
        _check(_lib.kvc_get_table(self._h, int(seq_id), out.ctypes.data_as(_P32), nb.value, ctypes.byref(nb),
                                  ctypes.byref(ln)), "kvc_get_table")
        return out[:nb.value].tolist(), ln.value

    def check_shared_prefix(self, seq_ids, prefix_tokens):
        """Raise KvcError unless every sequence holds more than prefix_tokens
        tokens and starts with seq_ids[0]'s first prefix_tokens / block_size blocks."""
        ids, pids = _i64_array(seq_ids)
        _check(_lib.kvc_check_shared_prefix(self._h, len(ids), pids, int(prefix_tokens)), "kvc_check_shared_prefix")

    def stats(self) -> dict:
        st = KvcStats()
        _check(_lib.kvc_stats(self._h, ctypes.byref(st)), "kvc_stats")
        return {n: getattr(st, n) for n, _ in KvcStats._fields_}

    # device work
    def _ensure_scratch(self, active, total):
        import torch
        need = scratch_bytes(active, total)
        if self.scratch is None or self.scratch.numel() < need:
            self.scratch = torch.empty(max(need, 4096), dtype=torch.uint8, device=self.device)
            _check(_lib.kvc_set_scratch(self._h, ctypes.c_void_p(self.scratch.data_ptr()), self.scratch.numel()),
                   "kvc_set_scratch")

    def append(self, seq_ids, k_new, v_new, n_new=None, stream=None):
        """k_new / v_new: device tensors [num_layers, T, Hkv, D] (or [T, Hkv, D] for one layer).
        Both None: reserve the slots (and copy shared blocks) only; the decode
        then writes each sequence's newest row (``decode(..., k_new=, v_new=)``)."""
        ids, pids = _i64_array(seq_ids)
        nn, pnn = (None, None) if n_new is None else _i32_array(n_new)
        total = len(ids) if n_new is None else int(np.sum(nn))
        active = len(ids) if n_new is None else int(np.count_nonzero(nn))
        if k_new is None and v_new is None:
            self._ensure_scratch(active, total)
            _check(_lib.kvc_append(self._h, len(ids), pids, pnn, None, None, BF16, _stream_ptr(stream)),
                   "kvc_append")
            return
        for t in (k_new, v_new):
            expect = self.num_layers * total * self.num_kv_heads * self.head_dim
            if not t.is_contiguous() or t.numel() != expect or not t.is_cuda:
                raise ValueError(f"append rows must be contiguous device tensors of {expect} elements")
        self._ensure_scratch(active, total)
        _check(_lib.kvc_append(self._h, len(ids), pids, pnn, ctypes.c_void_p(k_new.data_ptr()),
                               ctypes.c_void_p(v_new.data_ptr()), _dtype_code(k_new.dtype), _stream_ptr(stream)),
               "kvc_append")

    def export_tables(self, seq_ids, max_blocks=None, block_table=None, context_lens=None, stream=None):
        import torch
        ids, pids = _i64_array(seq_ids)
        if max_blocks is None:
            max_blocks = max(1, max(len(self.get_table(s)[0]) for s in ids))
        if block_table is None:
            block_table = torch.empty((len(ids), max_blocks), dtype=torch.int32, device=self.device)
        if context_lens is None:
            context_lens = torch.empty((len(ids),), dtype=torch.int32, device=self.device)
        _check(_lib.kvc_export_tables(self._h, len(ids), pids, ctypes.c_void_p(block_table.data_ptr()),
                                      int(max_blocks), ctypes.c_void_p(context_lens.data_ptr()),
                                      _stream_ptr(stream)), "kvc_export_tables")
        return block_table, context_lens

    def decode(self, q, block_table, context_lens, max_context_len, scale, layer=0, out=None, workspace=None,
               partition_tokens=0, kernel=0, work_items=0, pool_pieces=0, pool_shift=0, split_events=None,
               stream=None, window=0, shared_prefix=0, seq_ids=None, k_new=None, v_new=None):
        """Decode attention for one layer.  q: [B, Hq, D] device tensor.
        ``window`` > 0: each token sees at most that many rows ending at its own.
        ``shared_prefix`` > 0: the first that many tokens of every sequence are one
        shared prefix, attended once for the batch (the cascade split);
        ``seq_ids`` (the batch's sequence ids) has the library check that first.
        ``k_new`` / ``v_new``: this layer's new rows [B, Hkv, D] (q's dtype), written
        to each sequence's newest position before it is attended."""
        import torch
        B, Hq, D = q.shape
        if not q.is_contiguous():
            raise ValueError("q must be contiguous")
        opts = KvcDecodeOpts(int(partition_tokens), int(kernel), int(work_items), int(pool_pieces), int(pool_shift),
                             None, None, int(window), 0, int(shared_prefix))
        if seq_ids is not None:
            ids_arr, opts.seq_ids = _i64_array(seq_ids)
            if len(ids_arr) != B:
                raise ValueError("seq_ids must name one sequence per row of q")
        if (k_new is None) != (v_new is None):
            raise ValueError("k_new and v_new go together")
        if k_new is not None:
            for t in (k_new, v_new):
                if not t.is_contiguous() or t.numel() != B * self.num_kv_heads * D or t.dtype != q.dtype:
                    raise ValueError("k_new / v_new must be contiguous [B, Hkv, D] tensors in q's dtype")
            opts.k_new, opts.v_new = k_new.data_ptr(), v_new.data_ptr()
        if split_events is not None:
            opts.split_start = split_events[0].cuda_event
            opts.split_end = split_events[1].cuda_event
        ws_need = _lib.kvc_decode_workspace_bytes(B, Hq, self.num_kv_heads, D, int(max_context_len),
                                                  ctypes.byref(opts))
        if workspace is None or workspace.numel() < ws_need:
            workspace = torch.empty(max(ws_need, 256), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        _check(_lib.kvc_decode_attention(
            self._h, int(layer), ctypes.c_void_p(q.data_ptr()), _dtype_code(q.dtype),
            ctypes.c_void_p(block_table.data_ptr()), int(block_table.shape[1]),
            ctypes.c_void_p(context_lens.data_ptr()), int(max_context_len), B, Hq, self.num_kv_heads, D,
            self.block_size, float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel(), ctypes.byref(opts), _stream_ptr(stream)), "kvc_decode_attention")
        return out

    def decode_static(self, q, block_table, context_lens, max_context_len, scale, layer=0, out=None,
                      partition_tokens=0, kernel=0, work_items=0, pool_pieces=0, pool_shift=0, stream=None, window=0,
                      shared_prefix=0, k_new=None, v_new=None):
        """decode() through kvc_decode_attention_static: no workspace, the
        library's static one (calls on one GPU must not overlap)."""
        import torch
        B, Hq, D = q.shape
        if not q.is_contiguous():
            raise ValueError("q must be contiguous")
        opts = KvcDecodeOpts(int(partition_tokens), int(kernel), int(work_items), int(pool_pieces), int(pool_shift),
                             None, None, int(window), 0, int(shared_prefix))
        if (k_new is None) != (v_new is None):
            raise ValueError("k_new and v_new go together")
        if k_new is not None:
            opts.k_new, opts.v_new = k_new.data_ptr(), v_new.data_ptr()
        if out is None:
            out = torch.empty_like(q)
        _check(_lib.kvc_decode_attention_static(
            self._h, int(layer), ctypes.c_void_p(q.data_ptr()), _dtype_code(q.dtype),
            ctypes.c_void_p(block_table.data_ptr()), int(block_table.shape[1]),
            ctypes.c_void_p(context_lens.data_ptr()), int(max_context_len), B, Hq, self.num_kv_heads, D,
            self.block_size, float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.byref(opts), _stream_ptr(stream)),
            "kvc_decode_attention_static")
        return out

    def extend(self, q, query_start, max_query_len, block_table, context_lens, max_context_len, scale, layer=0,
               out=None, workspace=None, work_items=0, split_events=None, stream=None, window=0, tiles_per_wave=0,
               kernel=0):
        """Attention of several new tokens per sequence (causal among them) for
        one layer.  q: [total_query, Hq, D] device tensor; query_start: device
        int32 [B + 1] (rows of sequence b are query_start[b] .. query_start[b+1]-1).
        ``kernel``: 0 auto, 2 rows split over waves and merged, 3 one wave per
        32 (token, head) columns over all their rows."""
        import torch
        T, Hq, D = q.shape
        B = int(context_lens.shape[0])
        if not q.is_contiguous():
            raise ValueError("q must be contiguous")
        if query_start.dtype != torch.int32 or query_start.numel() != B + 1:
            raise ValueError("query_start must be int32 with batch + 1 entries")
        opts = KvcDecodeOpts(0, int(kernel), int(work_items), 0, 0, None, None, int(window), int(tiles_per_wave))
        if split_events is not None:
            opts.split_start = split_events[0].cuda_event
            opts.split_end = split_events[1].cuda_event
        ws_need = _lib.kvc_extend_workspace_bytes(B, Hq, self.num_kv_heads, D, int(max_query_len), int(max_context_len),
                                                  ctypes.byref(opts))
        if workspace is None or workspace.numel() < ws_need:
            workspace = torch.empty(max(ws_need, 256), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty_like(q)
        _check(_lib.kvc_extend_attention(
            self._h, int(layer), ctypes.c_void_p(q.data_ptr()), _dtype_code(q.dtype),
            ctypes.c_void_p(query_start.data_ptr()), T, int(max_query_len),
            ctypes.c_void_p(block_table.data_ptr()), int(block_table.shape[1]),
            ctypes.c_void_p(context_lens.data_ptr()), int(max_context_len), B, Hq, self.num_kv_heads, D,
            self.block_size, float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel(), ctypes.byref(opts), _stream_ptr(stream)), "kvc_extend_attention")
        return out


class Scheduler:
    """Continuous-batching scheduler (libkvc's kvc_sched_*) over a KVCache.

    Each iteration: ``plan()`` -> the rows to append per request, then the
    caller appends them (``cache.append(ids, k, v, n_new)``) and runs the
    attention, then ``commit()`` -> the requests that finished."""

    def __init__(self, cache: "KVCache", max_batch: int, chunk_tokens: int, max_tokens: int):
        self.cache = cache
        self.max_batch = int(max_batch)
        cfg = KvcSchedConfig(int(max_batch), int(chunk_tokens), int(max_tokens))
        h = ctypes.c_void_p()
        _check(_lib.kvc_sched_create(cache.handle, ctypes.byref(cfg), ctypes.byref(h)), "kvc_sched_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _lib.kvc_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, req_id, prompt_len, max_new_tokens):
        _check(_lib.kvc_sched_submit(self._h, int(req_id), int(prompt_len), int(max_new_tokens)), "kvc_sched_submit")

    def plan(self):
        """-> dict(ids, n_new, start, emits, preempted) for the next iteration."""
        cap = self.max_batch
        ids, pids = _i64_array(np.zeros(cap))
        n, pn = _i32_array(np.zeros(cap))
        st, pst = _i32_array(np.zeros(cap))
        em, pem = _i32_array(np.zeros(cap))
        pre, ppre = _i64_array(np.zeros(max(cap, 64)))
        batch, npre = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_lib.kvc_sched_plan(self._h, cap, pids, pn, pst, pem, ctypes.byref(batch), ppre, len(pre),
                                   ctypes.byref(npre)), "kvc_sched_plan")
        b, k = batch.value, min(npre.value, len(pre))
        return dict(ids=[int(x) for x in ids[:b]], n_new=[int(x) for x in n[:b]], start=[int(x) for x in st[:b]],
                    emits=[int(x) for x in em[:b]], preempted=[int(x) for x in pre[:k]])

    def commit(self):
        """-> ids of the requests that finished in this iteration."""
        cap = max(self.max_batch, 1)
        fin, pfin = _i64_array(np.zeros(cap))
        nf = ctypes.c_int32(0)
        _check(_lib.kvc_sched_commit(self._h, pfin, cap, ctypes.byref(nf)), "kvc_sched_commit")
        return [int(x) for x in fin[:min(nf.value, cap)]]

    def stats(self) -> dict:
        st = KvcSchedStats()
        _check(_lib.kvc_sched_get_stats(self._h, ctypes.byref(st)), "kvc_sched_get_stats")
        return {n: int(getattr(st, n)) for n, _ in KvcSchedStats._fields_}
