"""Drive one workload through the HIP library and through the oracle.

The two sides share only the workload (``workloads``): the GPU side runs the
setup operations through libkvc, the oracle side through ``oracle.kvstore``.
``pool_layout`` reads device pools back into (block, layer, head, slot, dim)
order following the layout documented in include/kvc.h.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import make_values, setup_ops

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BITS_TORCH = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}
BITS_NP = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8, "int8": np.uint8}
QUANTISED = ("fp8", "int8")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}


def to_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw storage bits of a tensor of the given dtype, as an unsigned numpy array."""
    t = t.detach().cpu().contiguous()
    if dtype in QUANTISED:
        return t.view(torch.uint8).numpy()
    return t.view(BITS_TORCH[dtype]).numpy().view(BITS_NP[dtype])


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


# -- pool layout (include/kvc.h) ------------------------------------------------

def read_pools(cache):
    """Pools of a KVCache as raw bits [N, L, H, block_size, D] (and fp8 scales [N, L, H]).

    K pool [L][N][H][D/x][bs][x], V pool [L][N][H][D][bs], x = 16 / element bytes.
    """
    L, N, H, D, bs, dt = (cache.num_layers, cache.num_blocks, cache.num_kv_heads, cache.head_dim,
                          cache.block_size, cache.kv_dtype)
    x = 16 // ELEM_BYTES[dt]
    k = cache.k_pool.detach().cpu().numpy().view(BITS_NP[dt]).reshape(L, N, H, D // x, bs, x)
    k = k.transpose(1, 0, 2, 4, 3, 5).reshape(N, L, H, bs, D)
    v = cache.v_pool.detach().cpu().numpy().view(BITS_NP[dt]).reshape(L, N, H, D, bs)
    v = v.transpose(1, 0, 2, 4, 3)
    out = dict(k=np.ascontiguousarray(k), v=np.ascontiguousarray(v))
    if dt in QUANTISED:
        out["k_scale"] = cache.k_scale.cpu().numpy().reshape(L, N, H).transpose(1, 0, 2).copy()
        out["v_scale"] = cache.v_scale.cpu().numpy().reshape(L, N, H).transpose(1, 0, 2).copy()
    return out


# -- GPU side -------------------------------------------------------------------

def gpu_setup(wl, values, device="cuda", pool_fill=None):
    """Build the cache and the history through libkvc; returns the KVCache.
    ``pool_fill``: a byte value written over both pools before anything else."""
    from paged_kv_cache_split_amd import KVCache
    cache = KVCache(wl.num_layers, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.kv_dtype,
                    block_size=wl.block_size, device=device, free_order=wl.free_order)
    if pool_fill is not None:
        cache.k_pool.fill_(pool_fill)
        cache.v_pool.fill_(pool_fill)
    k_hist = values["k_hist"].to(device)
    v_hist = values["v_hist"].to(device)
    row = 0
    for op in setup_ops(wl):
        if op[0] == "add":
            cache.add_seq(op[1], op[2])
        elif op[0] == "fork":
            cache.fork(op[1], op[2])
        elif op[0] == "append":
            seqs, n_new = op[1], op[2]
            t = int(sum(n_new))
            if t:
                cache.append(seqs, k_hist[:, row:row + t].contiguous(), v_hist[:, row:row + t].contiguous(),
                             n_new=n_new)
            row += t
        elif op[0] == "evict":
            cache.evict(op[1], op[2])
    return cache


POISON_BYTE = 0xFF   # as float32 a NaN, as int32 -1


def poisoned_buffers(cache, q, max_context_len, **opts):
    """A decode workspace and an output filled with 0xFF bytes: a partial,
    chunk record or output the kernels read or leave without having written
    it turns into NaN (or an out-of-range chunk index) in one run."""
    from paged_kv_cache_split_amd import decode_workspace_bytes
    B, Hq, D = q.shape
    keys = ("partition_tokens", "kernel", "work_items", "pool_pieces", "pool_shift", "shared_prefix")
    need = decode_workspace_bytes(B, Hq, cache.num_kv_heads, D, int(max_context_len),
                                  **{k: int(v) for k, v in opts.items() if k in keys})
    ws = torch.full((max(need, 256),), POISON_BYTE, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    out.view(torch.uint8).fill_(POISON_BYTE)
    return ws, out


def decode_poisoned(cache, q, block_table, context_lens, max_context_len, scale, **kw):
    """cache.decode into a poisoned workspace and output (unless given)."""
    ws, out = poisoned_buffers(cache, q, max_context_len, **kw)
    kw.setdefault("workspace", ws)
    kw.setdefault("out", out)
    return cache.decode(q, block_table, context_lens, max_context_len, scale, **kw)


def extend_poisoned(cache, q, query_start, max_query_len, block_table, context_lens, max_context_len, scale, **kw):
    """cache.extend into a workspace and an output filled with 0xFF bytes."""
    from paged_kv_cache_split_amd import extend_workspace_bytes
    T, Hq, D = q.shape
    B = int(context_lens.shape[0])
    need = extend_workspace_bytes(B, Hq, cache.num_kv_heads, D, int(max_query_len), int(max_context_len),
                                  work_items=int(kw.get("work_items", 0)),
                                  tiles_per_wave=int(kw.get("tiles_per_wave", 0)), kernel=int(kw.get("kernel", 0)))
    if "workspace" not in kw:
        kw["workspace"] = torch.full((max(need, 256),), POISON_BYTE, dtype=torch.uint8, device=q.device)
    if "out" not in kw:
        out = torch.empty_like(q)
        out.view(torch.uint8).fill_(POISON_BYTE)
        kw["out"] = out
    return cache.extend(q, query_start, max_query_len, block_table, context_lens, max_context_len, scale, **kw)


def gpu_step(cache, wl, values, kernel=0, partition_tokens=0, device="cuda", out=None, work_items=0, **split):
    """The decode step: append each sequence's new token, export tables, decode
    (into a poisoned workspace and output).  ``split``: pool_pieces /
    pool_shift of the MFMA kernel."""
    seqs = list(range(wl.batch))
    cache.append(seqs, values["k_new"].to(device).contiguous(), values["v_new"].to(device).contiguous())
    bt, cl = cache.export_tables(seqs)
    q = values["q"].to(device).contiguous()
    ws, out_p = poisoned_buffers(cache, q, wl.max_context_len, kernel=kernel, partition_tokens=partition_tokens,
                                 work_items=work_items, **split)
    o = cache.decode(q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=partition_tokens,
                     out=out_p if out is None else out, workspace=ws, work_items=work_items, window=wl.window,
                     **split)
    return o, bt, cl


def gpu_decode_again(cache, wl, values, bt, cl, kernel=0, partition_tokens=0, device="cuda", work_items=0, **split):
    """Decode again on the same tables, into a poisoned workspace and output."""
    q = values["q"].to(device).contiguous()
    ws, out = poisoned_buffers(cache, q, wl.max_context_len, kernel=kernel, partition_tokens=partition_tokens,
                               work_items=work_items, **split)
    return cache.decode(q, bt, cl, wl.max_context_len, wl.scale, kernel=kernel, partition_tokens=partition_tokens,
                        work_items=work_items, window=wl.window, out=out, workspace=ws, **split)


# -- oracle side ------------------------------------------------------------------

def oracle_run(wl, values):
    """Execute the setup and the step's append on the oracle's store; return it."""
    from oracle.kvstore import KVStoreModel
    st = KVStoreModel(wl.num_layers, wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.kv_dtype,
                      free_order=wl.free_order, in_dtype=wl.new_dtype)
    kb = to_bits(values["k_hist"], wl.new_dtype)
    vb = to_bits(values["v_hist"], wl.new_dtype)
    row = 0
    for op in setup_ops(wl):
        if op[0] == "add":
            assert st.allocate(op[1], op[2]) == 0
        elif op[0] == "fork":
            assert st.fork(op[1], op[2]) == 0
        elif op[0] == "append":
            t = int(sum(op[2]))
            status, _, _ = st.append(op[1], op[2], kb[:, row:row + t], vb[:, row:row + t])
            assert status == 0
            row += t
        elif op[0] == "evict":
            assert st.evict(op[1], op[2]) == 0
    seqs = list(range(wl.batch))
    status, slots, cow = st.append(seqs, [int(x) for x in wl.q_lens], to_bits(values["k_new"], wl.new_dtype),
                                   to_bits(values["v_new"], wl.new_dtype))
    assert status == 0
    return st


def oracle_decode(st, wl, values, seqs=None, layer=0):
    """fp64 decode outputs [len(seqs), Hq, D] from the oracle store's stored values."""
    from oracle.attention import decode_attention, extend_attention
    q = to_f64(values["q"])
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    out = np.empty((len(seqs), wl.num_heads, wl.head_dim))
    for i, b in enumerate(seqs):
        if wl.window:
            n = st.tables.lens[b]
            k, v = st.gather(b, layer, start=max(0, n - wl.window))
            out[i] = extend_attention(q[b:b + 1], k, v, wl.scale, window=wl.window)[0]
        else:
            k, v = st.gather(b, layer)
            out[i] = decode_attention(q[b], k, v, wl.scale)
    return out


def query_start(wl):
    """Exclusive prefix sum of the step's new tokens per sequence: [B + 1]."""
    return np.concatenate([[0], np.cumsum(wl.q_lens)]).astype(np.int32)


def gpu_extend_step(cache, wl, values, device="cuda", work_items=0):
    """A step with several new tokens per sequence: append them all, export the
    tables, then attention of every new token (causal among them)."""
    seqs = list(range(wl.batch))
    cache.append(seqs, values["k_new"].to(device).contiguous(), values["v_new"].to(device).contiguous(),
                 n_new=[int(x) for x in wl.q_lens])
    bt, cl = cache.export_tables(seqs)
    qs = torch.from_numpy(query_start(wl)).to(device)
    q = values["q"].to(device).contiguous()
    o = extend_poisoned(cache, q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, work_items=work_items,
                     window=wl.window)
    return o, bt, cl, qs


def oracle_extend(st, wl, values, seqs=None, layer=0):
    """fp64 outputs [Q, Hq, D] of every new token from the oracle store's stored
    values (rows of sequence b at query_start[b] ..)."""
    from oracle.attention import extend_attention
    q = to_f64(values["q"])
    qs = query_start(wl)
    out = np.full((wl.total_queries, wl.num_heads, wl.head_dim), np.nan)
    for b in (range(wl.batch) if seqs is None else seqs):
        if qs[b + 1] == qs[b]:
            continue
        n = st.tables.lens[b]
        first = max(0, n - int(qs[b + 1] - qs[b]) + 1 - wl.window) if wl.window else 0
        k, v = st.gather(b, layer, start=first)
        out[qs[b]:qs[b + 1]] = extend_attention(q[qs[b]:qs[b + 1]], k, v, wl.scale, window=wl.window)
    return out


def logical_history(wl, values, b, layer=0):
    """The unquantised K/V rows of sequence b in position order (history + new
    token), as fp64, straight from the workload tensors."""
    k_hist, v_hist = values["k_hist"], values["v_hist"]
    rows = _history_rows(wl, b)
    k = torch.cat([k_hist[layer, rows], values["k_new"][layer, b:b + 1]]).to(torch.float64).cpu().numpy()
    v = torch.cat([v_hist[layer, rows], values["v_new"][layer, b:b + 1]]).to(torch.float64).cpu().numpy()
    return k, v


def _history_rows(wl, b):
    from workloads import history_rows_of
    return torch.from_numpy(history_rows_of(wl, b))


def check_close(gpu: np.ndarray, ref: np.ndarray, atol: float, rtol: float, what: str):
    """Per element |gpu - ref| <= atol + rtol * |ref|; returns (max_abs, max_rel)."""
    d = np.abs(gpu - ref)
    bad = d > atol + rtol * np.abs(ref)
    max_abs = float(d.max()) if d.size else 0.0
    big = np.abs(ref) > 1e-3
    max_rel = float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"(atol {atol}, rtol {rtol}); first at {tuple(idx)}: gpu {gpu[tuple(idx)]!r} "
                             f"ref {ref[tuple(idx)]!r}; max_abs {max_abs:.3e} max_rel {max_rel:.3e}")
    return max_abs, max_rel
