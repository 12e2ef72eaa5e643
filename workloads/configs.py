"""The five decode workloads (and scaled-down variants) as seeded synthetic inputs.

Shapes follow the pages' workloads: a LLaMA2-7B-shaped MHA layer (32/32 heads,
head_dim 128, fp16, 2048 context), a 70B-shaped GQA layer (64 query / 8 KV
heads) at page 5's 4096-token inputs, a 32K context with a shared system-prompt
prefix forked copy-on-write, and an fp8 (E4M3) KV cache over a mixed batch of
up to 16K tokens.  Every config has one layer and 16-token blocks.

Draw order (fixed): context lengths, placement permutation (numpy
``default_rng(seed)``), then the tensors K history, V history, q, k_new,
v_new (torch generator seeded with ``seed`` on the device they are made on),
each drawn as float32 N(0, 1) and rounded to nearest-even into its storage
dtype.  The placement permutation is the initial free-list order handed to the
allocator; blocks are then popped from its end in logical order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16

TORCH_DTYPE_NAMES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}
QUANTISED = ("fp8", "int8")   # caches of one-byte codes; q and the appended rows are bf16


@dataclass
class Workload:
    name: str
    batch: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str            # dtype of q and of the output
    kv_dtype: str           # storage dtype of the cache: f32 / f16 / bf16 / fp8
    new_dtype: str          # dtype of the appended k_new / v_new rows
    context_lens: np.ndarray  # [B] tokens already cached before the step (L_b)
    shared_prefix: int      # tokens of sequence 0 shared by every sequence via fork (0 = none)
    num_blocks: int
    free_order: np.ndarray  # [num_blocks] int32 permutation
    seed: int
    num_layers: int = 1
    block_size: int = BLOCK_SIZE
    extra: dict = field(default_factory=dict)
    query_lens: np.ndarray | None = None   # [B] new tokens per sequence in the step (None: 1 each, decode)
    window: int = 0         # sliding window (0 = none): the history is written in chunks of
    evict_chunk: int = 0    # evict_chunk rows and what leaves the window is evicted after each

    @property
    def q_lens(self) -> np.ndarray:
        """New tokens each sequence appends and queries in the step."""
        if self.query_lens is None:
            return np.ones(self.batch, dtype=np.int64)
        return np.asarray(self.query_lens, dtype=np.int64)

    @property
    def total_queries(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_query_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the fp32 value passed to the kernel."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def attend_lens(self) -> np.ndarray:
        """Rows each sequence holds in the step: L_b plus its appended token(s)."""
        return self.context_lens + self.q_lens

    @property
    def history_rows(self) -> int:
        """Rows of K/V history written during setup (a shared prefix counts once)."""
        if self.shared_prefix:
            return int(self.shared_prefix + np.sum(self.context_lens - self.shared_prefix))
        return int(np.sum(self.context_lens))

    @property
    def max_context_len(self) -> int:
        return int(np.max(self.attend_lens))


def _blocks(n: int) -> int:
    return (n + BLOCK_SIZE - 1) // BLOCK_SIZE


def _exact_pool(lens, shared_prefix: int, q_lens=None) -> int:
    lens = np.asarray(lens)
    q_lens = np.ones(len(lens), dtype=np.int64) if q_lens is None else np.asarray(q_lens)
    if shared_prefix:
        return _blocks(shared_prefix) + int(np.sum([_blocks(l + q) - _blocks(shared_prefix)
                                                    for l, q in zip(lens, q_lens)]))
    return int(np.sum([_blocks(l + q) for l, q in zip(lens, q_lens)]))


def _lengths(cid: int, rng, p) -> np.ndarray:
    kind = p["lens"]
    if kind[0] == "fixed":
        return np.asarray(kind[1], dtype=np.int64)
    if kind[0] == "const":
        return np.full(p["batch"], kind[1], dtype=np.int64)
    if kind[0] == "lognormal":
        _, median, sigma, lo, hi = kind
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=p["batch"])
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind[0] == "uniform":
        _, lo, hi = kind
        return rng.integers(lo, hi, size=p["batch"], endpoint=True).astype(np.int64)
    raise ValueError(kind)


# Full-size configs (the measured workloads) and scaled-down twins with the
# same structure that the oracle finishes in seconds.
CONFIGS = {
    1: dict(name="tiny paged decode, fp32, B4, 8/2 heads, D64, L{17,33,100,256}",
            batch=4, num_heads=8, num_kv_heads=2, head_dim=64, q_dtype="f32", kv_dtype="f32",
            lens=("fixed", [17, 33, 100, 256]), shared_prefix=0, pool=128),
    2: dict(name="LLaMA2-7B-shaped MHA layer, fp16, B32, 32/32 heads, D128, L2048",
            batch=32, num_heads=32, num_kv_heads=32, head_dim=128, q_dtype="f16", kv_dtype="f16",
            lens=("const", 2048), shared_prefix=0, pool=None),
    3: dict(name="70B-shaped GQA layer, bf16, B64, 64/8 heads, D128, L lognormal(median 4096) in [128, 8192]",
            batch=64, num_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
            lens=("lognormal", 4096, 1.0, 128, 8192), shared_prefix=0, pool=None),
    4: dict(name="long-context GQA with 4096-token shared prefix, bf16, B16, 32/8 heads, D128, L32768",
            batch=16, num_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
            lens=("const", 32768), shared_prefix=4096, pool=None),
    5: dict(name="fp8 E4M3 KV mixed batch, bf16 q, B128, 64/8 heads, D128, L uniform 256..16384",
            batch=128, num_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="fp8",
            lens=("uniform", 256, 16384), shared_prefix=0, pool=None),
}

SMALL = {
    1: dict(CONFIGS[1]),
    2: dict(CONFIGS[2], name="MHA fp16 (scaled down), B4, 32/32 heads, D128, L300",
            batch=4, lens=("const", 300)),
    3: dict(CONFIGS[3], name="GQA bf16 (scaled down), B8, 64/8 heads, D128, L lognormal(median 300) in [1, 1200]",
            batch=8, lens=("lognormal", 300, 1.0, 1, 1200)),
    4: dict(CONFIGS[4], name="shared-prefix GQA bf16 (scaled down), B4, 32/8 heads, D128, L700, prefix 256",
            batch=4, lens=("const", 700), shared_prefix=256),
    5: dict(CONFIGS[5], name="fp8 KV (scaled down), B8, 64/8 heads, D128, L uniform 256..1000",
            batch=8, lens=("uniform", 256, 1000)),
}


def make_workload(cid: int, seed: int | None = None, small: bool = False, **override) -> Workload:
    """Build config ``cid`` (1..5).  ``seed`` defaults to the config number."""
    p = dict((SMALL if small else CONFIGS)[cid])
    p.update(override)
    if "kv_dtype" in override and override["kv_dtype"] != CONFIGS[cid]["kv_dtype"]:
        p["name"] = f"{p['name']} -- {override['kv_dtype']} cache instead"
        # q in the cache's own dtype for 16-bit caches, bf16 with one-byte codes
        if "q_dtype" not in override:
            p["q_dtype"] = "bf16" if override["kv_dtype"] in QUANTISED else override["kv_dtype"]
    seed = cid if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = _lengths(cid, rng, p)
    pool = p["pool"] or _exact_pool(lens, p["shared_prefix"])
    free_order = rng.permutation(pool).astype(np.int32)
    kv = p["kv_dtype"]
    return Workload(name=p["name"], batch=p["batch"], num_heads=p["num_heads"],
                    num_kv_heads=p["num_kv_heads"], head_dim=p["head_dim"],
                    q_dtype=p["q_dtype"], kv_dtype=kv,
                    new_dtype=("bf16" if kv in QUANTISED else kv),
                    context_lens=lens, shared_prefix=int(p["shared_prefix"]),
                    num_blocks=int(pool), free_order=free_order, seed=seed)


def custom_workload(batch, num_heads, num_kv_heads, head_dim, kv_dtype, context_lens,
                    q_dtype=None, num_blocks=None, seed=0, shared_prefix=0, name="custom",
                    query_lens=None) -> Workload:
    """A workload of any shape (used by edge-case and sweep tests).
    ``query_lens``: new tokens per sequence in the step (default 1 each)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    rng = np.random.default_rng(seed)
    qls = None if query_lens is None else np.asarray(query_lens, dtype=np.int64)
    pool = num_blocks or _exact_pool(lens, shared_prefix, qls)
    free_order = rng.permutation(pool).astype(np.int32)
    q_dtype = q_dtype or ("bf16" if kv_dtype in QUANTISED else kv_dtype)
    return Workload(name=name, batch=batch, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype,
                    new_dtype=("bf16" if kv_dtype in QUANTISED else kv_dtype),
                    context_lens=lens, shared_prefix=int(shared_prefix), num_blocks=int(pool),
                    free_order=free_order, seed=seed, query_lens=qls)


# Steps with several new tokens per sequence.  "verify": the target model's
# pass over gamma = 5 draft tokens of speculative decoding ("LLM推理优化实战…"
# §4.2 uses gamma = 5) on the 70B-shaped GQA layer's batch; "prefill": page 5
# PART 04's attention benchmark shape (batch 1, 16 heads, head_dim 64, fp16,
# causal, 2048 tokens) as one uncached prompt written into the paged cache;
# "chunk": the last 512-token chunk of a 4096-token prompt (PART 04's long-
# input group) over its first 3584 tokens cached, on the 70B-shaped layer.
EXTEND_CONFIGS = {
    "verify": dict(name="speculative verify, 5 draft tokens, 70B-shaped GQA bf16, B64, 64/8 heads, D128, "
                        "L lognormal(median 4096) in [128, 8192]",
                   batch=64, num_heads=64, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                   lens=("lognormal", 4096, 1.0, 128, 8192), q=("const", 5)),
    "prefill": dict(name="causal prefill of a 2048-token prompt into the paged cache, fp16, B1, 16/16 heads, D64",
                    batch=1, num_heads=16, num_kv_heads=16, head_dim=64, kv_dtype="f16",
                    lens=("const", 0), q=("const", 2048)),
    "chunk": dict(name="chunked prefill, 512-token chunk over 3584 cached, 70B-shaped GQA bf16, B4, 64/8 heads, D128",
                  batch=4, num_heads=64, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                  lens=("const", 3584), q=("const", 512)),
}

EXTEND_SMALL = {
    "verify": dict(EXTEND_CONFIGS["verify"], name="speculative verify (scaled down), B8, 64/8 heads, D128",
                   batch=8, lens=("lognormal", 300, 1.0, 1, 1200)),
    "prefill": dict(EXTEND_CONFIGS["prefill"], name="causal prefill (scaled down), fp16, B1, 16/16 heads, D64, 160 tokens",
                    q=("const", 160)),
    "chunk": dict(EXTEND_CONFIGS["chunk"], name="chunked prefill (scaled down), B2, 64/8 heads, D128, 64 over 200",
                  batch=2, lens=("const", 200), q=("const", 64)),
}

EXTEND_SEEDS = {"verify": 3, "prefill": 6, "chunk": 7}


def make_extend_workload(kind: str, seed: int | None = None, small: bool = False) -> Workload:
    """Build a multi-token step workload ("verify", "prefill" or "chunk")."""
    p = dict((EXTEND_SMALL if small else EXTEND_CONFIGS)[kind])
    seed = EXTEND_SEEDS[kind] if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = _lengths(0, rng, p)
    qls = _lengths(0, rng, dict(p, lens=p["q"]))
    pool = _exact_pool(lens, 0, qls)
    free_order = rng.permutation(pool).astype(np.int32)
    kv = p["kv_dtype"]
    return Workload(name=p["name"], batch=p["batch"], num_heads=p["num_heads"], num_kv_heads=p["num_kv_heads"],
                    head_dim=p["head_dim"], q_dtype=("bf16" if kv in QUANTISED else kv), kv_dtype=kv,
                    new_dtype=("bf16" if kv in QUANTISED else kv), context_lens=lens, shared_prefix=0,
                    num_blocks=int(pool), free_order=free_order, seed=seed, query_lens=qls)


def setup_ops(wl: Workload):
    """The operations that build the cached history, in order.

    ("add", seq, 0)            create an empty sequence
    ("append", seqs, n_new)    append n_new[i] history rows to seqs[i]; rows are
                               taken in order from the K/V history tensors
    ("fork", parent, child)    share the parent's blocks copy-on-write
    ("evict", seq, keep_from)  release the blocks of seq holding only positions
                               before keep_from (sliding window)
    """
    ops = []
    B = wl.batch
    if wl.window:
        # chunks of evict_chunk rows for every sequence, then eviction of what
        # the step's oldest new token (at position L_b) will not see
        for b in range(B):
            ops.append(("add", b, 0))
        lens = [int(l) for l in wl.context_lens]
        done = [0] * B
        while any(d < l for d, l in zip(done, lens)):
            n_new = [min(wl.evict_chunk, l - d) for d, l in zip(done, lens)]
            ops.append(("append", list(range(B)), n_new))
            done = [d + n for d, n in zip(done, n_new)]
            for b in range(B):
                keep = max(0, min(done[b], lens[b] - wl.window + 1))
                if n_new[b] and keep > 0:
                    ops.append(("evict", b, keep))
        return ops
    if wl.shared_prefix:
        ops.append(("add", 0, 0))
        ops.append(("append", [0], [wl.shared_prefix]))
        for b in range(1, B):
            ops.append(("fork", 0, b))
        ops.append(("append", list(range(B)), [int(l) - wl.shared_prefix for l in wl.context_lens]))
    else:
        for b in range(B):
            ops.append(("add", b, 0))
        ops.append(("append", list(range(B)), [int(l) for l in wl.context_lens]))
    return ops


def history_rows_of(wl: Workload, b: int):
    """Indices, in the K/V history tensors, of sequence b's history rows in
    position order (the order setup_ops consumes rows in)."""
    lens = [int(x) for x in wl.context_lens]
    if wl.window:
        rows, base, done = [], 0, [0] * wl.batch
        while any(d < l for d, l in zip(done, lens)):
            n_new = [min(wl.evict_chunk, l - d) for d, l in zip(done, lens)]
            rows.extend(range(base + sum(n_new[:b]), base + sum(n_new[:b]) + n_new[b]))
            base += sum(n_new)
            done = [d + n for d, n in zip(done, n_new)]
        return np.asarray(rows, dtype=np.int64)
    if wl.shared_prefix:
        p = wl.shared_prefix
        start = p + sum(l - p for l in lens[:b])
        return np.concatenate([np.arange(0, p), np.arange(start, start + lens[b] - p)]).astype(np.int64)
    start = sum(lens[:b])
    return np.arange(start, start + lens[b], dtype=np.int64)


# Decode (or several new tokens) under a sliding window with eviction: the
# 70B-shaped GQA layer over 16K-token contexts, each token seeing the last
# 4096 positions ("苦猿的大模型日记" PART 02's sliding window / KV eviction; the
# window length is a builder's choice, the pages give none), the history
# written 1024 rows at a time with what leaves the window evicted after each.
WINDOW_CONFIGS = {
    "decode": dict(name="sliding-window decode, window 4096 over 16K contexts, evicted, 70B-shaped GQA bf16, "
                        "B64, 64/8 heads, D128",
                   batch=64, num_heads=64, num_kv_heads=8, head_dim=128, kv_dtype="bf16", lens=16384, q=1,
                   window=4096, chunk=1024),
}
WINDOW_SMALL = {
    "decode": dict(WINDOW_CONFIGS["decode"], name="sliding-window decode (scaled down), window 200, B4, 32/8, D128",
                   batch=4, num_heads=32, lens=700, window=200, chunk=64),
}


def make_window_workload(kind: str = "decode", seed: int = 8, small: bool = False, kv_dtype=None,
                         query_lens=None) -> Workload:
    p = dict((WINDOW_SMALL if small else WINDOW_CONFIGS)[kind])
    rng = np.random.default_rng(seed)
    B, W, C = p["batch"], p["window"], p["chunk"]
    lens = np.full(B, p["lens"], dtype=np.int64)
    qls = None if query_lens is None else np.asarray(query_lens, dtype=np.int64)
    q_max = 1 if qls is None else int(qls.max())
    # live blocks per sequence never exceed those of window + chunk + new rows
    pool = B * ((W + C + q_max + BLOCK_SIZE - 1) // BLOCK_SIZE + 2)
    free_order = rng.permutation(pool).astype(np.int32)
    kv = kv_dtype or p["kv_dtype"]
    return Workload(name=p["name"], batch=B, num_heads=p["num_heads"], num_kv_heads=p["num_kv_heads"],
                    head_dim=p["head_dim"], q_dtype=("bf16" if kv in QUANTISED else kv), kv_dtype=kv,
                    new_dtype=("bf16" if kv in QUANTISED else kv), context_lens=lens, shared_prefix=0,
                    num_blocks=int(pool), free_order=free_order, seed=seed, query_lens=qls, window=W,
                    evict_chunk=C)


def _randn(shape, dtype_name, gen, device):
    import torch
    tdt = getattr(torch, TORCH_DTYPE_NAMES[dtype_name])
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, dtype=torch.float32, device=device).to(tdt)
    return out


def make_request_values(seed: int, req_id: int, num_layers: int, length: int, num_heads: int, num_kv_heads: int,
                        head_dim: int, q_dtype: str, kv_in_dtype: str, device="cpu"):
    """K/V rows and queries of one request's tokens 0..length-1, drawn from a
    torch generator seeded by (seed, req_id) in the order k, v, q, each as
    float32 N(0, 1) rounded to its dtype.  A request recomputed after
    preemption draws the same values.

    returns dict(k=[layers, length, Hkv, D], v=..., q=[length, Hq, D])"""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + int(req_id))
    k = _randn((num_layers, length, num_kv_heads, head_dim), kv_in_dtype, gen, device)
    v = _randn((num_layers, length, num_kv_heads, head_dim), kv_in_dtype, gen, device)
    q = _randn((length, num_heads, head_dim), q_dtype, gen, device)
    return dict(k=k, v=v, q=q)


LOG2E = 1.4426950408889634


def shape_scores(wl: Workload, values: dict, pattern: str, strength: float = 10.0, q_dim0: float = 16.0):
    """Reshape drawn inputs (in place) so that the scores of a decode or
    several-token step follow a planted profile over the positions, in units
    of log2 of a softmax weight (score * scale * log2 e):

    * "ramp": every query row gets q[..., 0] = q_dim0 and key row p gets
      k[0] = offset(p) / (scale * log2 e * q_dim0) with offset(p) = strength *
      ((p // 16) % 24): the block maxima climb by `strength` per block for 24
      blocks, then fall back and climb again;
    * "sink": as "ramp" but offset(p) = strength for one key row per sequence
      at position ~0.7 n placed mid-block (slot 7), 0 elsewhere;
    * "qscale": every query value multiplied by `strength` (no key change).

    Other values keep their N(0, 1) draws.  The step's new key rows sit at the
    positions after the history.  Returns values (modified)."""
    import torch
    unit = 1.0 / (wl.scale * LOG2E * q_dim0)
    if pattern == "qscale":
        values["q"] = (values["q"].float() * strength).to(values["q"].dtype)
        return values
    if pattern not in ("ramp", "sink"):
        raise ValueError(pattern)
    values["q"][..., 0] = q_dim0
    qls = wl.q_lens
    q0 = np.concatenate([[0], np.cumsum(qls)])
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        n = L + int(qls[b])
        pos = np.arange(n)
        if pattern == "ramp":
            off = strength * ((pos // 16) % 24)
        else:
            off = np.zeros(n)
            p_s = (int(0.7 * n) // 16) * 16 + 7
            if p_s >= n:
                p_s = n - 1
            off[p_s] = strength
        col = torch.from_numpy(off * unit).to(torch.float32)
        rows = torch.from_numpy(history_rows_of(wl, b))
        kh, kn = values["k_hist"], values["k_new"]
        kh[:, rows.to(kh.device), :, 0] = col[:L, None].to(kh.dtype).to(kh.device)
        kn[:, int(q0[b]):int(q0[b + 1]), :, 0] = col[L:, None].to(kn.dtype).to(kn.device)
    return values


def make_values(wl: Workload, device="cpu"):
    """Tensors of the workload, drawn on ``device`` (torch generator seeded with wl.seed).

    k_hist, v_hist: [layers, history_rows, Hkv, D] (new_dtype), rows in setup-op order
    q: [Q, Hq, D] (q_dtype); k_new, v_new: [layers, Q, Hkv, D] (new_dtype), where Q
    is the step's new tokens (B for decode; rows of sequence b follow those of b - 1)
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(wl.seed))
    L, T, H, D = wl.num_layers, wl.history_rows, wl.num_kv_heads, wl.head_dim
    k_hist = _randn((L, T, H, D), wl.new_dtype, gen, device)
    v_hist = _randn((L, T, H, D), wl.new_dtype, gen, device)
    Q = wl.total_queries
    q = _randn((Q, wl.num_heads, D), wl.q_dtype, gen, device)
    k_new = _randn((L, Q, H, D), wl.new_dtype, gen, device)
    v_new = _randn((L, Q, H, D), wl.new_dtype, gen, device)
    return dict(k_hist=k_hist, v_hist=v_hist, q=q, k_new=k_new, v_new=v_new)
