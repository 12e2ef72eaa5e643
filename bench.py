"""Benchmark one paged GQA decode step on one MI355X.

A step is the whole hot path over one batch: the slot reservation of every
sequence's new token (host bookkeeping, kvc_append without rows), then
kvc_decode_attention with the new K/V rows, which writes them into their
slots and attends (for 16-bit caches the split-K kernel's walk writes them
itself; one-byte caches run the quantising append kernel first), then the
merge kernel.  ``--append kernel`` times the two-call form instead (kvc_append
with rows, its own kernel, then the decode).  The step is made repeatable by
truncating every sequence back to its history length afterwards (host
bookkeeping only, one kvc_truncate_many call), so every step appends into the
same slots.

Prints ONE JSON line: value = KV-read GB/s (distinct K/V bytes the step
attends / step time), plus us_per_step, the split kernel's roofline (HIP
events on the launch stream), the fp64 CPU oracle timed on a sample, the
plain copy kernel's bandwidth on the same box, the shader and memory clocks
seen while the steps ran, and -- on the default run -- the same measurements
for the other decode workloads (configs 2, 4, 4 with its shared prefix
attended once, and 5) under "also".

``--extend verify|prefill|chunk`` times a step with several new tokens per
sequence instead (kvc_append of all of them, then kvc_extend_attention), with
its own metric line; the roofline is HBM or the matrix cores, whichever the
workload's flops per algorithmic byte puts it under.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged GQA decode attn: µs/step, KV-read HBM GB/s and % of MI355X peak"
EVENT_EVERY = 4   # timed steps per HIP-event-bracketed split-kernel launch
PEAK_HBM_GBS = 8000.0
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: 70B-shaped GQA layer)")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--kernel", type=int, default=0, help="0 auto, 1 fp32 FMA, 2 MFMA")
    p.add_argument("--partition-tokens", type=int, default=0, help="FMA kernel partition size (0 auto)")
    p.add_argument("--work-items", type=int, default=0, help="MFMA kernel waves per KV head (0 auto)")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="time budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-calibrate", action="store_true", help="skip timing the plain copy kernel (2 GiB)")
    p.add_argument("--no-clocks", action="store_true", help="skip sampling the shader clock under load")
    p.add_argument("--no-also", action="store_true",
                   help="default run only: skip the extra workloads (configs 2, 4, 4 with the shared prefix "
                        "attended once, 5) measured after the headline one")
    p.add_argument("--append", choices=["fold", "kernel"], default="fold",
                   help="decode step's append: 'fold' = slots reserved without rows, the rows handed to the "
                        "decode (written by the decode walk itself for 16-bit caches); 'kernel' = kvc_append "
                        "with rows (its own kernel) before the decode")
    p.add_argument("--extend", choices=["verify", "prefill", "chunk"], default=None,
                   help="time a step with several new tokens per sequence instead of decode: the verify pass "
                        "of speculative decoding (5 draft tokens, 70B-shaped batch), a 2048-token causal "
                        "prefill, or a 512-token prefill chunk over 3584 cached tokens")
    p.add_argument("--pool-pieces", type=int, default=0,
                   help="MFMA decode: pieces of each run handed out at run time (0 = static split, the default)")
    p.add_argument("--pool-shift", type=int, default=0, help="MFMA decode: the pool is the last 1/2^shift of a run")
    p.add_argument("--shared-prefix", action="store_true",
                   help="decode: attend the workload's shared prefix once for the batch (cascade split)")
    p.add_argument("--extend-kernel", type=int, choices=[0, 2, 3], default=0,
                   help="several-token kernel: 0 auto, 2 rows split over waves, 3 one wave per 32 columns")
    p.add_argument("--tiles-per-wave", type=int, default=0,
                   help="--extend: 16-column tiles each wave holds (1..4, 0 auto)")
    p.add_argument("--kv", choices=["f32", "f16", "bf16", "fp8", "int8"], default=None,
                   help="cache dtype override for --config (e.g. --config 5 --kv int8: the mixed batch with an "
                        "int8 cache)")
    p.add_argument("--window", action="store_true",
                   help="time decode under a sliding window of 4096 over 16K-token contexts whose older blocks "
                        "were evicted (70B-shaped batch) instead of --config")
    return p.parse_args()


class TimingEvent:
    """A HIP event used only to time the kernels between two records on one
    stream.  Made with hipEventDisableSystemFence: its record takes no
    system-scope fence, so it does not write back and invalidate the caches
    between the kernels it brackets (default events do, and that cost ~6 us of
    every timed decode step).  Elapsed times are read after a device
    synchronize; the library records it through `cuda_event`, as it would a
    torch event's handle."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch has loaded
        h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self, stream_handle: int):
        rc = self._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    @staticmethod
    def pairs(n: int):
        """n (start, end) pairs, each recorded once on the current stream so
        that no first-use cost lands in a timed step."""
        import torch
        out = [(TimingEvent(), TimingEvent()) for _ in range(n)]
        h = torch.cuda.current_stream().cuda_stream
        for a, b in out:
            a.record(h)
            b.record(h)
        torch.cuda.synchronize()
        return out

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                           ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.cuda_event:
            self._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def algorithmic_bytes(wl):
    """Bytes the decode must move, per step (what the method reads and writes)."""
    eb = ELEM_BYTES[wl.kv_dtype]
    tokens = wl.history_rows + wl.batch            # distinct rows attended (shared prefix once)
    if wl.window:                                  # only the rows inside each window
        tokens = int(sum(min(int(n), wl.window) for n in wl.attend_lens))
    kv = 2 * tokens * wl.num_kv_heads * wl.head_dim * eb
    blocks_distinct = wl.num_blocks
    scales = 2 * 4 * blocks_distinct * wl.num_kv_heads if wl.kv_dtype in ("fp8", "int8") else 0
    qb = ELEM_BYTES[wl.q_dtype]
    q = wl.batch * wl.num_heads * wl.head_dim * qb
    out = q
    tables = 4 * sum((int(n) + 15) // 16 for n in wl.attend_lens) + 4 * wl.batch
    if wl.window:
        tables = 4 * sum((int(n) + 15) // 16 - max(0, int(n) - wl.window) // 16 for n in wl.attend_lens) + 4 * wl.batch
    append = 2 * wl.batch * wl.num_kv_heads * wl.head_dim * eb
    return dict(kv=kv, scales=scales, q=q, out=out, tables=tables, append=append,
                split_kernel=kv + scales + q + tables)


def workload_key(args):
    """The workload a run measures, as the profile summaries name it."""
    if args.extend:
        return f"extend {args.extend}"
    if args.window:
        return "window"
    return f"config {args.config}" + (f" kv {args.kv}" if args.kv else "")


def profiled_traffic(key, combined=False):
    """HBM bytes per split-kernel launch from a committed rocprofv3 summary
    (FETCH_SIZE and WRITE_SIZE passes scaled by a plain copy kernel's counts)
    of the workload `key`, or None when no summary was taken on the current
    sources (the kernels, and the host code that plans their launches).
    combined: the sum over every kernel the summary records for `key` (the
    shared-prefix decode times its prefix pass and its split kernel as one)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_split_amd", "csrc")
    try:
        sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                      for f in ("kvc_kernels.hip", "kvc_host.cpp"))).hexdigest()
    except OSError:
        return None
    total, source = 0, None
    for fn in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(fn).read()
        for line in text.splitlines():
            if line.startswith("{") and "traffic_bytes_per_launch" in line:
                try:
                    rec = json.loads(line)
                except ValueError:
                    continue
                if rec.get("workload_key") == key and rec.get("kernel_source_sha256") == sha:
                    if not combined:
                        return rec["traffic_bytes_per_launch"], os.path.relpath(fn, ROOT)
                    total += rec["traffic_bytes_per_launch"]
                    source = os.path.relpath(fn, ROOT)
    return (total, source) if source else None


def cpu_baseline(wl, values, budget_s):
    """Time the fp64 oracle on a sample of the same workload (sequences in order
    until the budget is spent); report GB/s of KV it processed and the cores it
    kept busy (process CPU time / wall time)."""
    import numpy as np
    import torch
    from oracle.attention import decode_attention
    lens = [int(x) for x in wl.context_lens]
    p = wl.shared_prefix
    q = values["q"].to(torch.float64).cpu().numpy()
    kh, vh = values["k_hist"], values["v_hist"]
    done_bytes, n_seq, wall, cpu = 0, 0, 0.0, 0.0
    start_row = p if p else 0
    for b in range(wl.batch):
        rows = (torch.cat([torch.arange(0, p), torch.arange(start_row, start_row + lens[b] - p)]) if p
                else torch.arange(start_row, start_row + lens[b]))
        start_row += lens[b] - p
        k = torch.cat([kh[0, rows.to(kh.device)], values["k_new"][0, b:b + 1]]).cpu()
        v = torch.cat([vh[0, rows.to(vh.device)], values["v_new"][0, b:b + 1]]).cpu()
        if wl.kv_dtype == "fp8":
            pass  # the oracle is timed on the unquantised rows (same arithmetic, same sizes)
        t0, c0 = time.perf_counter(), time.process_time()
        decode_attention(q[b], k.to(torch.float64).numpy(), v.to(torch.float64).numpy(), wl.scale)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        n_seq += 1
        done_bytes += 2 * (lens[b] + 1) * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
        if wall > budget_s:
            break
    all_bytes = sum(2 * (n + 1) * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype] for n in lens)
    return {"value": round(done_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            # the whole step (every sequence) at the sample's rate, beside the GPU's us_per_step
            "us_per_step": round(wall * all_bytes / done_bytes * 1e6, 1),
            "sample": f"{n_seq} of {wl.batch} sequences of the same workload ({done_bytes / 1e9:.3f} GB of KV, "
                      f"fp64 NumPy, {wall:.1f} s wall), one decode step each; "
                      f"os.cpu_count()={os.cpu_count()}"}


def cpu_baseline_window(wl, values, budget_s):
    """The fp64 oracle's windowed attention (one new token per sequence, over
    the rows of its window) on sequences of the same workload until the budget
    is spent; GB/s of KV in the windows it processed."""
    import numpy as np
    import torch
    from oracle.attention import extend_attention
    from workloads import history_rows_of
    q = values["q"].to(torch.float64).cpu().numpy()
    done_bytes, n_seq, wall, cpu = 0, 0, 0.0, 0.0
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        keep = min(L + 1, wl.window) - 1                  # history rows inside the window
        rows = torch.from_numpy(history_rows_of(wl, b)[L - keep:]).to(values["k_hist"].device)
        k = torch.cat([values["k_hist"][0, rows], values["k_new"][0, b:b + 1]]).to(torch.float64).cpu().numpy()
        v = torch.cat([values["v_hist"][0, rows], values["v_new"][0, b:b + 1]]).to(torch.float64).cpu().numpy()
        t0, c0 = time.perf_counter(), time.process_time()
        extend_attention(q[b:b + 1], k, v, wl.scale, window=wl.window)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        n_seq += 1
        done_bytes += 2 * (keep + 1) * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
        if wall > budget_s:
            break
    all_bytes = sum(2 * min(int(n) + 1, wl.window) * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
                    for n in wl.context_lens)
    return {"value": round(done_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "us_per_step": round(wall * all_bytes / done_bytes * 1e6, 1),
            "sample": f"{n_seq} of {wl.batch} sequences of the same workload ({done_bytes / 1e9:.3f} GB of KV in "
                      f"their windows, fp64 NumPy, {wall:.1f} s wall); os.cpu_count()={os.cpu_count()}"}


EXTEND_METRIC = "paged multi-token attention (causal among the new tokens): µs/step, KV-read GB/s, TFLOP/s"
PEAK_MFMA_TFLOPS = 2500.0   # dense bf16 / fp16 matrix-core peak


def extend_work(wl):
    """Algorithmic bytes and flops of one multi-token attention call: distinct
    K/V rows once, q, out, tables; 4 * D flops per (query token, head, visible
    row) -- QK^T and PV, counted on the definition (no causal padding)."""
    eb = ELEM_BYTES[wl.kv_dtype]
    rows = int(wl.attend_lens.sum())
    kv = 2 * rows * wl.num_kv_heads * wl.head_dim * eb
    scales = 2 * 4 * wl.num_blocks * wl.num_kv_heads if wl.kv_dtype in ("fp8", "int8") else 0
    q = wl.total_queries * wl.num_heads * wl.head_dim * ELEM_BYTES[wl.q_dtype]
    tables = 4 * sum((int(n) + 15) // 16 for n in wl.attend_lens) + 8 * wl.batch + 4
    visible = sum(int(ql) * (int(n) - int(ql)) + int(ql) * (int(ql) + 1) // 2
                  for n, ql in zip(wl.attend_lens, wl.q_lens))
    flops = 4 * wl.head_dim * wl.num_heads * visible
    return dict(kv=kv, bytes=kv + scales + 2 * q + tables, flops=flops)


def cpu_baseline_extend(wl, values, budget_s):
    """The fp64 oracle's multi-token attention on sequences of the same
    workload, in order, until the budget is spent; reported in TFLOP/s of the
    definition's work."""
    import numpy as np
    import torch
    from oracle.attention import extend_attention
    qs = np.concatenate([[0], np.cumsum(wl.q_lens)])
    lens = [int(x) for x in wl.context_lens]
    q = values["q"].to(torch.float64).cpu().numpy()
    done_flops, n_seq, wall, cpu, row = 0, 0, 0.0, 0.0, 0
    for b in range(wl.batch):
        hist = slice(row, row + lens[b])
        row += lens[b]
        k = torch.cat([values["k_hist"][0, hist], values["k_new"][0, qs[b]:qs[b + 1]]]).to(torch.float64).cpu()
        v = torch.cat([values["v_hist"][0, hist], values["v_new"][0, qs[b]:qs[b + 1]]]).to(torch.float64).cpu()
        t0, c0 = time.perf_counter(), time.process_time()
        extend_attention(q[qs[b]:qs[b + 1]], k.numpy(), v.numpy(), wl.scale)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        n_seq += 1
        ql, n = int(wl.q_lens[b]), lens[b] + int(wl.q_lens[b])
        done_flops += 4 * wl.head_dim * wl.num_heads * (ql * (n - ql) + ql * (ql + 1) // 2)
        if wall > budget_s:
            break
    all_flops = sum(4 * wl.head_dim * wl.num_heads * (int(ql) * int(L) + int(ql) * (int(ql) + 1) // 2)
                    for ql, L in zip(wl.q_lens, lens))
    return {"value": round(done_flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "us_per_step": round(wall * all_flops / done_flops * 1e6, 1),
            "sample": f"{n_seq} of {wl.batch} sequences of the same workload, fp64 NumPy, {wall:.1f} s wall; "
                      f"os.cpu_count()={os.cpu_count()}"}


def step_percentiles(step_ev):
    """Median and 95th percentile of single steps (events on the current
    stream around each step of a pass after the timed one), in microseconds."""
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in step_ev)
    p95 = us[min(len(us) - 1, int(round(0.95 * (len(us) - 1))))]
    return {"step_us_median": round(us[len(us) // 2], 2), "step_us_p95": round(p95, 2)}


def _dpm_files():
    """The power-management clock tables (sysfs) of the device torch uses:
    (shader clock file, memory clock file) or None."""
    import glob
    import torch
    prop = torch.cuda.get_device_properties(0)
    bus = getattr(prop, "pci_bus_id", None)
    cands = []
    if bus is not None:
        dom = getattr(prop, "pci_domain_id", 0) or 0
        dv = getattr(prop, "pci_device_id", 0) or 0
        cands.append(f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{dv:02x}.0")
    cands += sorted(os.path.dirname(p) for p in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    for d in cands:
        s, m = os.path.join(d, "pp_dpm_sclk"), os.path.join(d, "pp_dpm_mclk")
        if os.path.exists(s):
            return s, (m if os.path.exists(m) else None), d
    return None


def _read_dpm(path):
    """(levels in MHz, current level's MHz or None) of one pp_dpm_* table."""
    import re
    levels, cur = [], None
    try:
        for line in open(path).read().splitlines():
            m = re.search(r"(\d+)\s*Mhz(\s*\*)?", line, re.I)
            if m:
                levels.append(int(m.group(1)))
                if m.group(2):
                    cur = int(m.group(1))
    except OSError:
        return None, None
    return levels, cur


def sample_clocks_under_load(step, seconds=0.3):
    """Shader and memory clocks read from the power-management tables every
    ~2 ms while decode steps run back to back for `seconds`."""
    import threading
    import torch
    files = _dpm_files()
    if not files:
        return {"source": "no pp_dpm_sclk table readable"}
    sfile, mfile, dev_dir = files
    samples_s, samples_m, stop = [], [], threading.Event()

    def poll():
        while not stop.is_set():
            _, c = _read_dpm(sfile)
            if c is not None:
                samples_s.append(c)
            if mfile:
                _, cm = _read_dpm(mfile)
                if cm is not None:
                    samples_m.append(cm)
            time.sleep(0.002)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    stop.set()
    th.join()
    sl, _ = _read_dpm(sfile)
    ml, _ = _read_dpm(mfile) if mfile else (None, None)

    def summary(xs):
        xs = sorted(xs)
        return {"samples": len(xs), "min": xs[0], "median": xs[len(xs) // 2], "max": xs[-1]} if xs else None
    return {"source": dev_dir, "sclk_levels_mhz": sl, "mclk_levels_mhz": ml, "steps_run": n,
            "sclk_mhz_under_load": summary(samples_s), "mclk_mhz_under_load": summary(samples_m)}


def environment(clocks=None):
    """Software and device the numbers were taken on (and the clocks seen
    while the steps ran, when sampled)."""
    import torch
    prop = torch.cuda.get_device_properties(0)
    env = {"torch": torch.__version__, "hip": torch.version.hip, "device": prop.name,
           "arch": getattr(prop, "gcnArchName", None), "compute_units": prop.multi_processor_count,
           "memory_gib": round(prop.total_memory / 2 ** 30, 1)}
    if clocks is not None:
        env["clocks"] = clocks
    return env


def calibrate_copy(dev):
    """Time the plain 2 GiB copy kernel (its known bytes scale the profiler's
    HBM byte counters) and a plain streaming read of the same 2 GiB (the
    achievable read rate, the decode's own ceiling on this machine)."""
    import torch
    import paged_kv_cache_split_amd as kvc
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    kvc.stream_copy(dst, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        kvc.stream_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del dst
    # the achievable streaming read rate: every byte of 2 GiB read once
    sink = torch.empty(1 << 16, dtype=torch.uint32, device=dev)
    kvc.stream_read(src, sink)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        kvc.stream_read(src, sink)
    e1.record()
    torch.cuda.synchronize()
    ms_r = e0.elapsed_time(e1) / 5
    del src, sink
    return {"copy_bytes": n, "copy_read_plus_write_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "read_GBs": round(n / (ms_r * 1e-3) / 1e9, 1)}


def run_extend(args):
    import numpy as np
    import torch
    import paged_kv_cache_split_amd as kvc
    from workloads import make_extend_workload, make_values, setup_ops

    dev = "cuda"
    torch.cuda.set_device(0)
    wl = make_extend_workload(args.extend, seed=args.seed)
    print(f"[bench] extend {args.extend}: {wl.name}; blocks {wl.num_blocks}, {wl.total_queries} queries",
          file=sys.stderr, flush=True)
    values = make_values(wl, dev)
    cache = kvc.KVCache(wl.num_layers, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.kv_dtype, device=dev,
                        free_order=wl.free_order)
    row = 0
    for op in setup_ops(wl):
        if op[0] == "add":
            cache.add_seq(op[1], op[2])
        elif op[0] == "append":
            t = int(sum(op[2]))
            if t:
                cache.append(op[1], values["k_hist"][:, row:row + t].contiguous(),
                             values["v_hist"][:, row:row + t].contiguous(), n_new=op[2])
            row += t
    seqs = list(range(wl.batch))
    hist_len = [int(x) for x in wl.context_lens]
    n_new = [int(x) for x in wl.q_lens]
    k_new, v_new, q = values["k_new"].contiguous(), values["v_new"].contiguous(), values["q"].contiguous()
    cache.append(seqs, k_new, v_new, n_new=n_new)
    bt, cl = cache.export_tables(seqs)
    cache.truncate_many(seqs, hist_len)
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(wl.q_lens)]).astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    ws = torch.empty(max(256, kvc.extend_workspace_bytes(wl.batch, wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                                         wl.max_query_len, wl.max_context_len, args.work_items,
                                                         args.tiles_per_wave, args.extend_kernel)),
                     dtype=torch.uint8, device=dev)
    ev = TimingEvent.pairs((args.steps + EVENT_EVERY - 1) // EVENT_EVERY)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(events=None):
        cache.append(seqs, k_new, v_new, n_new=n_new)
        cache.extend(q, qs, wl.max_query_len, bt, cl, wl.max_context_len, wl.scale, out=out, workspace=ws,
                     work_items=args.work_items, split_events=events, tiles_per_wave=args.tiles_per_wave,
                     kernel=args.extend_kernel)
        cache.truncate_many(seqs, hist_len)

    # a full garbage-collector pass over the setup's objects inside the timed
    # loop costs tens of milliseconds: collect now and exempt what exists
    gc.collect()
    gc.freeze()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i // EVENT_EVERY] if i % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-step percentiles from a second pass, so the markers do not touch the timed region
    for i in range(args.steps):
        step_ev[i][0].record()
        step()
        step_ev[i][1].record()
    torch.cuda.synchronize()
    split_ms = sorted(a.elapsed_time(b) for a, b in ev)
    step_stats = step_percentiles(step_ev)
    split_avg_ms = sum(split_ms) / len(split_ms)
    ms_per_step = wall * 1e3 / args.steps
    w = extend_work(wl)
    intensity = w["flops"] / w["bytes"]
    mfma_bound = intensity > PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = w["flops"] / (split_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_TFLOPS, 4)}
    else:
        achieved = w["bytes"] / (split_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    prof = (profiled_traffic(workload_key(args))
            if not args.work_items and not args.tiles_per_wave and not args.extend_kernel else None)
    roof.update({"traffic": prof[0] if prof else None, "traffic_source": prof[1] if prof else None,
                 "kernel": "multi-token split-K kernel", "avg_launch_us": round(split_avg_ms * 1e3, 2),
                 "median_launch_us": round(split_ms[len(split_ms) // 2] * 1e3, 2),
                 "algorithmic_bytes_per_launch": w["bytes"], "algorithmic_flops_per_launch": w["flops"],
                 "intensity_flop_per_byte": round(intensity, 1)})
    kv_gbs = w["kv"] / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": EXTEND_METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "tflops_step": round(w["flops"] / (ms_per_step * 1e-3) / 1e12, 2),
        "pct_of_peak_hbm": round(100.0 * kv_gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, seeded lengths and block placement)",
        "config": {"workload": wl.name, "extend": args.extend, "batch": wl.batch, "num_heads": wl.num_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "new_tokens": wl.total_queries, "rows_attended": int(wl.attend_lens.sum()), "kv_bytes": w["kv"],
                   "kernel": {0: "auto", 2: "rows split over waves", 3: "one wave per 32 columns"}[args.extend_kernel],
                   "work_items": args.work_items or "auto", "tiles_per_wave": args.tiles_per_wave or "auto",
                   "parallelism": "single GPU"},
        "roofline": roof,
        **step_stats,
        "env": environment(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_extend(wl, values, args.cpu_seconds)
    if not args.no_calibrate:
        result["calibration"] = calibrate_copy(dev)
    print(json.dumps(result), flush=True)


def build_decode_cache(wl, dev):
    """The workload's cache with its history written through the library."""
    import paged_kv_cache_split_amd as kvc
    from workloads import make_values, setup_ops
    values = make_values(wl, dev)
    cache = kvc.KVCache(wl.num_layers, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.kv_dtype, device=dev,
                        free_order=wl.free_order)
    row = 0
    for op in setup_ops(wl):
        if op[0] == "add":
            cache.add_seq(op[1], op[2])
        elif op[0] == "fork":
            cache.fork(op[1], op[2])
        elif op[0] == "evict":
            cache.evict(op[1], op[2])
        else:
            t = int(sum(op[2]))
            cache.append(op[1], values["k_hist"][:, row:row + t].contiguous(),
                         values["v_hist"][:, row:row + t].contiguous(), n_new=op[2])
            row += t
    return cache, values


def time_decode(wl, values, cache, o, steps, warmup, dev, load_clock=False):
    """Time `steps` decode steps of one workload (after `warmup` untimed ones).

    A step: the slot reservation and append of every sequence's new token,
    the decode (split-K kernel and merge), and the host rollback that makes the
    next step append into the same slots.  With o.append == "fold" the append
    is kvc_append without rows plus the rows handed to the decode, which
    writes them itself (16-bit caches) or runs the append kernel first;
    with "kernel" it is kvc_append with rows (its own kernel), then the
    decode."""
    import torch
    import paged_kv_cache_split_amd as kvc
    seqs = list(range(wl.batch))
    hist_len = [int(x) for x in wl.context_lens]
    k_new, v_new, q = values["k_new"].contiguous(), values["v_new"].contiguous(), values["q"].contiguous()
    k_row, v_row = k_new[0].contiguous(), v_new[0].contiguous()
    # tables as they are after the step's append (the decode reads L+1 tokens)
    cache.append(seqs, k_new, v_new)
    bt, cl = cache.export_tables(seqs)
    cache.truncate_many(seqs, hist_len)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    prefix = wl.shared_prefix if o.shared_prefix else 0
    ws = torch.empty(max(256, kvc.decode_workspace_bytes(wl.batch, wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                                         wl.max_context_len, o.partition_tokens, o.kernel,
                                                         o.work_items, o.pool_pieces, o.pool_shift, prefix)),
                     dtype=torch.uint8, device=dev)
    # HIP events bracket the split kernel of every EVENT_EVERY-th timed step:
    # each record is a packet the GPU processes between kernels (~2 us), so
    # bracketing every launch would add ~4 us to every timed step
    ev = TimingEvent.pairs((steps + EVENT_EVERY - 1) // EVENT_EVERY)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    fold = o.append == "fold"

    def step(events=None):
        if fold:
            cache.append(seqs, None, None)
        else:
            cache.append(seqs, k_new, v_new)
        cache.decode(q, bt, cl, wl.max_context_len, wl.scale, out=out, workspace=ws, kernel=o.kernel,
                     partition_tokens=o.partition_tokens, work_items=o.work_items, split_events=events,
                     window=wl.window, pool_pieces=o.pool_pieces, pool_shift=o.pool_shift, shared_prefix=prefix,
                     k_new=k_row if fold else None, v_new=v_row if fold else None)
        cache.truncate_many(seqs, hist_len)

    # a full garbage-collector pass over the setup's objects inside the timed
    # loop costs tens of milliseconds: collect now and exempt what exists
    gc.collect()
    gc.freeze()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i // EVENT_EVERY] if i % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-step percentiles from a second pass, so the markers do not touch the timed region
    for i in range(steps):
        step_ev[i][0].record()
        step()
        step_ev[i][1].record()
    torch.cuda.synchronize()
    clocks = sample_clocks_under_load(step) if load_clock else None
    gc.unfreeze()
    split_ms = sorted(a.elapsed_time(b) for a, b in ev)
    split_avg_ms = sum(split_ms) / len(split_ms)
    ms_per_step = wall * 1e3 / steps
    ab = algorithmic_bytes(wl)
    if fold and wl.kv_dtype in ("f16", "bf16") and o.kernel in (0, 2) and not o.pool_pieces:
        # the walk also reads the new rows and writes them into their slots
        ab["split_kernel"] += 2 * ab["append"]
    kv_gbs = ab["kv"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["split_kernel"] / (split_avg_ms * 1e-3) / 1e9
    return dict(ms_per_step=ms_per_step, kv_gbs=kv_gbs, ab=ab, achieved=achieved, split_avg_ms=split_avg_ms,
                split_median_ms=split_ms[len(split_ms) // 2], step_stats=step_percentiles(step_ev), clocks=clocks)


class DecodeOpts:
    def __init__(self, args, shared_prefix=None):
        self.kernel, self.partition_tokens, self.work_items = args.kernel, args.partition_tokens, args.work_items
        self.pool_pieces, self.pool_shift = args.pool_pieces, args.pool_shift
        self.shared_prefix = args.shared_prefix if shared_prefix is None else shared_prefix
        self.append = args.append


def also_entry(cid, shared_prefix, args, dev):
    """A compact record of another decode workload measured in the same process."""
    import torch
    from workloads import make_workload
    wl = make_workload(cid)
    print(f"[bench] also: config {cid}{' shared prefix' if shared_prefix else ''}: {wl.name}", file=sys.stderr,
          flush=True)
    cache, values = build_decode_cache(wl, dev)
    o = DecodeOpts(args, shared_prefix=shared_prefix)
    r = time_decode(wl, values, cache, o, args.steps, args.warmup, dev)
    key = f"config {cid}"
    prof = ((profiled_traffic(key + " shared prefix", combined=True) if shared_prefix else profiled_traffic(key))
            if o.kernel in (0, 2) else None)
    entry = {"workload": wl.name, "config_id": cid, "shared_prefix": wl.shared_prefix if shared_prefix else 0,
             "dtype": wl.kv_dtype, "us_per_step": round(r["ms_per_step"] * 1e3, 2), "value": round(r["kv_gbs"], 2),
             "unit": "GB/s", "pct_of_peak_hbm": round(100.0 * r["kv_gbs"] / PEAK_HBM_GBS, 2),
             "kv_bytes": r["ab"]["kv"],
             "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(r["achieved"] / PEAK_HBM_GBS, 4),
                          "kernel": "decode split-K kernel" + (" (prefix pass + own rows)" if shared_prefix else ""),
                          "avg_launch_us": round(r["split_avg_ms"] * 1e3, 2),
                          "traffic": prof[0] if prof else None, "traffic_source": prof[1] if prof else None},
             **r["step_stats"]}
    del cache, values
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path here is single-GPU by design "
              f"(--gpus {args.gpus} requested); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.extend:
        run_extend(args)
        return
    import torch
    from workloads import make_window_workload, make_workload

    dev = "cuda"
    torch.cuda.set_device(0)
    over = {"kv_dtype": args.kv} if args.kv else {}
    wl = make_window_workload() if args.window else make_workload(args.config, seed=args.seed, **over)
    print(f"[bench] {'window' if args.window else 'config %d' % args.config}: {wl.name}; blocks {wl.num_blocks}, "
          f"attended tokens {int(wl.attend_lens.sum())}", file=sys.stderr, flush=True)
    if args.shared_prefix and not wl.shared_prefix:
        raise SystemExit("--shared-prefix needs a workload with a shared prefix (config 4)")
    cache, values = build_decode_cache(wl, dev)
    o = DecodeOpts(args)
    r = time_decode(wl, values, cache, o, args.steps, args.warmup, dev, load_clock=not args.no_clocks)
    print(f"[bench] timed {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    prefix = wl.shared_prefix if args.shared_prefix else 0
    ab, ms_per_step, kv_gbs, achieved = r["ab"], r["ms_per_step"], r["kv_gbs"], r["achieved"]
    prof = None
    if args.kernel in (0, 2) and not args.work_items and not args.pool_pieces:
        prof = (profiled_traffic(workload_key(args) + " shared prefix", combined=True) if args.shared_prefix
                else profiled_traffic(workload_key(args)))
    traffic = prof[0] if prof else None
    result = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak_hbm": round(100.0 * kv_gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-e4m3 kv / bf16 q", "int8": "int8 kv / bf16 q"}.get(wl.kv_dtype, wl.kv_dtype),
        "data": "synthetic (seeded N(0,1) K/V/q, seeded lengths and block placement)",
        "config": {"workload": wl.name, "config_id": None if args.window else args.config, "window": wl.window,
                   "batch": wl.batch, "num_heads": wl.num_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "attended_tokens": int(wl.attend_lens.sum()), "kv_bytes": ab["kv"],
                   "kernel": ["auto", "fma", "mfma"][args.kernel], "partition_tokens": args.partition_tokens or "auto",
                   "work_items": args.work_items or "auto", "pool_pieces": args.pool_pieces,
                   "shared_prefix": prefix, "append": args.append, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     # with a shared prefix: the prefix pass and the own-rows decode together, over the
                     # same unique bytes as the plain decode (the prefix counted once in both)
                     "kernel": "decode split-K kernel" + (" (prefix pass + own rows)" if prefix else ""),
                     "avg_launch_us": round(r["split_avg_ms"] * 1e3, 2),
                     "median_launch_us": round(r["split_median_ms"] * 1e3, 2),
                     "algorithmic_bytes_per_launch": ab["split_kernel"],
                     "traffic_source": prof[1] if prof else None},
        **r["step_stats"],
        "env": environment(r["clocks"]),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = (cpu_baseline_window(wl, values, args.cpu_seconds) if wl.window
                                  else cpu_baseline(wl, values, args.cpu_seconds))
    del cache, values
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_calibrate:
        cal = calibrate_copy(dev)
        cal["kv_read_pct_of_read_GBs"] = round(100.0 * kv_gbs / cal["read_GBs"], 2)
        cal["split_kernel_pct_of_read_GBs"] = round(100.0 * achieved / cal["read_GBs"], 2)
        result["calibration"] = cal
    default_run = (not args.window and args.config == 3 and not args.kv and args.seed is None and not args.kernel
                   and not args.work_items and not args.pool_pieces and not args.shared_prefix
                   and not args.partition_tokens and args.append == "fold")
    if default_run and not args.no_also:
        result["also"] = [also_entry(cid, sp, args, dev) for cid, sp in ((2, False), (4, False), (4, True), (5, False))]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
