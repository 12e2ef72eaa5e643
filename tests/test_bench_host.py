"""Host-side checks of bench.py's accounting and its command line (no GPU).

The byte counts behind the reported GB/s and roofline fraction are pinned to
closed forms written out from the workload shapes: K and V rows of every
distinct token attended (a shared prefix counted once), the per-(block, KV
head) scales of one-byte caches, the queries and the block-table entries.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_window_workload, make_workload  # noqa: E402


def test_kv_bytes_count_a_shared_prefix_once():
    # 16 sequences of 32768 cached tokens, the first 4096 shared, plus one new
    # token each; 8 KV heads of 128 bf16 values for K and for V
    wl = make_workload(4)
    tokens = 4096 + 16 * (32768 - 4096) + 16
    assert bench.algorithmic_bytes(wl)["kv"] == 2 * tokens * 8 * 128 * 2


def test_split_kernel_bytes_add_scales_queries_and_tables():
    wl = make_workload(5)                       # fp8 cache: one fp32 scale per (block, KV head) for K and V
    ab = bench.algorithmic_bytes(wl)
    lens = [int(n) for n in wl.context_lens]
    assert ab["kv"] == 2 * (sum(lens) + wl.batch) * 8 * 128 * 1
    assert ab["scales"] == 2 * 4 * wl.num_blocks * 8
    assert ab["q"] == wl.batch * 64 * 128 * 2
    assert ab["tables"] == 4 * sum((n + 1 + 15) // 16 for n in lens) + 4 * wl.batch
    assert ab["split_kernel"] == ab["kv"] + ab["scales"] + ab["q"] + ab["tables"]


def test_window_bytes_cover_only_the_rows_inside_each_window():
    # 64 sequences of 16384 cached tokens + 1 new, each token seeing the last 4096
    wl = make_window_workload("decode")
    ab = bench.algorithmic_bytes(wl)
    assert ab["kv"] == 2 * (64 * 4096) * 8 * 128 * 2
    # table entries: the blocks holding the window's rows (16385 - 4096 = 12289 rows before
    # it, 768 whole blocks of them skipped), plus one length per sequence
    assert ab["tables"] == 4 * 64 * ((16385 + 15) // 16 - 12289 // 16) + 4 * 64


def test_profiled_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    src_dir = tmp_path / "paged_kv_cache_split_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "kvc_kernels.hip").write_bytes(b"// kernel source A\n")
    (src_dir / "kvc_host.cpp").write_bytes(b"// host source A\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    import hashlib
    sha_a = hashlib.sha256(b"// kernel source A\n// host source A\n").hexdigest()
    rec = {"workload_key": "config 3", "kernel_source_sha256": sha_a, "traffic_bytes_per_launch": 123}
    (prof / "k.md").write_text("# summary\n\n```\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("config 3") == (123, os.path.join("profiles", "k.md"))
    assert bench.profiled_traffic("config 4") is None
    (src_dir / "kvc_host.cpp").write_bytes(b"// host source B\n")      # the launch planning changed since
    assert bench.profiled_traffic("config 3") is None
    (src_dir / "kvc_host.cpp").write_bytes(b"// host source A\n")
    (src_dir / "kvc_kernels.hip").write_bytes(b"// kernel source B\n")   # the kernel changed since
    assert bench.profiled_traffic("config 3") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profiled_traffic_matches_sources_and_sums_a_shared_prefix(tmp_path, monkeypatch):
    # summaries count only for the sources they were taken on; the
    # shared-prefix decode times its prefix pass and split kernel as one, so
    # its traffic is the sum of both kernels' records
    import hashlib
    csrc = tmp_path / "paged_kv_cache_split_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "kvc_kernels.hip").write_bytes(b"kernels")
    (csrc / "kvc_host.cpp").write_bytes(b"host")
    sha = hashlib.sha256(b"kernelshost").hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    recs = [{"kernel": "a", "workload_key": "config 4 shared prefix", "kernel_source_sha256": sha,
             "traffic_bytes_per_launch": 100},
            {"kernel": "b", "workload_key": "config 4 shared prefix", "kernel_source_sha256": sha,
             "traffic_bytes_per_launch": 23},
            {"kernel": "b", "workload_key": "config 3", "kernel_source_sha256": "0" * 64,
             "traffic_bytes_per_launch": 7}]
    (prof / "x.md").write_text("# x\n\n```\n" + "\n".join(json.dumps(r) for r in recs) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("config 4 shared prefix", combined=True) == (123, os.path.join("profiles", "x.md"))
    assert bench.profiled_traffic("config 4 shared prefix") == (100, os.path.join("profiles", "x.md"))
    assert bench.profiled_traffic("config 3") is None          # taken on other sources
    assert bench.profiled_traffic("config 2", combined=True) is None
