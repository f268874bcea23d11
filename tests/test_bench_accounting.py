"""Host-side accounting of bench.py: unique K/V bytes and the one-GPU rule (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_268_amd import workloads as W  # noqa: E402


def brute_unique_tokens(tables, lens, bs):
    """Token slots of distinct blocks, a block counted by the most slots any sequence uses."""
    most = {}
    for s, n in enumerate(lens):
        for t in range(int(n)):
            b = int(tables[s, t // bs])
            most[b] = max(most.get(b, 0), t % bs + 1)
    return sum(most.values())


def test_unique_bytes_hand_case():
    # Two sequences share block 7 (full) and block 3 (partly used by both); one private block each.
    bs, tok = 4, 10
    tables = np.array([[7, 3, 5], [7, 3, 9]], dtype=np.int32)
    lens = np.array([10, 6], dtype=np.int32)          # blocks 7 (4), 3 (4 / 2), 5 (2) | 7 (4), 3 (2)
    assert bench.unique_kv_bytes(tables, lens, bs, tok) == (4 + 4 + 2) * tok
    assert bench.unique_kv_bytes(tables, np.array([0, 0], dtype=np.int32), bs, tok) == 0


def test_unique_bytes_equal_logical_without_sharing():
    wl = W.config(3)
    tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    assert bench.unique_kv_bytes(wl.block_tables, wl.context_lens, wl.block_size, tok) == \
        int(wl.context_lens.sum()) * tok


def test_unique_bytes_shared_prefix_config_matches_brute_force():
    wl = W.config(5)
    sub = slice(0, 48)                                  # six groups of eight: shared prefixes and long members
    tables, lens = wl.block_tables[sub], wl.context_lens[sub]
    got = bench.unique_kv_bytes(tables, lens, wl.block_size, 1)
    assert got == brute_unique_tokens(tables, lens, wl.block_size)
    assert got < int(lens.sum())                        # the prefixes are counted once


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_carried_over_only_for_same_sources_and_workload(tmp_path, monkeypatch):
    """roofline.traffic: the committed counters' traffic per algorithmic byte, applied to this
    run's algorithmic bytes, only while the kernel sources hash to the recorded value and the
    summary was taken on the same workload (any step counts)."""
    import bench
    f = tmp_path / "summary.txt"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(f))
    body = ("# comment: with a colon\n"
            "workload_args: --config 3 --steps 50 --warmup 10\n"
            f"kernel_sources_sha256: {bench.kernel_sources_sha256()}\n"
            "traffic_bytes_per_launch: 1010\n"
            "algorithmic_bytes_per_launch: 1000\n")
    f.write_text(body)
    assert bench.measured_traffic(3, 2_000_000) == 2_020_000
    assert bench.measured_traffic(5, 2_000_000) is None
    f.write_text(body.replace(bench.kernel_sources_sha256(), "0" * 64))
    assert bench.measured_traffic(3, 2_000_000) is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic(3, 2_000_000) is None
