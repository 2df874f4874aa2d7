"""Host-side checks of bench.py: the one-GPU contract, the FLOP count and the
counter-traffic lookup (no GPU needed)."""

import os
import subprocess
import sys

import numpy as np

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_causal_pair_count_matches_the_oracle_mask():
    for nq, nk, off in ((1, 1, 0), (7, 7, 0), (5, 9, 4), (9, 5, -4), (64, 300, 236)):
        # brute force: row i (position i + off) sees keys j <= i + off
        mask = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + off
        assert bench.causal_pairs(nq, nk, off) == int(mask.sum())
        assert bench.causal_pairs(nq, nk, off) == oracle.visible_pairs(nq, nk, True, off)
    # 4k causal prefill: N(N+1)/2 pairs per head, 4d flops per pair
    assert bench.prefill_flops(1, 32, 4096, 128) == 4.0 * 128 * 32 * 4096 * 4097 / 2


def test_counter_traffic_is_null_for_other_sources():
    got = bench.counter_traffic("prefill_4k", "prefill_bf16_kernel<128,true,false>",
                                ["common.h", "prefill_bf16.hip"])
    assert got is None or (isinstance(got, int) and got > 0)
    assert bench.counter_traffic("prefill_4k", "prefill_bf16_kernel<128,true,false>",
                                 ["common.h", "kv_cache.hip"]) is None
    assert bench.counter_traffic("no_such_stage", "x", ["common.h"]) is None


def test_fingerprint_covers_code_not_comments(tmp_path, monkeypatch):
    base = "// a kernel\nint f(int x) {\n  return x + 1;  // add one\n}\n"
    (tmp_path / "a.hip").write_text(base)
    (tmp_path / "b.hip").write_text("/* reworded\n   header */\n// other words\n\nint f(int x) {\n"
                                    "  return x + 1;  // plus one\n\n}\n")
    (tmp_path / "c.hip").write_text(base.replace("x + 1", "x + 2"))
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    fa = bench.source_fingerprint(["a.hip"])
    assert fa == bench.source_fingerprint(["b.hip"])
    assert fa != bench.source_fingerprint(["c.hip"])
    assert len(fa) == 16


def test_counter_traffic_reads_only_a_matching_fingerprint(tmp_path, monkeypatch):
    (tmp_path / "k.hip").write_text("int k() { return 3; }\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    fp = bench.source_fingerprint(["k.hip"])
    summary = tmp_path / "traffic.md"
    summary.write_text(
        "# notes\n"
        f"traffic st kern<1,2> bytes_per_launch=1234 read_bytes=1000 write_bytes=234 sources_sha256={fp}\n"
        "traffic st other bytes_per_launch=9 read_bytes=9 write_bytes=0 sources_sha256=0000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.counter_traffic("st", "kern<1,2>", ["k.hip"]) == 1234
    assert bench.counter_traffic("st", "other", ["k.hip"]) is None  # stale fingerprint
    assert bench.counter_traffic("st2", "kern<1,2>", ["k.hip"]) is None
    (tmp_path / "k.hip").write_text("int k() { return 4; }\n")  # the kernel changed
    assert bench.counter_traffic("st", "kern<1,2>", ["k.hip"]) is None
