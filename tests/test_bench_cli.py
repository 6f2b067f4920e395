"""Host-side checks of bench.py (no GPU): the one-GPU contract and the link
between the committed counter summary and the decode kernel sources."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GQA_KV_BYTES = 8 * 8 * 4096 * 128 * 2 * 2  # B x H_kv x keys x d x bf16 x (K and V)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line for an unmeasured configuration


def test_committed_counter_summary_matches_the_decode_sources():
    """The PMC summary under profiles/ was taken on the current decode kernel, so
    the benchmark's roofline.traffic is filled (it is null once the sources change)."""
    t = bench.read_traffic("gqa-decode")
    assert t is not None, "profiles/decode_partial_gqa-decode_pmc.md is stale or missing"
    # every valid K and V row once, plus line-granularity slack; writes are the
    # partial records and the output (well under 1% of the stream)
    assert 1.0 <= t["fetch_bytes_per_launch"] / GQA_KV_BYTES < 1.05
    assert t["write_bytes_per_launch"] < 0.01 * GQA_KV_BYTES


def test_digest_changes_with_the_sources(tmp_path, monkeypatch):
    d0 = bench.kernel_source_digest()
    src = os.path.join(tmp_path, "local_linear_attention_amd", "csrc")
    os.makedirs(src)
    for f in ("decode.hip", "device_common.h"):
        with open(os.path.join(ROOT, "local_linear_attention_amd", "csrc", f)) as fh:
            text = fh.read()
        with open(os.path.join(src, f), "w") as fh:
            fh.write(text + ("\n// edited\n" if f == "decode.hip" else ""))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_digest() != d0
