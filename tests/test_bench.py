"""bench.py's reporting logic on the CPU: the algorithmic byte counts its
rooflines divide by, the traffic lookup's source check, and the refusal of
more than one GPU."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes():
    # q, k, v bf16 (3 x 256) + alpha fp32 (512) + beta (4) + o fp32 (512)
    assert bench.layer_bytes("channel") == 1796
    assert bench.layer_bytes("head") == 1796 - 512 + 4
    # the 64 KiB state read and written, plus one token's inputs and output
    assert bench.decode_bytes("channel") == 2 * 65536 + 1796
    assert bench.decode_bytes("head") == 2 * 65536 + 1288
    assert bench.verify_bytes(2) == 3 * 65536 + 2 * 1796
    # q, k, v, alpha, beta, dO read; dq, dk, dv, dalpha (fp32) and dbeta written
    assert bench.backward_bytes() == 768 + 512 + 4 + 512 + 4 * 512 + 4


def test_kernel_bytes_follow_the_record_size():
    rb = bench.record_bytes_per_token(128)
    assert rb == 1736  # 111,104-byte record per 64-token chunk and head
    kb = bench.kernel_bytes(128)
    assert kb["chunk_local_kernel"] == 512 + 512 + 4 + rb
    assert kb["chunk_state_kernel"] == rb + 256 + 512


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_SUMMARY) as f:
        summary = json.load(f)
    k = summary["kernels"]["chunk_state_kernel"]
    # the committed summary was taken on the committed kernel source
    assert bench._traffic("chunk_state_kernel", "prefill_4k") == k["fetch_bytes"] + k["write_bytes"]
    assert bench._traffic("chunk_state_kernel", "varlen_8seq") is None
    other = tmp_path / "kda_prefill.hip"
    other.write_text("// another kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(other))
    assert bench._traffic("chunk_state_kernel", "prefill_4k") is None


def test_decode_traffic_matches_its_algorithmic_bytes():
    # the committed decode summary was taken on the committed decode source;
    # its counters read within 1% of the algorithmic bytes of a B=256 step
    t = bench._traffic("decode_kernel", "decode_b256", bench.DECODE_TRAFFIC_SUMMARY, bench.DECODE_SOURCE)
    assert t is not None
    algorithmic = 256 * 32 * bench.decode_bytes("channel")
    assert abs(t / algorithmic - 1) < 0.01
    assert bench._traffic("decode_kernel", "decode_b1024", bench.DECODE_TRAFFIC_SUMMARY,
                          bench.DECODE_SOURCE) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
