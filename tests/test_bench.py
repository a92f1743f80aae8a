"""bench.py's reporting logic on the CPU: the algorithmic byte counts its
rooflines divide by, the traffic lookup's source check, and the refusal of
more than one GPU."""

import json
import os
import subprocess
import sys

import pytest

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
    # scalar gate: k and q exact (1 KiB fragments) plus two per-token factors:
    # 16 + 16 + 32 + 12 KiB + 512 + 512 B = 78,848 B per chunk
    assert bench.exact_record_bytes_per_token(128) == 78848 / 64
    assert bench.kernel_bytes(128, "head")["chunk_state_kernel"] == 78848 / 64 + 256 + 512


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    import hashlib
    src = tmp_path / "kda_prefill.hip"
    src.write_text("// a kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    summary = tmp_path / "traffic.json"
    summary.write_text(json.dumps({"workload": "prefill_4k", "source_sha256": sha, "kernels": {
        "chunk_state_kernel": {"fetch_bytes": 3.0, "write_bytes": 4.0}}}))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    assert bench._traffic("chunk_state_kernel", "prefill_4k") == 7.0
    assert bench._traffic("chunk_state_kernel", "varlen_8seq") is None
    assert bench._traffic("chunk_local_kernel", "prefill_4k") is None
    src.write_text("// another kernel source\n")
    assert bench._traffic("chunk_state_kernel", "prefill_4k") is None


@pytest.mark.parametrize("B", [256, 1024])
def test_decode_traffic_matches_its_algorithmic_bytes(B):
    # each committed decode summary was taken on the committed decode source;
    # its counters read within 1% of the algorithmic bytes of one step at B
    t = bench._traffic("decode_kernel", "decode_b%d" % B, bench.DECODE_TRAFFIC_SUMMARY % B, bench.DECODE_SOURCE)
    assert t is not None
    algorithmic = B * 32 * bench.decode_bytes("channel")
    assert abs(t / algorithmic - 1) < 0.01
    # a summary answers only for its own batch
    other = 1024 if B == 256 else 256
    assert bench._traffic("decode_kernel", "decode_b%d" % other, bench.DECODE_TRAFFIC_SUMMARY % B,
                          bench.DECODE_SOURCE) is None


def test_verify_traffic_matches_its_algorithmic_bytes():
    # speculative verification (B=256, two tokens, state history): the counters
    # of the verify kernel read within 1% of the state read once, two states
    # written and the tokens' inputs and outputs
    t = bench._traffic("decode_tokens_kernel", "verify_b256_k2", bench.VERIFY_TRAFFIC_SUMMARY % (256, 2),
                       bench.DECODE_SOURCE)
    assert t is not None
    assert abs(t / (256 * 32 * bench.verify_bytes(2)) - 1) < 0.01


def test_multi_token_decode_traffic_matches_its_algorithmic_bytes():
    # four tokens per sequence per call at B=256: the state read and written
    # once, the four tokens' inputs read and outputs written, within 1%
    B, K, H = 256, 4, 32
    t = bench._traffic("decode_tokens_kernel", "decode_tokens_b%d_k%d" % (B, K),
                       bench.DECODE_TOKENS_TRAFFIC_SUMMARY % (B, K), bench.DECODE_SOURCE)
    assert t is not None
    assert abs(t / (B * H * (2 * 128 * 128 * 4 + K * (768 + 512 + 4 + 512))) - 1) < 0.01


def test_verify_by_recomputation_traffic_matches_its_algorithmic_bytes():
    # a round of verify_tokens + accept_tokens (B=256, two tokens, the seeded
    # accepted counts of the bench: 182 accepting sequences) moves within 1%
    # of its algorithmic bytes, and fewer than the history round (verify with
    # the history, then commit)
    B, K, H, acc = 256, 2, 32, 182
    t = bench._round_traffic(B, K)
    assert t is not None
    state, tok = 128 * 128 * 4, K * (768 + 512 + 4 + 512)
    algorithmic = B * H * (state + tok) + acc * H * (2 * state + K * (768 + 512 + 4))
    assert abs(t / algorithmic - 1) < 0.01
    hist = (bench._traffic("decode_tokens_kernel", "verify_b256_k2", bench.VERIFY_TRAFFIC_SUMMARY % (B, K),
                           bench.DECODE_SOURCE)
            + bench._traffic("commit_kernel", "verify_b256_k2", bench.VERIFY_TRAFFIC_SUMMARY % (B, K),
                             bench.DECODE_SOURCE))
    assert t < 0.6 * hist


def test_fused_round_traffic_matches_its_algorithmic_bytes():
    # accept + verify in one pass: the state read once and written once for
    # an accepting sequence (182 of 256 in the bench's seeded counts)
    B, K, H, acc = 256, 2, 32, 182
    t = bench._traffic("decode_tokens_kernel", "verify_fused_b%d_k%d" % (B, K),
                       bench.VERIFY_FUSED_TRAFFIC_SUMMARY % (B, K), bench.DECODE_SOURCE)
    assert t is not None
    state = 128 * 128 * 4
    algorithmic = B * H * (state + K * (768 + 512 + 4 + 512)) + acc * H * (state + K * (768 + 512 + 4))
    assert abs(t / algorithmic - 1) < 0.01
    assert t < 0.8 * bench._round_traffic(B, K)


@pytest.mark.parametrize("suffix", ["_head", "_preact"])
def test_prefill_variants_have_their_own_counter_summaries(suffix):
    # the scalar-gate and pre-activation prefills are profiled on their own
    # runs (bench.py --only prefill_head / prefill_preact): each summary
    # answers for its variant only, on the committed prefill source
    issued = bench._mfma_issued("prefill_4k", suffix)
    assert issued is not None and issued["chunk_state_kernel"] > 0 and issued["chunk_local_kernel"] > 0
    t = bench._traffic("chunk_state_kernel", "prefill_4k" + suffix,
                       bench._variant_path(bench.TRAFFIC_SUMMARY, suffix))
    assert t is not None
    assert bench._traffic("chunk_state_kernel", "prefill_4k", bench._variant_path(bench.TRAFFIC_SUMMARY, suffix)) is None


def test_backward_traffic_is_summarised_for_both_kernels():
    # the backward summary covers both of its kernels on the committed source;
    # its bytes exceed the layer's algorithmic 3,848 per token and head (the
    # checkpoints and the per-slice partial rows make a round trip through HBM)
    parts = [bench._traffic(k, "prefill_4k", bench.BACKWARD_TRAFFIC_SUMMARY, bench.BACKWARD_SOURCE)
             for k in ("bwd_kernel", "bwd_reduce_kernel")]
    assert None not in parts
    assert sum(parts) > 4096 * 32 * bench.backward_bytes()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_roofline_uses_the_layer_bytes():
    """roofline.achieved = 1,796 B per token-head x token-heads of one call /
    the dominant kernel's time; the kernels' own record traffic is reported
    separately."""
    pf = {"total_tokens": 4096, "H": 32, "D": 128, "ms": 0.25,
          "phases_ms": {"chunk_local": 0.10, "state_pass": 0.14}}
    s = bench.prefill_summary(pf, "channel")
    r = s["roofline"]
    assert r["kernel"] == "chunk_state_kernel" and r["bytes_per_token_head"] == 1796
    assert abs(r["achieved"] - 4096 * 32 * 1796 / 0.14e-3 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12
    assert s["kernels"]["chunk_state_kernel"]["own_bytes_per_token_head"] == bench.kernel_bytes(128)[
        "chunk_state_kernel"]
    m = s["mfma"]
    assert abs(m["useful_tflops"] - 4096 * 32 * 139264 / 0.25e-3 / 1e12) < 1e-9
    # without a counter summary for the source, the issued rate is not reported
    assert m["issued_tflops"] is None
    assert abs(m["ceiling_tokens_per_s"] - 8e12 / (1796 * 32)) < 1e-3
