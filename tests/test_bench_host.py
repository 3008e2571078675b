"""Host-side checks of the benchmark's contract (no GPU): the multi-GPU
refusal, the algorithmic byte and flop counts behind the roofline figures
(recomputed here from the data layout), and the counter records' gating on
the kernel source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

METRIC_SHAPE = dict(B=128, gamma=16, V=151936, r=256, logit_dtype="bf16", w_dtype="bf16")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_algorithmic_bytes_of_the_metric_workload():
    """Only the method's inputs and outputs count: U, W2 once, the gathered W1
    rows, the anchors, and the tokens, log Z and q(x) written; the kernel's own
    softmax summaries (scratch it writes and reads back) do not."""
    B, g, V, r = 128, 16, 151936, 256
    want = B * g * V * 2 + r * V * 2 + B * g * r * 2 + B * 4 + B * g * 12
    kb = bench.kernel_bytes(METRIC_SHAPE)
    assert kb["draft_persist"] == want == 701194752
    assert kb["verify_rows_p"] == B * (g + 1) * V * 2 == 661225472
    # the streamed final draw: two rows per residual draw, one per bonus draw
    kb = bench.kernel_bytes(METRIC_SHAPE, n_resid=100)
    assert kb["verify_resid"] == 100 * V * 4 + 28 * V * 2 + r * V * 2 + 100 * r * 2
    # the q-free cycle: draft + target rows + final draw
    assert bench.cycle_bytes(METRIC_SHAPE, "qfree", 100) == \
        701194752 + 661225472 + kb["verify_resid"]


def test_algorithmic_bytes_of_ragged_lengths():
    shape = dict(METRIC_SHAPE, B=4, lens=[1, 16, 3, 0])
    kb = bench.kernel_bytes(shape)
    assert kb["verify_rows_p"] == (20 + 4) * 151936 * 2


def test_bias_flops_of_the_metric_workload():
    assert bench.bias_flops(METRIC_SHAPE)["draft_persist"] == 2.0 * 128 * 256 * 151936 * 16


def test_counter_records_are_gated_on_the_source(tmp_path, monkeypatch):
    """A traffic record counts only while its source hash matches the kernel's
    sources; a record with another hash reads as unmeasured."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.source_sha(bench.KERNEL_SOURCES["draft_persist"])
    for name, h in (("ok", sha), ("stale", "0" * 16)):
        (prof / f"draft_persist__{name}.traffic.json").write_text(
            json.dumps({"source_sha": h, "traffic_bytes_per_launch": 123.0}))
        (prof / f"draft_persist__{name}.mfma.json").write_text(
            json.dumps({"source_sha": h, "mfma_busy_frac": 0.25}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # source_sha reads the sources relative to ROOT: point it back at the repository
    monkeypatch.setattr(bench, "source_sha", lambda paths: sha)
    assert bench.measured_traffic("draft_persist", "ok") == 123.0
    assert bench.measured_traffic("draft_persist", "stale") is None
    assert bench.measured_traffic("draft_persist", "absent") is None
    assert bench.measured_mfma("draft_persist", "ok") == 0.25
    assert bench.measured_mfma("draft_persist", "stale") is None


def test_committed_records_are_plausible():
    """Whatever the committed draft records say, when they match the current
    source the counted traffic is within a plausible factor of the
    algorithmic bytes (re-reads show up as a factor well above 1)."""
    t = bench.measured_traffic("draft_persist", "markov-152k-b128")
    if t is None:
        pytest.skip("no record for the current draft source")
    ratio = t / bench.kernel_bytes(METRIC_SHAPE)["draft_persist"]
    assert 0.8 < ratio < 2.0, ratio
