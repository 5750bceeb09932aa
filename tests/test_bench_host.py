"""Host-side logic of bench.py, on the CPU: the work and byte counts the
reported rates are computed from, the gate that reports counter-measured
figures only for the kernel sources they were taken with, and the refusal
to run on more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_effective_ops_canonical():
    # 512 ops per (query, key) pair: 128 INT8 and 128 FP8 multiply-adds
    assert bench.effective_ops(1, 37810, 56) == 4.0 * 37810 ** 2 * 56 * 128
    assert abs(bench.effective_ops(1, 37810, 56) - 4.0989e13) / 4.0989e13 < 1e-4


def test_prepass_bytes_canonical():
    # Q once and K, V twice in BF16, then INT8 Q (padded to 128 rows), INT8 K
    # and FP8 V (padded to 64 rows)
    B, N, H = 1, 37810, 56
    reads = 5 * 2 * B * N * H * 128
    writes = B * H * (37888 + 2 * 591 * 64) * 128
    assert bench.prepass_bytes(B, N, H) == reads + writes
    assert abs(bench.prepass_bytes(B, N, H) - 3.52e9) / 3.52e9 < 0.01


def _summary(tmp_path, sha, workload="canonical", extra="hbm_bytes_per_launch: 6.2e9\n"):
    p = tmp_path / "s.md"
    p.write_text("# summary\n\nsome text: with a colon\nworkload: %s\nkernel_source_sha256: `%s`\n%s"
                 % (workload, sha, extra))
    return str(p)


def test_recorded_fields_follow_the_kernel_sources(tmp_path):
    sha = bench.kernel_source_hash()
    good = _summary(tmp_path, sha)
    assert bench.recorded_fields(good, "canonical", ("hbm_bytes_per_launch",)) == {"hbm_bytes_per_launch": 6.2e9}
    # another workload, other sources, a missing field or file: nothing is reported
    assert bench.recorded_fields(good, "mid", ("hbm_bytes_per_launch",)) is None
    assert bench.recorded_fields(_summary(tmp_path, "0" * 64), "canonical", ("hbm_bytes_per_launch",)) is None
    assert bench.recorded_fields(good, "canonical", ("hbm_bytes_per_launch", "missing")) is None
    assert bench.recorded_fields(str(tmp_path / "none.md"), "canonical", ("hbm_bytes_per_launch",)) is None


def test_kernel_source_hash_covers_the_mainloop_sources(tmp_path, monkeypatch):
    h0 = bench.kernel_source_hash()
    csrc = tmp_path / "quantized_exact_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_exact_attention_amd", "csrc", name), "rb") as f:
            (csrc / name).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash() == h0
    (csrc / "attn_mainloop.hip").write_bytes((csrc / "attn_mainloop.hip").read_bytes() + b"\n")
    assert bench.kernel_source_hash() != h0


def test_committed_summaries_parse():
    """The committed counter summaries carry every field the bench line
    reports (whether they match the current sources is the bench's run-time
    check)."""
    for path, names in ((bench.TRAFFIC_FILE, ("hbm_bytes_per_launch",)),
                        (bench.COUNTERS_FILE, ("mfma_busy_frac", "mfma_ops_per_active_cycle_frac",
                                               "valu_active_frac", "mainloop_clock_ghz"))):
        text = open(path).read()
        for n in ("workload", "kernel_source_sha256") + names:
            assert "\n%s:" % n in text, (path, n)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_probe_matrix_ops_per_iteration():
    # one wave tile's matrix work: 32 queries x 64 keys x 128 channels for QK
    # and 32 queries x 128 channels x 64 keys for PV, 2 ops per multiply-add
    assert bench.PROBE_MATRIX_OPS_PER_ITER == 2 * (32 * 64 * 128) + 2 * (32 * 128 * 64)
    # a 64-query x 64-key block of the workload count holds two wave tiles
    assert bench.PROBE_MATRIX_OPS_PER_ITER == bench.effective_ops(1, 64, 1) / 2
