"""bench.py's host-side contract (no GPU): more than one GPU is refused with a
message, and the algorithmic byte count follows the row geometry."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_250k_workload():
    sys.path.insert(0, ROOT)
    import bench
    from long_context_sparse_sketch_amd import configs as C
    sketch, gathered, small = bench.algorithmic_bytes(C.C3)
    assert sketch == 8 * 4 * 245904 * 64                      # 503.6 MB
    assert gathered == 8 * 4 * (2048 + 4096) * 2 * 256        # 100.7 MB
    s5, g5, _ = bench.algorithmic_bytes(C.C5)
    assert s5 == 4 * 8 * (65539 - 4096) * 64                  # one pass for the 3 rows
    assert g5 == sum(4 * 8 * 6144 * 2 * 130 for _ in range(3))


def test_counted_traffic_follows_the_score_sources(tmp_path, monkeypatch):
    """A counter summary is used only for its workload and score-pass mode and
    only while the score kernel's sources hash to the value recorded with it."""
    import hashlib
    sys.path.insert(0, ROOT)
    import bench
    h = hashlib.sha256()
    for f in bench.SCORE_SOURCES:
        h.update(open(os.path.join(ROOT, "long_context_sparse_sketch_amd", "csrc", f), "rb").read())
    body = ("workload: multi_agent_250k\nkernel: score_kernel\n"
            f"score_sources_sha256: {h.hexdigest()}\ntraffic_bytes_per_launch: 537628512\n")
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "score_kernel_{workload}_hbm_counters.txt"))
    (tmp_path / "score_kernel_multi_agent_250k_hbm_counters.txt").write_text(body)
    assert bench.counted_traffic("multi_agent_250k", "stores") == 537628512
    assert bench.counted_traffic("multi_agent_250k", "candidates") is None
    assert bench.counted_traffic("tiny", "stores") is None
    (tmp_path / "score_kernel_multi_agent_250k_hbm_counters.txt").write_text(
        body + "mode: candidates\n")
    assert bench.counted_traffic("multi_agent_250k", "candidates") == 537628512
    assert bench.counted_traffic("multi_agent_250k", "stores") is None
    (tmp_path / "score_kernel_multi_agent_250k_hbm_counters.txt").write_text(
        body.replace("score_sources_sha256: ", "score_sources_sha256: 00"))
    assert bench.counted_traffic("multi_agent_250k", "stores") is None


def test_committed_counter_summary_parses():
    sys.path.insert(0, ROOT)
    import bench
    fields = dict(ln.split(":", 1) for ln in open(bench.COUNTERS.format(workload="multi_agent_250k"))
                  if ln.startswith(("workload:", "traffic_bytes_per_launch:", "score_sources_sha256:")))
    assert fields["workload"].strip() == "multi_agent_250k"
    assert 5.0e8 < int(fields["traffic_bytes_per_launch"]) < 6.0e8   # ~1.07 x the 503.6 MB of sketch
    assert len(fields["score_sources_sha256"].strip()) == 64
