"""bench.py's contract on the host: more than one GPU is refused with a message
before any GPU work, and the counter-record key ignores comments but not code."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    import bench

    csrc = tmp_path / "block_quantized_gemv_q8_amd" / "csrc"
    csrc.mkdir(parents=True)
    base = "int f(int a) { return a + 1; } // one\n/* two */\n"
    for rel in bench.KERNEL_SOURCES:
        (tmp_path / rel).write_text(base)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    for rel in bench.KERNEL_SOURCES:
        (tmp_path / rel).write_text("int f(int a)  {\n  return a + 1;\n} // changed\n")
    assert bench.kernel_source_hash() == h0
    (tmp_path / bench.KERNEL_SOURCES[0]).write_text("int f(int a) { return a + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_committed_traffic_records_match_the_kernel_sources():
    """The HBM-traffic records under profiles/ were taken on the kernel
    sources as they are: bench.py reports their bytes as the roofline's
    traffic only then (else null), so a kernel change without new counter
    passes shows here."""
    import json

    import bench

    h = bench.kernel_source_hash()
    for path in (bench.PMC_RECORD, bench.PMC_RECORD_GATE_UP):
        with open(path) as f:
            rec = json.load(f)
        assert rec["kernel_source_hash"] == h, os.path.basename(path)
        assert rec["hbm_bytes_per_launch"] > 0
    assert bench.pmc_traffic() is not None
