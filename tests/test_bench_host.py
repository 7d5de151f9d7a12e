"""Host-side contract of bench.py that needs no GPU: the one-GPU guard, and the counter-measured
traffic record, which is reported only while the GEMM sources are the ones it was taken on."""

import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _record(text):
    return json.loads(text.split("```json", 1)[1].split("```", 1)[0])


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "sparse_layer_rho_amd", "csrc")
    dst = tmp_path / "sparse_layer_rho_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("gemm.hip", "kernels.h", "common.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    rec_path = tmp_path / "traffic.md"
    text = open(bench.TRAFFIC_RECORD).read()
    rec = _record(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec_path))
    # a record whose hash is that of these sources is reported
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "kernels.h", "common.h"):
        h.update((dst / f).read_bytes())
    rec["source_sha256"] = h.hexdigest()
    rec_path.write_text("x\n```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.measured_traffic() == rec["traffic_bytes"]
    # any change to the GEMM sources voids it
    (dst / "gemm.hip").write_text((dst / "gemm.hip").read_text() + "\n// edited\n")
    assert bench.measured_traffic() is None
    # as does a missing or unreadable record
    rec_path.write_text("no record here")
    assert bench.measured_traffic() is None


def test_default_line_is_the_layer_stack(monkeypatch):
    """The metric is branch-tokens/s per layer stack: with no arguments bench.py measures the
    28-layer 1.5B-shape stack (its single layer rides along as a sub-object)."""
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    from synth import WORKLOADS
    wl = WORKLOADS[args.workload]
    assert args.workload == "stack-1.5b" and wl.layers == 28 and wl.steps == 8
    assert wl.shape.prefix_len == 2048 and wl.shape.hidden == 1536 and not args.no_layer


def test_committed_traffic_records_match_the_current_gemm_sources():
    """Both committed gate/up records (single layer, stack) were taken on these GEMM sources, so
    the line reports their traffic; they sit within 10 % of the algorithmic bytes."""
    for path in (bench.TRAFFIC_RECORD, bench.stack_traffic_record("stack-1.5b")):
        rec = _record(open(path).read())
        assert bench.measured_traffic(path) == rec["traffic_bytes"]
        assert 5.7e7 < rec["traffic_bytes"] < 6.4e7
