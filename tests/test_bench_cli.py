"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message, and measured HBM traffic is only reported for the
kernel sources it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""  # no JSON line


def test_traffic_tied_to_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic("q8b", "no.such.kernel") is None
    # a copy of the tree whose decode-step source differs reports no traffic
    t = bench.TRAFFIC[("q8b", "decode.step")]
    for src in t["sources"]:
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        data = open(os.path.join(ROOT, src), "rb").read()
        dst.write_bytes(data + (b"\n// changed\n" if src.endswith("decode_step.hip") else b""))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("q8b", "decode.step") is None
