"""Host-side checks of bench.py: the refusal of several GPUs and the rule that
profiled HBM traffic is reported only for the kernel source it was taken on."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profiled_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    (tmp_path / "profiles").mkdir()
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "k.md").write_text(
        "# k\n\n| counter | x |\n|---|---|\n\ntraffic_bytes_per_launch: 12345\n"
        f"source: kernel.hip\nsource_sha256: {digest}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("k.md", "kernel.hip") == 12345.0
    src.write_text("// kernel v2\n")                 # the kernel changed since profiling
    assert bench.profiled_traffic("k.md", "kernel.hip") is None
    assert bench.profiled_traffic("missing.md", "kernel.hip") is None


def test_committed_profiles_parse():
    for name, src in (("fwd_bf16_layer_1p3b_bf16.md", "gated_delta_rule_22_amd/csrc/fwd_bf16.hip"),
                      ("decode_256x16.md", "gated_delta_rule_22_amd/csrc/decode.hip")):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "traffic_bytes_per_launch:" in text and "source_sha256:" in text
        assert "rocprofv3" in text
        t = bench.profiled_traffic(name, src)
        assert t is None or t > 0
