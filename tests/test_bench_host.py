"""Host-side checks of bench.py's reporting (no GPU)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counter summary while the kernel sources hash to the
    value recorded there, and is null otherwise."""
    with open(bench.TRAFFIC_PROFILE) as f:
        text = f.read()
    prof = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    good = text.replace(text.split("sources_sha256: ")[1].split("\n")[0], bench.kernel_sources_sha256())
    prof.write_text(good)
    got = bench.measured_traffic("bwd_records_launch_traffic_bytes")
    assert isinstance(got, int) and got > 3_221_225_472  # at least the algorithmic bytes
    assert isinstance(bench.measured_traffic("train_fwd_launch_traffic_bytes"), int)
    prof.write_text(good.replace(bench.kernel_sources_sha256(), "0" * 64))
    assert bench.measured_traffic("bwd_records_launch_traffic_bytes") is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("bwd_records_launch_traffic_bytes") is None


def test_byte_and_flop_models_match_the_stated_per_token_figures():
    # per token-head at C = 64, d = 128: forward 2304 B (+1024 with chunk states), backward 6144 B
    assert bench.fwd_bytes(64, 128, save_states=False) == 2304
    assert bench.fwd_bytes(64, 128) == 3328
    assert bench.bwd_bytes(64, 128) == 6144
    assert round(bench.fwd_flops(64, 128)) == 181589
    assert round(bench.bwd_flops(64, 128)) == 476501
