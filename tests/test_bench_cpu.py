"""Host-side checks of bench.py: the one-GPU contract, and the counter summary it reads."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    import bench

    h0 = bench.kernel_source_hash()
    copies = {}
    for rel in bench.KERNEL_SOURCES:
        src = open(os.path.join(ROOT, rel)).read()
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        copies[rel] = (dst, src)
        dst.write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash() == h0
    dst, src = copies[bench.KERNEL_SOURCES[0]]
    dst.write_text(src + "\n// a comment\n/* and\n another */\n")
    assert bench.kernel_source_hash() == h0
    dst.write_text(src.replace("c = a.c;", "c = a.c * 1.0f;", 1))
    assert bench.kernel_source_hash() != h0


def test_counter_summary_is_parsed():
    import bench

    traffic, note = bench.traffic_from_profile()
    if note == "kernel changed since counters were taken":
        pytest.skip("forward kernel edited since the counters were recorded")
    assert note == "ok"
    # algorithmic bytes of the workload are 2.156e9; traffic cannot be below them
    assert 2.0e9 < traffic < 2.0e10


def test_amd_smi_metric_text_is_parsed():
    import bench

    clocks = (1983, 1883, 1975, 1929, 2005, 1913, 1962, 1909)
    txt = "GPU: 0\n    POWER:\n        SOCKET_POWER: 1344 W\n        GFX_VOLTAGE: N/A\n    CLOCK:\n"
    for i, c in enumerate(clocks):
        txt += f"        GFX_{i}:\n            CLK: {c} MHz\n            MIN_CLK: 500 MHz\n            MAX_CLK: 2400 MHz\n"
    txt += "        MEM_0:\n            CLK: 2000 MHz\n"
    watts, mhz = bench.parse_smi_metric(txt)
    assert watts == 1344.0
    assert mhz == pytest.approx(sum(clocks) / 8)   # the memory clock is not a GFX clock
    assert bench.parse_smi_metric("amd-smi: command not found") is None
