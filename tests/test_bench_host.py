"""Host-side logic of bench.py (no GPU): the SMI reading it keeps, the recorded
HBM-traffic lookup and its staleness check, and the one-GPU refusal."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_compact_clocks_keeps_clock_and_power():
    b = load_bench()
    clk = {f"gfx_{i}": {"clk": {"value": 1800 + i, "unit": "MHz"}} for i in range(8)}
    clk["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    clk["vclk_0"] = {"clk": {"value": 59, "unit": "MHz"}}
    reading = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1300, "unit": "W"}}, "clock": clk}]}
    got = b.compact_clocks(reading)
    assert got == {"gfx_clk_mhz_per_xcd": [1800 + i for i in range(8)], "mem_clk_mhz": 2000, "socket_power_w": 1300}
    assert "reading" in b.compact_clocks({"unexpected": 1})


def test_recorded_traffic_follows_the_kernel_sources(tmp_path):
    b = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    rel = os.path.relpath(src, ROOT)
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    prof.write_text(f"# t\n\nworkload: w1\nkernel: k1\nkernel_sources: {rel}\nkernel_sources_sha256: {sha}\n"
                    f"traffic_bytes_per_launch: 1.5e+09\n")
    b.TRAFFIC_FILE = str(prof)
    assert b.recorded_traffic("w1", "k1") == 1.5e9
    assert b.recorded_traffic("w2", "k1") is None and b.recorded_traffic("w1", "k2") is None
    src.write_text("// kernel source, changed since the counters were taken\n")
    assert b.recorded_traffic("w1", "k1") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
