"""bench.py's command line on a machine without a GPU (no kernels run)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for mode in ("bench", "profile", "power", "selection", "workloads"):
        assert mode in r.stdout


def test_clock_sampler_reads_the_gfx_clocks_of_amd_smi_json(monkeypatch):
    """The bench line's GPU clock: the mean of the gfx_* clocks of one
    `amd-smi metric --clock --json` reading (memory and video clocks and
    non-numeric values left out), and a window summary of the readings."""
    import json
    import subprocess as sp
    import types

    sys.path.insert(0, ROOT)
    import bench

    reading = {"gpu_data": [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 1600, "unit": "MHz"}},
        "gfx_1": {"clk": {"value": 1700, "unit": "MHz"}},
        "gfx_2": {"clk": {"value": "N/A", "unit": "MHz"}},
        "gfx_3": {"clk": "N/A"},
        "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
        "vclk_0": {"clk": {"value": 59, "unit": "MHz"}}}}]}
    monkeypatch.setattr(sp, "run", lambda *a, **k: types.SimpleNamespace(stdout=json.dumps(reading), returncode=0))
    cs = bench.ClockSampler()
    assert cs._read() == 1650.0
    cs.samples = [(1.0, 1.9, 1500.0), (2.0, 2.9, 1650.0), (3.0, 3.4, 1600.0), (3.4, 4.2, 1700.0),
                  (9.0, 9.5, 100.0)]
    # readings count only when their call began and ended inside the window
    assert cs.summary(0.5, 3.5) == {"samples": 3, "median": 1600.0, "min": 1500.0, "max": 1650.0}
    assert cs.summary(4.0, 5.0) is None
