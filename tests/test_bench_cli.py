"""The benchmark's command-line contract, checked without a GPU: more than one GPU is
refused with a message before anything touches a device, and the options parse."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--density", "--dense", "--mass", "--uneven", "--balanced", "--fused-select", "--no-cpu-baseline",
                "--steps", "--warmup", "--sustain", "--no-report", "--mfma-probe"):
        assert opt in r.stdout, opt


def test_sequence_and_scale_names_resolve():
    sys.path.insert(0, ROOT)
    import bench
    from block_sparse_attention_aggregated_amd import inputs as I
    assert [c.name for c in bench.workload_configs("clip1")] == [c.name for c in I.CLIP1]
    assert bench.workload_configs("720p")[0] is I.S720P
    assert len(bench.workload_configs("sweep")) == 4


def test_uneven_lists_recipe():
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    rp, ci, counts = bench.uneven_lists(50, 40, 3, 10, seed=1)
    assert rp[0] == 0 and rp[-1] == len(ci) and np.all(np.diff(rp) == counts + 3)
    for r in range(50):
        row = ci[rp[r]:rp[r + 1]]
        assert list(row[:3]) == [0, 1, 2] and np.all(np.diff(row) > 0) and row.max() < 40
    assert 1 <= counts.min() and counts.max() <= 19
    _, _, even = bench.uneven_lists(50, 40, 3, 10, seed=1, even=True)
    assert np.all(even == 10)
    for B, H, n_q, block in ((1, 2, 11, 128), (2, 3, 13, 64), (1, 5, 563, 128), (1, 1, 1, 256), (3, 1, 9, 128)):
        order = bench.dispatch_order(B, H, n_q, block)
        assert sorted(order.tolist()) == list(range(B * H * n_q))
    # b = 128: XCDs 0-3 split the even head into 4 segments, XCDs 4-7 the odd one
    order = bench.dispatch_order(1, 2, 11, 128)
    assert order[:8].tolist() == [0, 3, 6, 9, 11 + 0, 11 + 3, 11 + 6, 11 + 9]
    # b = 64, or an odd head count: 8 segments, one head at a time
    order = bench.dispatch_order(1, 2, 16, 64)
    assert order[:8].tolist() == [0, 2, 4, 6, 8, 10, 12, 14]
    order = bench.dispatch_order(1, 3, 16, 128)
    assert order[:8].tolist() == [0, 2, 4, 6, 8, 10, 12, 14]


def test_cache_flush_and_cpu_model_helpers():
    sys.path.insert(0, ROOT)
    import bench
    flush = bench.infinity_cache_flush("cpu", mb=4)
    flush()
    assert isinstance(bench.cpu_model(), str)


def test_parse_smi_reads_power_and_xcd_clocks():
    sys.path.insert(0, ROOT)
    import bench
    clk = lambda v: {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                     "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "N/A"}
    gpu = {"gpu": 0, "power": {"socket_power": {"value": 1390, "unit": "W"}, "gfx_voltage": "N/A"},
           "clock": {**{f"gfx_{i}": clk(1500 + 10 * i) for i in range(8)}, "mem_0": clk(2000),
                     "vclk_0": clk(59)}}
    other = {"gpu": 1, "power": {"socket_power": {"value": 200, "unit": "W"}}, "clock": {"gfx_0": clk(100)}}
    r = bench.parse_smi({"gpu_data": [gpu, other]})
    assert r["power_w"] == 1390
    assert r["gfx_mhz"] == [1500 + 10 * i for i in range(8)]
    assert r["mem_mhz"] == 2000
    assert bench.parse_smi({"gpu_data": [{"gpu": 0, "power": "N/A"}]}) is None
