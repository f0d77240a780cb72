"""bench.py's command-line contract, without a GPU: more than one GPU is
refused with exit status 2 and a message, every workload is selectable, and
the algorithmic byte counts the roofline uses match their definitions."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workload_choices():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for w in ("llama7b_down", "llama3_block", "phi4_ffn_stat", "qwen_ffn_b16", "llama2_ffn_chain",
              "llama2_ds_decode"):
        assert w in r.stdout


def test_algorithmic_bytes():
    sys.path.insert(0, ROOT)
    import bench
    # kept columns x rows x 2 B + x (bf16) + c (fp32) + y (fp32)
    assert bench.algorithmic_bytes(4096, 11008, 5504) == 5504 * 4096 * 2 + 11008 * 2 + 11008 * 4 + 4096 * 4
    # per pair: label rows + kept key and value rows + q + out; plus channels and lengths
    B, H, S, d, r, k = 16, 32, 8192, 128, 8, 512
    assert bench.ds_algorithmic_bytes(B, H, S, d, r, k) == \
        B * H * (S * r * 2 + k * d * 4 + d * 2 + d * 4) + H * r * 4 + B * 4
    # dense (k >= n): no label rows
    assert bench.ds_algorithmic_bytes(B, H, S, d, r, S) == B * H * (S * d * 4 + d * 6) + H * r * 4 + B * 4


def test_cpu_baseline_reports_both_thread_settings():
    sys.path.insert(0, ROOT)
    import bench
    calls = []
    res = bench._two_thread_settings(lambda i: calls.append(i), 0.05, 50, "tokens/s", "units of a test")
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in res
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s" and res["value"] > 0
    assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0
    assert res["host"]["cpus_visible"] == os.cpu_count()
    assert len(calls) <= 100


def test_parse_defaults_and_legs():
    sys.path.insert(0, ROOT)
    import bench
    a = bench.parse([])
    assert a.gpus == 1 and a.workload == "llama7b_down" and a.only == "all"
    for leg in ("sparse50", "sparse65", "fixed50", "dense", "ceiling"):
        assert bench.parse(["--only", leg]).only == leg


def test_timeline_summary_phases():
    """Phase times from synthetic timestamp arrays: microseconds since the
    launch's first workgroup started (100 MHz clock), the gate's slots as
    medians over launches, the product workgroups' percentiles, and the
    fraction of early polls that returned the pair."""
    import numpy as np
    import bench
    launches = []
    for L in range(3):
        a = np.zeros((8, 32), dtype=np.int64)
        base = 1000 + 50 * L
        a[0, 0] = base + 10             # gate starts 0.1 us after the first product workgroup
        a[0, 3] = base + 100
        a[0, 1] = base + 500            # published at 5 us
        a[0, 2] = base + 900
        for w in range(1, 6):
            a[w, 0] = base + (0 if w == 1 else 20)
            a[w, 1] = base + 120
            a[w, 2] = base + 700
            a[w, 20] = 1 if w <= 2 else 0   # 2 of 5 early polls saw the pair
            a[w, 4:20] = base + 800 + 10 * w
            a[w, 22] = base + 900 + 10 * w
        launches.append(a)
    res = bench.timeline_summary(launches)
    assert res["workgroups"] == 6
    assert res["gate_us"]["published"] == 5.0 and res["gate_us"]["keys"] == 1.0
    assert "threshold" not in res["gate_us"]
    assert res["product_us"]["compacted"]["median"] == 1.2
    assert res["product_us"]["end"]["max"] == 9.5
    assert res["product_us"]["wave_end_max"]["max"] == 8.5
    assert res["early_poll_saw_pair"] == 0.4
