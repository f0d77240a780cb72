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
