"""Host logic of bench.py that runs without a GPU: the traffic digest, traffic keys, the one-GPU rule."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_lines_but_keeps_code():
    a = "int x = 1;  // one\n\n// a whole comment line\nint y = 2;\n"
    b = "int x = 1;\n    \nint y = 2;   // two\n"
    assert bench._code_only(a) == bench._code_only(b) == "int x = 1;\nint y = 2;"
    assert bench._code_only("int x = 2;") != bench._code_only("int x = 1;")


def test_source_digest_is_stable_and_hex():
    d = bench.source_digest()
    assert d == bench.source_digest() and len(d) == 64 and int(d, 16) >= 0


def test_traffic_keys_name_the_variant():
    assert bench.traffic_key("grouped") == "grouped"
    assert bench.traffic_key("grouped", fast_math=True, planes="both") == "grouped_both_fast"
    assert bench.traffic_key("weight", tile16=True, dtype="fp16") == "weight_tile16_fp16"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env=dict(os.environ, CUDA_VISIBLE_DEVICES=""))
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
