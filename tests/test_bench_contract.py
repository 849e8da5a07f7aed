"""bench.py's command-line contract on the host (no GPU work is started)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_json_fields_are_documented():
    """The bench line's extra objects are emitted, and the committed traffic
    summary that fills roofline.traffic is well-formed."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    for key in ("roofline", "cpu_baseline", "traffic", "decode_graph_per_layer",
                "hbm_copy_context", "generation"):
        assert f'"{key}"' in src, key
    traffic = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert "decode_partials" in traffic and "source_hash" in traffic["decode_partials"]
