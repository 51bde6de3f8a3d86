"""bench.py's command line on a machine without a GPU: --gpus above 1 is
refused with exit status 2 before any GPU work, and the module imports."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_module_names_exist():
    # every binding function bench.py calls exists in the package
    import exact_attention_30_amd as attn
    src = open(os.path.join(ROOT, "bench.py")).read()
    for name in ("prefill", "decode", "decode_waves"):
        assert f"attn.{name}(" in src
        assert hasattr(attn, name)
