"""Host-side contract checks (no GPU): the bench refuses multi-GPU runs, and
the binding refuses to import without the built HIP library (there is no
CPU fallback)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_binding_fails_loudly_without_library(tmp_path):
    pkg = tmp_path / "latentmoe_expert_layer_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "latentmoe_expert_layer_amd", "__init__.py"), pkg / "__init__.py")
    code = "import latentmoe_expert_layer_amd"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "liblatent_moe.so" in r.stderr
