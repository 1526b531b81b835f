"""Host-side checks of the benchmark's command line and of the product/checker boundary (no GPU needed)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=120):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args), cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_without_a_gpu_the_bench_stops_before_timing():
    r = run_bench("--no-traffic", "--no-cpu")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr


def imported_modules(path):
    tree = ast.parse(open(path).read())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            mods.add(node.module.split(".")[0])
    return mods


def test_the_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "decode_attention_bf16_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            assert "oracle" not in imported_modules(os.path.join(pkg, name)), name
    for name in os.listdir(os.path.join(pkg, "csrc")):
        src = open(os.path.join(pkg, "csrc", name)).read()
        assert "oracle" not in src, name


def test_the_oracle_shares_no_code_with_the_kernels():
    odir = os.path.join(ROOT, "oracle")
    for name in os.listdir(odir):
        if name.endswith((".c", ".h", ".py")):
            src = open(os.path.join(odir, name)).read()
            assert "decode_attention_bf16_amd" not in src and "csrc" not in src, name
