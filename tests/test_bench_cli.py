"""bench.py's command line on the CPU: more than one GPU is refused with a message before any
GPU work, and --help lists the modes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_help_lists_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--rotation-ablation", "--mlp", "--a16", "--workload"):
        assert flag in r.stdout


def test_bench_source_digest_covers_every_kernel_source():
    """--source-digest names a digest per kernel, and every file it hashes exists (a summary in
    profiles/ is only used while its digest matches these sources)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--source-digest"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    import json
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert set(d) == {"lut_gemm", "rpbh_quantize"}
    assert all(len(v) == 64 for v in d.values())
