"""Host side of bench.py: the argument contract checked before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and says why, before importing torch."""
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    """A launch under torch.distributed with several ranks is refused the same way."""
    r = run_bench(env_extra={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_the_contract_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--T", "--workload", "--small-set", "--window-widths"):
        assert flag in r.stdout
