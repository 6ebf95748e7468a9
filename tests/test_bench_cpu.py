"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    p = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert p.returncode != 0
    assert "one GPU" in p.stderr
    assert p.stdout == ""  # no JSON line for a configuration it does not measure


def test_launched_as_several_ranks_exits_with_a_message():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    p = _run("--steps", "1", "--warmup", "0", env=env)
    assert p.returncode != 0
    assert "one GPU" in p.stderr


def test_help_lists_the_contract_flags():
    p = _run("--help")
    assert p.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in p.stdout
