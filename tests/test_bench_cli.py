"""bench.py's host-side contract: it measures one GPU and says so when asked
for more (the forward shards by heads with no communication inside it), and
it refuses a multi-rank launch the same way.  Neither path touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_exits_with_a_message():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout
