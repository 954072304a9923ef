"""bench.py's command line on the host: it measures one GPU only, so a run
asked for several GPUs (by flag or by a launcher's WORLD_SIZE) stops with
exit status 2 and says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_several_gpus_by_flag_exit_with_a_message():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_several_ranks_by_launcher_exit_with_a_message():
    r = run_bench([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_the_profiling_legs():
    r = run_bench(["--help"])
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--prefill-only", "--short-prefill-only",
                 "--decode-only", "--no-chunked", "--no-cpu-baseline"):
        assert flag in r.stdout, flag
