"""bench.py's command line on the host: more than one GPU is refused with a
message and exit status 2 before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for extra_env, args in (({}, ["--gpus", "2"]), ({"WORLD_SIZE": "2"}, [])):
        env = dict(os.environ, **extra_env)
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (r.returncode, r.stderr)
        assert "one GPU" in r.stderr
        assert r.stdout == ""
