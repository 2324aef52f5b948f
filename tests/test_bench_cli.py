"""bench.py's command line on the host: more than one GPU is refused before
any device work, with a one-line JSON error and exit status 2."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for extra_env, args in (({}, ["--gpus", "2"]), ({"WORLD_SIZE": "4"}, [])):
        env = dict(os.environ, **extra_env)
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=120)
        assert p.returncode == 2, p.stderr
        line = p.stdout.strip().splitlines()[-1]
        assert "one GPU" in json.loads(line)["error"]
