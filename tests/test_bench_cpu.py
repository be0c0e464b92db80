"""The benchmark's contract on the host: it runs on exactly one GPU, so a
request for more (the --gpus flag, or a launcher's WORLD_SIZE) ends at once
with exit status 2 and one JSON line that says so, before any GPU work."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, timeout=120, env=e, cwd=ROOT)
    assert r.returncode == 2, r.stdout + r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
