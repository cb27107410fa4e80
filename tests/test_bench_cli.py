"""bench.py's command line (CPU only): more than one GPU is refused with a
message and a non-zero status before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "8"})):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
        assert p.returncode == 2, (argv, p.returncode, p.stderr[-300:])
        assert "one GPU only" in p.stderr and p.stdout == ""
