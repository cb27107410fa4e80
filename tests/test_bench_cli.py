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


def test_single_thread_oracle_timings():
    """cpu_baseline.single_thread: one oracle call per configuration, each
    with its seconds and algorithmic GB/s (small inputs here)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import synth
    g = synth.rng(5)
    tiny = synth.quant_weights(64, 64, g) + (g.standard_normal((8, 64)).astype(np.float32),)
    c, sm = synth.quant_weights(96, 128, g)
    xb = (g.standard_normal((2, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    table, num_pages = synth.page_table(1, 5, g)
    kp, vp = synth.kv_pages(num_pages, 2, 64, g)
    attn = (synth.f16_normal((1, 8, 64), g), kp, vp, table, 70, 0.125)
    zt = (g.standard_normal((6, 100)) * 3).astype(np.float32)
    zd = (g.standard_normal((4, 100)) * 3).astype(np.float32)
    ragged = (zt, zd, np.zeros(4, np.int32), np.array([0, 3, 6], np.int32), np.arange(2),
              np.array([10, 20]), 0.8)
    r = bench._single_thread_calls(tiny, (c, sm, xb[:1]), attn, (c, sm, xb), ragged)
    assert len(r) == 5
    for name, v in r.items():
        assert v["s"] > 0 and v["GBps"] > 0, name
