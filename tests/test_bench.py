"""bench.py parts that run without a GPU: the one-GPU guard and the algorithmic
byte count behind the roofline of the expert W1/W2 kernel."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_w12_algorithmic_bytes():
    """Each touched routed expert's and each shared expert's W1 and W2 once
    (2 * D * L bf16 values), each token's latent once, each expert row's gated
    hidden once."""
    cfg = synth.get_config("C2")
    counts = np.full(cfg.n, cfg.T * cfg.k // cfg.n)
    counts[:5] = 0                                   # five experts receive no token
    b, touched = bench.experts_w12_bytes(cfg, counts)
    rows = int(counts.sum()) + cfg.n_shared * cfg.T
    assert touched == cfg.n - 5
    assert b == (touched + cfg.n_shared) * 2 * cfg.D * cfg.L * 2 + cfg.T * cfg.L * 2 + rows * cfg.D * 2
    full = np.full(cfg.n, cfg.T * cfg.k // cfg.n)
    full[: (cfg.T * cfg.k) % cfg.n] += 1             # exactly T * k dispatched rows, every expert touched
    b2, t2 = bench.experts_w12_bytes(cfg, full)
    assert t2 == cfg.n and b2 == 6_801_063_936       # the prefill figure the benchmark reports
