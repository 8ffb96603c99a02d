"""Host-side pieces of bench.py: the parity figures it reports from the oracle
leg, the input digest of its provenance block, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_parity_metrics_closed_form():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.0 + 0.5], [0.1, 0.0]])
    m = bench.parity_metrics(got, ref, "exact fp64 attention")
    assert m["rows"] == 2 and m["against"] == "exact fp64 attention"
    assert m["max_abs"] == 0.5
    assert np.isclose(m["mean_abs"], 0.6 / 4)
    assert np.isclose(m["rel_l2"], np.sqrt(0.25 + 0.01) / 5.0)
    assert np.isclose(m["cosine"], 27.0 / (np.sqrt(9 + 20.25 + 0.01) * 5.0))
    same = bench.parity_metrics(ref[:1], ref[:1], "x")
    assert same["max_abs"] == 0 and same["rel_l2"] == 0 and np.isclose(same["cosine"], 1.0)


def test_input_digest_tracks_every_byte():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 1 << 16, size=(64, 3, 8), dtype=np.uint16)
    b = rng.standard_normal((2, 3, 8)).astype(np.float32)
    d1 = bench._input_digest([a, b])
    assert d1 == bench._input_digest([a.copy(), b.copy()])
    a2 = a.copy()
    a2[17, 1, 5] ^= 1
    assert bench._input_digest([a2, b]) != d1
    assert bench._input_digest([b, a]) != d1          # order matters


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
