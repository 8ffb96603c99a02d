"""The checked build (libh3attn_checked.so: the same sources with the
attention kernels' invariant checks and timing jitter compiled in) against the
product library.

For every case of tests/checked_run.py (the eight-wave kernel dense on a ragged
batch, a long sequence and sharp inputs, and block-sparse on caller lists; the
four-wave kernel dense and block-sparse; the INT8/FP8 and MXFP4 kernels on the
ragged batch and the long sequence), run in a child process on the checked
build with jitter seeds 0, 1, 2 and 3:
- every output is bit-identical to the product library's: the kernels are
  deterministic, and the jitter (per-wave delays before every fill and phase)
  moves the relative timing of waves and fills, so a race between an LDS fill
  and a fragment read would change bits;
- no invariant flag is set (work-item decode, query rows inside the padded
  layout, every fill inside the sequence's tiles, list entries in range);
- a caller list with an out-of-range entry (clamped by the kernels, no access
  leaves the buffers) sets exactly flag word 3, so the flags are live;
- the jittered calls take measurably longer, so the delays are live.
"""
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from audio_diffusion_transformer_amd import build as B
from tests import checked_run as R
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SEEDS = (0, 1, 2, 3)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def test_checked_build_matches_product_under_jitter(torch_dev):
    assert os.path.exists(B.LIB_CHECKED), "libh3attn_checked.so is not built"
    ref = R.run_all(torch_dev)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "checked.npz")
        env = dict(os.environ, H3ATTN_LIB=B.LIB_CHECKED)
        G.announce("checked build in a child process, jitter seeds %s" % (SEEDS,))
        r = subprocess.run([sys.executable, "-u", "-m", "tests.checked_run", path] + [str(s) for s in SEEDS],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        got = dict(np.load(path))
    for seed in SEEDS:
        flags = got["flags@%d" % seed]
        assert not flags.any(), "seed %d: invariant flags %s" % (seed, flags)
        for name, bits in ref.items():
            other = got["%s@%d" % (name, seed)]
            diff = int((other != bits).sum())
            assert diff == 0, "%s, jitter seed %d: %d of %d output elements differ" % (name, seed, diff, bits.size)
    bad = got["flags@bad_list"]
    assert bad[3] != 0 and not bad[:3].any(), bad
    # the delays are really there (about 0-3 x 128 cycles per wave per fill and phase)
    t0, t1 = float(got["ms@0"][0]), float(got["ms@1"][0])
    G.announce("long_d128 per call: %.4f ms without jitter, %.4f ms with" % (t0, t1))
    assert t1 > 1.05 * t0, (t0, t1)
