"""Which softmax-shift path the parity inputs exercise (CPU only).

The bf16 attention kernel fixes each query row's softmax shift at
mb = |q'| * max_k |k| (q' = qhat * softmax_scale * log2 e; both norms of the
stored bf16 rows; by Cauchy-Schwarz no score of the row exceeds it) when mb <= 48
for every row of a 32-row wave, and otherwise keeps a lazily rescaled running
maximum.  The two paths must both stay covered by the GPU parity tests: the
normal inputs take the fixed shift, the "sharp" inputs (norm weights near 2) the
running maximum.  This checks that on the oracle's prologue, rounded to bf16 as
the kernel stores it.
"""
import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import synth
from tests.test_gpu_parity import SMALL

LIMIT = 48.0          # kFixedShiftMax in attn_bf16.hip


def _bf16(x: np.ndarray) -> np.ndarray:
    return synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(x.astype(np.float32))).astype(np.float64)


def _row_bounds(w: synth.Workload, q_rows=None):
    """Per (token, head) bound mb for the query rows `q_rows` (default: all)."""
    inp = synth.generate(w)
    p = oracle.Problem.from_workload(w, inp)
    cu = w.cu_seqlens()
    all_rows = np.arange(w.N * w.H)
    k_hat = _bf16(p.prologue_rows(1, all_rows))
    knorm = np.linalg.norm(k_hat, axis=1).reshape(w.N, w.H)
    rows = all_rows if q_rows is None else q_rows
    q_hat = _bf16(p.prologue_rows(0, rows) * (p.scale / np.log(2.0)))
    qnorm = np.linalg.norm(q_hat, axis=1)
    tok, head = rows // w.H, rows % w.H
    seq = np.searchsorted(cu, tok, side="right") - 1
    kmax = np.zeros((len(cu) - 1, w.H))
    for s in range(len(cu) - 1):
        if cu[s + 1] > cu[s]:
            kmax[s] = knorm[cu[s]:cu[s + 1]].max(axis=0)
    return qnorm * kmax[seq, head]


@pytest.mark.parametrize("name", sorted(n for n in SMALL if not SMALL[n].sharp))
def test_normal_inputs_take_the_fixed_shift(name):
    mb = _row_bounds(SMALL[name])
    assert mb.max() < 0.75 * LIMIT, mb.max()


def test_sharp_inputs_take_the_running_max():
    mb = _row_bounds(SMALL["sharp_700"])
    assert np.mean(mb > LIMIT) > 0.95, np.mean(mb > LIMIT)


def test_bench_shape_takes_the_fixed_shift():
    # the joint bench shape, with the key maxima over all tokens and a sample of query rows
    w = synth.WORKLOADS["joint"]
    rows = synth.sample_rows(w, 512, seed=3)
    mb = _row_bounds(w, rows)
    assert mb.max() < 0.75 * LIMIT, mb.max()
