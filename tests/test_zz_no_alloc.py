"""h3attn_fwd_static (the workspace in a static device array, for callers
that cannot allocate) against h3attn_fwd with a caller-given workspace.

Two calls in a row on the same device: the largest shape the static array
takes at H = 24, then a smaller ragged batch, whose result must not depend on
what the first call left in the array.  Both run the same kernels on the same
inputs, so the outputs must be equal bit for bit; the second is also checked
against the fp64 oracle on sampled rows at the bf16 gate.
"""
import numpy as np
import pytest

from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
Seq = synth.Seq

CASES = [
    # 7,168 tokens x 24 heads: the largest bf16 workspace the static array holds
    synth.Workload("static_max_7168", H=24, d=128, seqs=(Seq(7, 32, 32),), split=(32, 48, 48),
                   k_offset_std=0.5, seed=71),
    # then a smaller ragged batch with an audio-only sequence
    synth.Workload("static_ragged_small", H=24, d=128, seqs=(Seq(3, 10, 11, 7), Seq(0, 1, 1, 40), Seq(1, 4, 5, 70)),
                   split=(32, 48, 48), seed=72),
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def test_static_workspace_matches_caller_workspace(torch_dev):
    torch = torch_dev
    assert h.h3attn_workspace_size(h.make_params(24, 128, 1, 3072, 3072, 3072, 3072), [0, CASES[0].N]) \
        <= h.H3ATTN_STATIC_WORKSPACE_BYTES
    for w in CASES:
        inp = synth.generate(w)
        t = G.to_device(inp, w)
        out_s = torch.full((w.N, w.H, w.d), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        G.announce("no-alloc entry h3attn_fwd_static workload=%s N=%d H=%d" % (w.name, w.N, w.H))
        h.h3attn_fwd_static(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], out_s, eps=w.eps)
        torch.cuda.synchronize()
        got = G.bits(out_s)
        want = G.bits(G.run(w, t, label=w.name + "_workspace"))
        assert np.array_equal(got, want), "%s: static-workspace output differs from h3attn_fwd" % w.name
    rows = synth.sample_rows(w, 512)
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), G.oracle_rows(w, inp, rows)), G.BF16_GATE, w.name)
