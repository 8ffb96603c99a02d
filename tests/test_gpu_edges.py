"""GPU parity at the edges of the boundary's limits, against the fp64 oracle.

- the largest batch the ABI takes (64 sequences), with ragged lengths from
  empty through single tokens, audio-only sequences and lengths on 64- and
  256-token boundaries, through both the bf16 and the quantised path;
- single-token sequences only (every tile has one valid key);
- a non-default softmax scale and RMSNorm epsilon;
- the most heads the ABI takes (4,096), on both paths.

All rows are compared (the cases are small).
"""
import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import h3attn as h, synth
from audio_diffusion_transformer_amd.synth import Seq
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _max_batch() -> synth.Workload:
    rng = np.random.default_rng(2024)
    seqs = []
    special = [0, 1, 63, 64, 65, 255, 256, 257]
    for i in range(h.H3ATTN_MAX_SEQS):
        if i < len(special):
            seqs.append(Seq(1, 1, special[i]))
        elif i % 9 == 0:
            seqs.append(Seq(0, 1, 1, int(rng.integers(1, 40))))      # audio only
        else:
            seqs.append(Seq(1, int(rng.integers(1, 4)), int(rng.integers(1, 60)), int(rng.integers(0, 3)) * 7))
    return synth.Workload("max_batch_64", H=2, d=128, seqs=tuple(seqs), split=(32, 48, 48),
                          k_offset_std=0.5, seed=21)


def _all_rows(w, inp, out_bits, gate, label, scale=None):
    p = oracle.Problem.from_workload(w, inp, scale=scale)
    rows = np.arange(w.N * w.H, dtype=np.int64)
    ref = p.attention_rows(rows, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(out_bits, rows, w.H), ref), gate, label)


@pytest.mark.parametrize("quantized", [False, True])
def test_largest_batch_of_sequences(torch_dev, quantized):
    w = _max_batch()
    assert len(w.seqs) == h.H3ATTN_MAX_SEQS
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    out = G.bits(G.run(w, t, quantized=quantized, label="max_batch_64"))
    _all_rows(w, inp, out, G.Q8_GATE if quantized else G.BF16_GATE,
              "max_batch_64" + ("_q8" if quantized else ""))


@pytest.mark.parametrize("d,quantized", [(128, False), (64, False), (128, True)])
def test_most_heads(torch_dev, d, quantized):
    """The most heads the ABI takes (4,096) on two short sequences (a partial
    tile and a 3-token tail): the work-item decode, the per-(sequence, head)
    slices and the quantised path's per-head scales at their largest head index."""
    split = (32, 48, 48) if d == 128 else (16, 24, 24)
    w = synth.Workload("most_heads_d%d" % d, H=4096, d=d, seqs=(Seq(1, 7, 10), Seq(1, 1, 3)), split=split,
                       k_offset_std=0.5, seed=23)
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    label = w.name + ("_q8" if quantized else "")
    out = G.bits(G.run(w, t, quantized=quantized, label=label))
    _all_rows(w, inp, out, G.Q8_GATE if quantized else G.BF16_GATE, label)


def test_single_token_sequences(torch_dev):
    w = synth.Workload("single_tokens", H=3, d=128, seqs=tuple(Seq(1, 1, 1) for _ in range(17)),
                       split=(32, 48, 48), seed=22)
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    out = G.bits(G.run(w, t, label="single_tokens"))
    # one key per sequence: softmax weight 1, so the output is that token's v (to bf16 rounding)
    v = synth.f32_from_bf16_bits(inp["v"]).astype(np.float64)
    got = G.decode(out)
    assert np.abs(got - v).max() <= 2.0 ** -8 * np.abs(v).max()
    _all_rows(w, inp, out, G.BF16_GATE, "single_tokens")


def test_softmax_scale_and_eps(torch_dev):
    w = synth.Workload("scale_eps", H=2, d=128, seqs=(Seq(3, 9, 10, 30), Seq(2, 5, 7)), split=(32, 48, 48),
                       eps=1e-3, seed=23)
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    scale = 0.05
    G.announce("scale_eps workload=%s N=%d scale=%g eps=%g" % (w.name, w.N, scale, w.eps))
    o = h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], eps=w.eps, softmax_scale=scale)
    torch_dev.cuda.synchronize()
    _all_rows(w, inp, G.bits(o), G.BF16_GATE, "scale_eps", scale=scale)


@pytest.mark.parametrize("quantized", [False, True, "mx"])
def test_side_stream_without_workspace(torch_dev, quantized):
    """A call on a side stream with no workspace given: the binding allocates
    the workspace and the output on that stream, so memory that the current
    stream allocates and overwrites right after the call (while the side
    stream's kernels may still run) is never the workspace.  The result must
    equal the same call on the current stream bit for bit."""
    torch = torch_dev
    w = synth.Workload("side_stream", H=4, d=128, seqs=(Seq(4, 16, 24), Seq(1, 8, 8, 50)), split=(32, 48, 48),
                       k_offset_std=0.5, seed=24, quantized=quantized is True, fp4=quantized == "mx")
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    want = G.bits(G.run(w, t, quantized=quantized, label="side_stream_current"))
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda:0")
    G.announce("side_stream quantized=%s N=%d H=%d" % (quantized, w.N, w.H))
    for _ in range(3):
        big = big @ big.t() * 1e-3                         # keeps the current stream busy
    side.wait_stream(cur)                                 # the call starts after that work
    o = h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], eps=w.eps, stream=side,
                     quantized=quantized)
    junk = [torch.full((1 << 24,), 0x7F, dtype=torch.uint8, device="cuda:0") for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    assert np.array_equal(G.bits(o), want)


@pytest.mark.parametrize("mix", range(6))
def test_mfma_ceiling_mixes_run(torch_dev, mix):
    """The matrix-core ceiling diagnostic (every mix: bf16, INT8 and FP4
    MFMAs, alone and with each path's vector work) runs on a small grid and
    leaves only finite values: its hashed operands and vector chains stay in
    range, so the measured rates come from well-defined arithmetic."""
    torch = torch_dev
    wg = 3
    out = torch.full((512 * wg,), float("nan"), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    G.announce("mfma_ceiling mix=%d workgroups=%d" % (mix, wg))
    st = h.mfma_ceiling_raw(mix, wg, 50, out.data_ptr(), int(stream.cuda_stream))
    assert st == 0, h.last_error()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
