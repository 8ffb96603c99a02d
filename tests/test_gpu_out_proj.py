"""GPU parity of the output projection with the gated residual
(h3attn_out_proj) and of the whole attention layer it closes
(h3attn_fwd_proj then h3attn_out_proj), against the fp64 oracle.

Element-wise: on seeded stand-in attention outputs, every output element
within 2^-8 |oracle| + 1e-5 (one bf16 rounding plus fp32 accumulation), for
ragged packings with an empty sequence, a channel count that leaves the last
256-channel pair half full, a gate of 1 / no residual, and the in-place
residual update; the 125,242-token shape (K = D = 3072) on 512 sampled
tokens.  Layer: x -> q, k, v -> attention -> out on every token of small
cases against the oracle's chain (projection, attention, output projection
in fp64), at the bf16 gates for the block output and, computed without the
residual, for the attention branch alone.
"""
import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
Seq = synth.Seq

CASES = {
    "out_ragged_D256": synth.Workload("out_ragged_D256", H=2, d=128, seqs=(Seq(2, 8, 9, 37), Seq(0, 1, 1), Seq(1, 3, 3)),
                                      split=(32, 48, 48), seed=41, model_dim=256),
    "out_half_pair_D384_d64": synth.Workload("out_half_pair_D384_d64", H=3, d=64, seqs=(Seq(2, 6, 10, 3), Seq(1, 5, 5)),
                                             split=(16, 24, 24), seed=42, model_dim=384),
    "out_single_D128": synth.Workload("out_single_D128", H=1, d=128, seqs=(Seq(3, 7, 9),), split=(32, 48, 48),
                                      seed=43, model_dim=128),
}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _up(torch, a):
    return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def _close(got, ref, label):
    err = np.abs(got - ref)
    bad = err > 2.0 ** -8 * np.abs(ref) + 1e-5
    assert not bad.any(), "%s: %d of %d elements off (worst %.3g)" % (label, int(bad.sum()), bad.size, err.max())


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("form", ["gated_residual", "plain", "in_place"])
def test_out_proj_all_elements(torch_dev, name, form):
    w = CASES[name]
    g = synth.generate_out(w)
    torch = torch_dev
    attn = _up(torch, g["attn"]).view(w.N, w.H, w.d)
    w_o = _up(torch, g["w_o"])
    gate = torch.from_numpy(g["gate"]).to("cuda:0") if form != "plain" else None
    resid = _up(torch, g["resid"]) if form != "plain" else None
    G.announce("out_proj %s %s N=%d H=%d d=%d D=%d" % (name, form, w.N, w.H, w.d, w.model_dim))
    out = h.h3attn_out_proj(attn, w_o, g["cu_seqlens"], gate=gate, resid=resid,
                            out=resid if form == "in_place" else None)
    torch.cuda.synchronize()
    if form == "in_place":
        assert out.data_ptr() == resid.data_ptr()
    ref = oracle.out_proj(g["attn"], g["w_o"], g["cu_seqlens"], gate=None if form == "plain" else g["gate"],
                          resid=None if form == "plain" else g["resid"])
    _close(G.decode(G.bits(out)), ref, "%s %s" % (name, form))


def test_out_proj_full_size_sampled(torch_dev):
    w = synth.WORKLOADS["proj_joint"]
    g = synth.generate_out(w)
    torch = torch_dev
    attn = _up(torch, g["attn"]).view(w.N, w.H, w.d)
    G.announce("out_proj proj_joint N=%d K=%d D=%d" % (w.N, w.H * w.d, w.model_dim))
    out = h.h3attn_out_proj(attn, _up(torch, g["w_o"]), g["cu_seqlens"],
                            gate=torch.from_numpy(g["gate"]).to("cuda:0"), resid=_up(torch, g["resid"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(w.N, 512, replace=False))
    toks[0], toks[-1] = 0, w.N - 1
    ref = oracle.out_proj(g["attn"], g["w_o"], g["cu_seqlens"], gate=g["gate"], resid=g["resid"], rows=toks)
    _close(G.decode(G.bits(out))[toks], ref, "proj_joint out_proj")


LAYER = {
    "layer_tiny": synth.WORKLOADS["proj_tiny"],
    "layer_ragged": synth.Workload("layer_ragged", H=2, d=128, seqs=(Seq(2, 8, 9, 37), Seq(0, 1, 1), Seq(1, 3, 3)),
                                   split=(32, 48, 48), seed=44, model_dim=256),
}


@pytest.mark.parametrize("name", sorted(LAYER))
def test_attention_layer_all_tokens(torch_dev, name):
    w = LAYER[name]
    inp, g = synth.generate(w), synth.generate_out(w)
    torch = torch_dev
    t = G.to_device(inp, w)
    o = G.run_proj(w, t, label=name + " layer")
    G.announce("out_proj %s layer" % name)
    gate = torch.from_numpy(g["gate"]).to("cuda:0")
    out = h.h3attn_out_proj(o, _up(torch, g["w_o"]), inp["cu_seqlens"], gate=gate, resid=_up(torch, g["resid"]))
    branch = h.h3attn_out_proj(o, _up(torch, g["w_o"]), inp["cu_seqlens"], gate=gate)
    torch.cuda.synchronize()
    p = oracle.Problem.from_projection(w, inp)
    attn = p.attention_rows(np.arange(w.N * w.H), nthreads=G.oracle_threads()).reshape(w.N, w.H * w.d)
    ref = oracle.out_proj(attn, g["w_o"], inp["cu_seqlens"], gate=g["gate"], resid=g["resid"])
    ref_branch = oracle.out_proj(attn, g["w_o"], inp["cu_seqlens"], gate=g["gate"])
    # the block output (dominated by the residual) and, without the residual, the
    # attention branch alone (so its error is not hidden under the residual's rounding)
    G.check(G.metrics(G.decode(G.bits(out)), ref), G.BF16_GATE, name + " out")
    G.check(G.metrics(G.decode(G.bits(branch)), ref_branch), G.BF16_GATE, name + " branch")
