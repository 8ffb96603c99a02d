"""The entry points under HIP graph capture (the header's claim: no call
allocates or copies host memory, cu_seqlens is read on the host and baked into
kernel arguments, so a call may be captured).  Each graph is replayed several
times with eager work between the replays, and every replay must reproduce the
eager result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
Seq = synth.Seq

W = synth.Workload("graph_ragged", H=2, d=128, seqs=(Seq(3, 10, 11, 7), Seq(1, 4, 5, 70)), split=(32, 48, 48),
                   k_offset_std=0.5, seed=61)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _replays(torch, fn, out, label, n=4):
    eager = out.clone()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):                       # capture on a side stream, as torch requires
        g = torch.cuda.CUDAGraph()
        out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.synchronize()
    for r in range(n):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda:0") * 3.0   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        G.announce("%s replay %d" % (label, r))
        assert torch.equal(out, eager), "%s: replay %d differs from the eager result" % (label, r)
        del junk


@pytest.mark.parametrize("path", ["bf16", "q8", "mx", "sparse"])
def test_attention_entry_points_replay(torch_dev, path):
    torch = torch_dev
    inp = synth.generate(W)
    t = G.to_device(inp, W)
    out = torch.empty_like(t["q"])
    quant = {"q8": True, "mx": "mx"}.get(path, False)
    ws = torch.empty(h.h3attn_workspace_size(h.params_for(t["q"], t["k"], t["v"], out, W.S), inp["cu_seqlens"],
                                             2 if path == "sparse" else quant), dtype=torch.uint8,
                     device="cuda:0")
    tiles = torch.empty((h.sparse_items(inp["cu_seqlens"], W.H), 3), dtype=torch.int32, device="cuda:0")

    def fn():
        if path == "sparse":
            h.h3attn_fwd_sparse(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], 3, block_tiles=tiles,
                                out=out, workspace=ws, eps=W.eps, stream=torch.cuda.current_stream())
        else:
            h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], out=out, workspace=ws,
                         eps=W.eps, quantized=quant, stream=torch.cuda.current_stream())

    G.announce("graph %s eager" % path)
    fn()
    torch.cuda.synchronize()
    _replays(torch, fn, out, "graph " + path)


@pytest.mark.parametrize("quantized", [False, True])
def test_layer_entry_points_replay(torch_dev, quantized):
    """The projection (bf16, or with the quantised prologue), the attention and
    the output projection captured as one graph."""
    torch = torch_dev
    w = synth.Workload("graph_layer", H=2, d=128, seqs=(Seq(2, 8, 9, 37), Seq(1, 3, 3)), split=(32, 48, 48),
                       seed=62, model_dim=256)
    inp, go = synth.generate(w), synth.generate_out(w)
    t = G.to_device(inp, w)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    w_o, resid, gate = up(go["w_o"]), up(go["resid"]), torch.from_numpy(go["gate"]).to("cuda:0")
    o = torch.empty((w.N, w.H, w.d), dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty((w.N, w.model_dim), dtype=torch.bfloat16, device="cuda:0")
    params = h._proj_params(t["x"], t["w_qkv"], w.H, w.d, w.S, o.stride(0), w.eps, 0.0)
    ws = torch.empty(h.h3attn_workspace_size(params, inp["cu_seqlens"], 4 if quantized else 0), dtype=torch.uint8,
                     device="cuda:0")

    def fn():
        s = torch.cuda.current_stream()
        h.h3attn_fwd_proj(t["x"], t["w_qkv"], t["norm_w"], t["rope"], t["cu"], w.H, w.d, out=o, workspace=ws,
                          eps=w.eps, stream=s, quantized=quantized)
        h.h3attn_out_proj(o, w_o, t["cu"], gate=gate, resid=resid, out=y, stream=s)

    label = "graph layer%s" % (" q8" if quantized else "")
    G.announce(label + " eager")
    fn()
    torch.cuda.synchronize()
    _replays(torch, fn, y, label)
