"""GPU parity of the fused QKV projection path (h3attn_fwd_proj,
h3attn_proj_prologue) against the fp64 oracle's projection
(``oracle.project``) followed by its RMSNorm, RoPE and attention.

Stage parity: the normalised, rotated q and k and the projected v of the
natural-layout export are compared element by element, |GPU - oracle| <=
2^-8 |oracle| + 1e-5 (storing in bf16 rounds to within 2^-8 relative, the
unit roundoff of its 8-bit significand; the fp32 matrix product and the fp32
norm and rotation add a few 1e-6 absolute).  End to end: the attention output at the bf16
gates.  Small cases cover every token and row: ragged and empty sequences,
audio tokens, both head dims, model dims of 1, 2, 3 and 5 pipeline slabs and
hidden states read through a token stride wider than the model dim, and at
head dim 128 model dims of 2 and 6 slabs (64, 192), the latter with three
heads (an odd number of feature blocks, so the last workgroup's second block
is absent).  The
125,242-token joint shape is checked on sampled rows (all three heads of one
GPU's share, and four of the 24 heads of the whole layer).
"""
import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
Seq = synth.Seq

SMALL = {
    "proj_tiny": synth.WORKLOADS["proj_tiny"],
    "proj_ragged_d128_D160": synth.Workload(
        "proj_ragged_d128_D160", H=2, d=128, seqs=(Seq(2, 8, 9, 37), Seq(0, 1, 1), Seq(1, 3, 3), Seq(0, 1, 1, 5)),
        split=(32, 48, 48), seed=31, model_dim=160),
    "proj_single_slab_D32": synth.Workload(
        "proj_single_slab_D32", H=1, d=128, seqs=(Seq(3, 7, 9),), split=(32, 48, 48), seed=32, model_dim=32),
    "proj_two_slabs_D64_long": synth.Workload(
        "proj_two_slabs_D64_long", H=2, d=128, seqs=(Seq(4, 15, 18, 20),), split=(32, 48, 48), seed=33,
        model_dim=64),
    "proj_ragged_d128_D192_h3": synth.Workload(
        "proj_ragged_d128_D192_h3", H=3, d=128, seqs=(Seq(2, 8, 9, 37), Seq(0, 1, 1), Seq(1, 5, 7, 3)),
        split=(32, 48, 48), seed=35, model_dim=192),
    "proj_one_slab_D64": synth.Workload(
        "proj_one_slab_D64", H=2, d=128, seqs=(Seq(3, 9, 11),), split=(32, 48, 48), seed=36, model_dim=64),
    "proj_three_slabs_D96_d64": synth.Workload(
        "proj_three_slabs_D96_d64", H=3, d=64, seqs=(Seq(2, 6, 10, 3), Seq(1, 5, 5)), split=(16, 24, 24),
        seed=34, model_dim=96),
}
X_PAD = {"proj_three_slabs_D96_d64": 64, "proj_ragged_d128_D160": 8,   # extra elements per x row
         "proj_ragged_d128_D192_h3": 40}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _upload(w, inp, torch):
    t = G.to_device(inp, w)
    pad = X_PAD.get(w.name, 0)
    x = t["x"]
    if pad:
        wide = torch.zeros((w.N, w.model_dim + pad), dtype=torch.bfloat16, device=x.device)
        wide[:, :w.model_dim] = x
        x = wide[:, :w.model_dim]
        assert x.stride(0) == w.model_dim + pad
    return t, x


def _stage_close(got, ref, label):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    bad = err > bound
    assert not bad.any(), "%s: %d of %d elements off (worst %.3g)" % (label, int(bad.sum()), bad.size, err.max())


def _sub_problem(w, inp, heads):
    """The oracle problem restricted to `heads` (heads are independent)."""
    hd = w.H * w.d
    sel = np.concatenate([part * hd + hh * w.d + np.arange(w.d) for part in range(3) for hh in heads])
    ws = w.replace(H=len(heads))
    sub = {"x": inp["x"], "w_qkv": np.ascontiguousarray(inp["w_qkv"][sel]),
           "norm_w": np.ascontiguousarray(inp["norm_w"][:, heads])}
    return ws, oracle.Problem.from_projection(ws, sub)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_projection_stage_all_tokens(torch_dev, name):
    w = SMALL[name]
    inp = synth.generate(w)
    t, x = _upload(w, inp, torch_dev)
    G.announce("proj stage %s N=%d H=%d d=%d D=%d x_stride=%d" % (name, w.N, w.H, w.d, w.model_dim, x.stride(0)))
    qh, kh, v = h.h3attn_proj_prologue(x, t["w_qkv"], t["norm_w"], t["rope"], t["cu"], w.H, w.d, eps=w.eps)
    torch_dev.cuda.synchronize()
    p = oracle.Problem.from_projection(w, inp)
    rows = np.arange(w.N * w.H, dtype=np.int64)
    for which, got in ((0, qh), (1, kh)):
        ref = p.prologue_rows(which, rows, nthreads=G.oracle_threads())
        _stage_close(G.decode(G.bits(got)).reshape(-1, w.d), ref, "%s %s" % (name, "qk"[which]))
    vref = oracle.project(inp["x"], inp["w_qkv"])[:, 2 * w.H * w.d:]
    _stage_close(G.decode(G.bits(v)).reshape(w.N, -1), vref, name + " v")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_projection_attention_all_rows(torch_dev, name):
    w = SMALL[name]
    inp = synth.generate(w)
    t, x = _upload(w, inp, torch_dev)
    out = G.bits(G.run_proj(w, t, x=x, label=name))
    p = oracle.Problem.from_projection(w, inp)
    rows = np.arange(w.N * w.H, dtype=np.int64)
    ref = p.attention_rows(rows, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(out, rows, w.H), ref), G.BF16_GATE, name)


def test_projection_one_gpu_share_sampled(torch_dev):
    # the 8-way head split of the joint layer: H=3, full hidden states
    w = synth.WORKLOADS["proj_joint_h3"]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    out = G.bits(G.run_proj(w, t, label="proj_joint_h3"))
    del t
    rows = synth.sample_rows(w, 4096)
    p = oracle.Problem.from_projection(w, inp)
    ref = p.attention_rows(rows, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(out, rows, w.H), ref), G.BF16_GATE, "proj_joint_h3")


def test_projection_full_layer_sampled(torch_dev):
    # all 24 heads on the GPU (the bench configuration); the oracle takes four
    # of them, stage outputs at 512 sampled tokens and 1024 sampled output rows
    w = synth.WORKLOADS["proj_joint"]
    heads = [0, 7, 13, 23]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    out = G.bits(G.run_proj(w, t, label="proj_joint"))
    G.announce("proj stage proj_joint (natural export)")
    qh, kh, v = h.h3attn_proj_prologue(t["x"], t["w_qkv"], t["norm_w"], t["rope"], t["cu"], w.H, w.d, eps=w.eps)
    torch_dev.cuda.synchronize()
    qh, kh, v = (G.decode(G.bits(a)) for a in (qh, kh, v))
    del t
    ws, p = _sub_problem(w, inp, heads)
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(w.N, 512, replace=False))
    toks[0], toks[-1] = 0, w.N - 1
    for j, hh in enumerate(heads):
        r = toks * len(heads) + j
        _stage_close(qh[toks, hh], p.prologue_rows(0, r, nthreads=G.oracle_threads()), "proj_joint q h%d" % hh)
        _stage_close(kh[toks, hh], p.prologue_rows(1, r, nthreads=G.oracle_threads()), "proj_joint k h%d" % hh)
        vref = oracle.project(inp["x"], inp["w_qkv"][2 * w.H * w.d + hh * w.d:2 * w.H * w.d + (hh + 1) * w.d],
                              rows=toks)
        _stage_close(v[toks, hh], vref, "proj_joint v h%d" % hh)
    otoks = np.sort(rng.choice(w.N, 256, replace=False))
    rows_sub = (otoks[:, None] * len(heads) + np.arange(len(heads))[None, :]).reshape(-1)
    ref = p.attention_rows(rows_sub, nthreads=G.oracle_threads())
    got = G.decode(out[otoks][:, heads]).reshape(-1, w.d)
    G.check(G.metrics(got, ref), G.BF16_GATE, "proj_joint")
