"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import os
import sys
from typing import Dict

import numpy as np

import oracle
from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives a lost box)."""
    sys.__stderr__.write("[gpu-step] %s\n" % msg)
    sys.__stderr__.flush()


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_device(inputs: Dict[str, np.ndarray], w: synth.Workload, device="cuda:0"):
    import torch
    t = {}
    for key in ("q", "k", "v", "x", "w_qkv"):
        if key in inputs:
            t[key] = torch.from_numpy(inputs[key].view(np.int16)).to(device).view(torch.bfloat16)
    t["norm_w"] = torch.from_numpy(inputs["norm_w"]).to(device)
    t["rope"] = torch.from_numpy(h.rope_table(w.seqs, w.split, w.d, w.theta)).to(device)
    t["cu"] = inputs["cu_seqlens"]
    return t


def run(w: synth.Workload, t, quantized=False, out=None, workspace=None, stream=None, label=""):
    import torch
    entry = {False: "h3attn_fwd", True: "h3attn_fwd_q8", "mx": "h3attn_fwd_mx"}[quantized]
    announce("%s workload=%s seed=%d N=%d H=%d d=%d entry=%s" % (label, w.name, w.seed, w.N, w.H, w.d, entry))
    o = h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], out=out,
                     workspace=workspace, eps=w.eps, stream=stream, quantized=quantized)
    torch.cuda.synchronize()
    return o


def run_proj(w: synth.Workload, t, out=None, workspace=None, x=None, label=""):
    """h3attn_fwd_proj on uploaded hidden states (``x`` overrides t["x"], e.g. a strided view)."""
    import torch
    announce("%s workload=%s seed=%d N=%d H=%d d=%d D=%d entry=h3attn_fwd_proj" % (
        label, w.name, w.seed, w.N, w.H, w.d, w.model_dim))
    o = h.h3attn_fwd_proj(t["x"] if x is None else x, t["w_qkv"], t["norm_w"], t["rope"], t["cu"], w.H, w.d,
                          out=out, workspace=workspace, eps=w.eps)
    torch.cuda.synchronize()
    return o


def bits(o) -> np.ndarray:
    import torch
    return o.view(torch.int16).cpu().numpy().view(np.uint16)


def decode(b: np.ndarray) -> np.ndarray:
    return synth.f32_from_bf16_bits(b).astype(np.float64)


def metrics(got: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    d = got - ref
    return {
        "max_abs": float(np.abs(d).max()),
        "mean_abs": float(np.abs(d).mean()),
        "rmse": float(np.sqrt((d * d).mean())),
        "rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)),
        "cosine": float((got * ref).sum() / max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300)),
        "ref_mean_abs": float(np.abs(ref).mean()),
    }


# bf16 path gates: the max/mean absolute bounds of the target, plus relative
# guards (rel-L2, cosine) that an all-zero or norm-skipping output would fail.
BF16_GATE = dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2, cosine=0.9999)
# Sharp diagnostic inputs (RMSNorm weights ~2, per-token scales): scores reach
# ~45, and storing qhat' and khat in bf16 alone (the oracle evaluated on the
# rounded values, tests/test_tolerance_floors.py) already gives max-abs 0.031,
# mean-abs 0.0020 and rel-L2 0.0070 on these inputs, above the target's max-abs.
# The gate is twice that floor (measured on the GPU: 0.026 / 0.0014 / 0.0072);
# BF16_GATE applies to every standard workload.
SHARP_GATE = dict(max_abs=6e-2, mean_abs=4e-3, rel_l2=1.4e-2, cosine=0.9999)
# Quantised path: mean-abs bound of the target plus relative guards set at the
# measured error (rel-L2 0.034-0.039, cosine >= 0.9992 on every case) plus margin;
# an all-zero output (rel-L2 1) or a dropped V scale would fail them.
Q8_GATE = dict(mean_abs=2e-2, rel_l2=0.06, cosine=0.998)
# Quantised path against the oracle's step-by-step emulation of it (same codes,
# scales, tiles, lazy maximum and e4m3 probabilities): what is left is the fp32
# arithmetic, the bf16 output rounding (unit roundoff 2^-8) and the odd code that
# fp32 rounds across a boundary.  Measured: rel-L2 0.0024-0.0026 (against 0.034-0.039
# for the exact oracle), cosine >= 0.999996, max-abs <= 0.016; the gate is twice that.
Q8_EMULATION_GATE = dict(max_abs=4e-2, mean_abs=1e-3, rel_l2=5e-3, cosine=0.99999)
# FP4 path against exact attention: a quality guard, not parity.  e2m1 keeps one
# mantissa bit, so P, V, qhat and khat each carry up to ~20% relative rounding;
# the oracle's own FP4 emulation lands at rel-L2 0.22-0.25, cosine 0.969-0.976
# from exact attention on every case.  The error is relative, so the target's
# absolute mean-abs bound (2e-2) is applied at the full-size workloads (outputs
# of mean size ~0.005, measured mean-abs <= 0.0014); the small cases, whose
# outputs are ten times larger, take the relative guards only.  rel-L2 and
# cosine sit just outside the emulation's spread: a dropped block scale
# (rel-L2 ~1) or a misplaced block fails them.
MX_GATE = dict(mean_abs=2e-2, rel_l2=0.30, cosine=0.96)
MX_SMALL_GATE = dict(rel_l2=0.30, cosine=0.96)
# Sharp diagnostic inputs (a few dominant keys per row) magnify the rounding of
# the largest probabilities: the FP4 emulation itself is at rel-L2 0.38, cosine
# 0.927 from exact attention there; the guard sits just outside.
MX_SHARP_GATE = dict(rel_l2=0.45, cosine=0.90)
# FP4 path against the oracle's step-by-step emulation of it (same codes,
# scales, tiles, lazy maximum and FP4 probabilities): what is left is the bf16
# output rounding (unit roundoff 2^-8, rel-L2 ~ 2^-8 / sqrt(3) ~ 0.0017 on
# uniform-ish values) and the rare code fp32 rounds across a boundary.
# Measured on five workloads: rel-L2 0.00157-0.00168, cosine >= 0.9999986,
# largest row rel error 0.0042; the gate is about twice that.
MX_EMULATION_GATE = dict(rel_l2=3.5e-3, cosine=0.999995, max_rel_row=1e-2)


def check(m: Dict[str, float], gate: Dict[str, float], label: str):
    bad = []
    for k, lim in gate.items():
        if k == "cosine":
            if not m[k] >= lim:
                bad.append("%s %.6g < %g" % (k, m[k], lim))
        elif not m[k] <= lim:
            bad.append("%s %.6g > %g" % (k, m[k], lim))
    announce("%s metrics %s" % (label, {k: round(v, 8) for k, v in m.items()}))
    assert not bad, "%s: %s" % (label, "; ".join(bad))


def oracle_rows(w: synth.Workload, inputs, rows: np.ndarray) -> np.ndarray:
    p = oracle.Problem.from_workload(w, inputs)
    return p.attention_rows(rows, nthreads=oracle_threads())


def gpu_rows(out_bits: np.ndarray, rows: np.ndarray, H: int) -> np.ndarray:
    return decode(out_bits[rows // H, rows % H])
