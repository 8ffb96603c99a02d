"""Seeded synthetic inputs for the fused RMSNorm + RoPE + attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no normalisation, rotation or attention).  Both the HIP
path and the CPU oracle consume exactly the arrays produced here, so neither
has to regenerate anything.

Workloads follow the token layout of a joint video+audio diffusion block: each
sequence is a t x h x w video latent grid in raster order, optionally followed
by audio tokens, and several sequences may be packed back to back (ragged
``cu_seqlens``).  The pages ("Buyer Questions: Current Evidence Status", Q4 and
Q10) describe these packed sequences but publish no tensors, so every value is
drawn here: Q/K/V ~ N(0, 1) rounded once to bf16 (round to nearest even),
RMSNorm weights 1 + 0.1 N(0, 1) in fp32, and for the joint workload a
per-(head, channel) mean offset N(0, 0.5^2) added to raw K before rounding.
Workloads with a model dimension D start one step earlier, at the attention
layer's input: hidden states x ~ N(0, 1) [N, D] and a QKV weight
W ~ N(0, 1/D) [3*H*d, D], both rounded once to bf16, so the projected q, k, v
have unit variance like the direct inputs (the pages publish no weights).

Random streams come from numpy's Philox counter-based generator, one
independent child stream per tensor (``SeedSequence.spawn``).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = ["Seq", "Workload", "WORKLOADS", "generate", "generate_out", "sample_rows",
           "bf16_bits_from_f32", "f32_from_bf16_bits", "total_tokens"]


@dataclasses.dataclass(frozen=True)
class Seq:
    """One packed sequence: a T x Hg x Wg video grid then ``n_audio`` tokens."""
    T: int
    Hg: int
    Wg: int
    n_audio: int = 0

    @property
    def n_video(self) -> int:
        return self.T * self.Hg * self.Wg

    @property
    def n(self) -> int:
        return self.n_video + self.n_audio


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    d: int
    seqs: Tuple[Seq, ...]
    split: Tuple[int, int, int]          # video RoPE dims for t, h, w
    theta: float = 10000.0
    eps: float = 1e-6
    k_offset_std: float = 0.0            # per-(head, channel) offset on raw K
    seed: int = 0
    quantized: bool = False
    fp4: bool = False                    # MXFP4 path (h3attn_fwd_mx)
    sharp: bool = False                  # diagnostic: per-token scale + larger weights
    model_dim: int = 0                   # D > 0: inputs are hidden states x [N, D] and W_qkv
    keep_tiles: int = 0                  # > 0: block-sparse attention keeping this many 64-key tiles per 256-row block
    description: str = ""

    @property
    def N(self) -> int:
        return sum(s.n for s in self.seqs)

    @property
    def S(self) -> int:
        return len(self.seqs)

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.S + 1, dtype=np.int32)
        cu[1:] = np.cumsum([s.n for s in self.seqs])
        return cu

    def flops(self) -> float:
        """Attention FLOP count 4 * sum(n_i^2) * d * H (QK^T and PV, exps excluded)."""
        return 4.0 * sum(float(s.n) ** 2 for s in self.seqs) * self.d * self.H

    def proj_flops(self) -> float:
        """QKV projection FLOP count 2 * N * D * 3*H*d (0 without a model dimension)."""
        return 2.0 * self.N * self.model_dim * 3 * self.H * self.d

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def total_tokens(seqs: Sequence[Seq]) -> int:
    return sum(s.n for s in seqs)


_SPLIT128 = (32, 48, 48)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", H=2, d=64, seqs=(Seq(4, 8, 8),), split=(16, 24, 24), seed=1001,
        description="t4 x h8 x w8 video grid, H=2, d=64"),
    "video": Workload(
        "video", H=24, d=128, seqs=(Seq(36, 30, 54),), split=_SPLIT128, seed=1002,
        description="video-only t36 x h30 x w54 = 58,320 tokens, H=24, d=128"),
    "joint": Workload(
        "joint", H=24, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128,
        k_offset_std=0.5, seed=1003,
        description="joint t31 x h48 x w84 video + 250 audio = 125,242 tokens, H=24, d=128"),
    "joint_h3": Workload(
        "joint_h3", H=3, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128,
        k_offset_std=0.5, seed=1006,
        description="one GPU's share of the joint workload under 8-way head sharding: "
                    "125,242 tokens, H=3, d=128"),
    "ragged": Workload(
        "ragged", H=24, d=128,
        seqs=(Seq(14, 36, 36), Seq(25, 30, 60, 250), Seq(8, 30, 30)), split=_SPLIT128,
        seed=1004,
        description="ragged 18,144 / 45,250 / 7,200 tokens, H=24, d=128"),
    "q8": Workload(
        "q8", H=24, d=128, seqs=(Seq(36, 30, 54),), split=_SPLIT128, seed=1005,
        quantized=True,
        description="INT8-QK / FP8-PV path at the 58,320-token video shape"),
    "mx": Workload(
        "mx", H=24, d=128, seqs=(Seq(36, 30, 54),), split=_SPLIT128, seed=1007, fp4=True,
        description="MXFP4 path at the 58,320-token video shape"),
    "sparse_joint": Workload(
        "sparse_joint", H=24, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128,
        k_offset_std=0.5, seed=1003, keep_tiles=490,
        description="block-sparse attention on the joint 125,242-token sequence (the joint inputs), "
                    "490 of its 1,957 64-key tiles (25%) kept per 256-row query block by pooled score"),
    "proj_tiny": Workload(
        "proj_tiny", H=2, d=64, seqs=(Seq(4, 8, 8),), split=(16, 24, 24), seed=1011, model_dim=128,
        description="QKV projection (D=128) + attention on the t4 x h8 x w8 grid, H=2, d=64"),
    "proj_joint": Workload(
        "proj_joint", H=24, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128, seed=1013,
        model_dim=3072,
        description="QKV projection (D=3072) + attention on the joint 125,242-token sequence, H=24"),
    "proj_q8_joint": Workload(
        "proj_q8_joint", H=24, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128, seed=1013,
        model_dim=3072, quantized=True,
        description="the proj_joint inputs on the quantised path: QKV projection (D=3072) with the INT8/FP8 "
                    "prologue in its epilogue + INT8/FP8 attention, H=24"),
    "proj_joint_h3": Workload(
        "proj_joint_h3", H=3, d=128, seqs=(Seq(31, 48, 84, 250),), split=_SPLIT128, seed=1016,
        model_dim=3072,
        description="one GPU's share of proj_joint under 8-way head sharding: full hidden states "
                    "x [125242, 3072], the 3 heads' rows of W"),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, offset=None, row_scale=None,
                 chunk_rows: int = 1 << 15) -> np.ndarray:
    """N(0,1) draws (plus optional per-(head, channel) offset / per-token scale) -> bf16 bits."""
    n = shape[0]
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if offset is not None:
            x += offset[None]
        if row_scale is not None:
            x *= row_scale[r0:r1].reshape((-1,) + (1,) * (len(shape) - 1))
        out[r0:r1] = bf16_bits_from_f32(x)
    return out


def generate(w: Workload) -> Dict[str, np.ndarray]:
    """Draw every input of workload ``w``.

    Returns q, k, v as uint16 bf16 bits of shape [N, H, d] (token-major,
    token stride H*d), norm_w float32 [2, H, d] (q weights then k weights),
    k_offset float32 [H, d] (zeros when unused) and cu_seqlens int32 [S+1].
    With a model dimension D the inputs are instead x (bf16 bits [N, D]) and
    w_qkv (bf16 bits [3*H*d, D]); q, k and v are then not drawn.
    """
    ss = np.random.SeedSequence(w.seed)
    kids = ss.spawn(10)
    gen = [np.random.Generator(np.random.Philox(k)) for k in kids]
    N, H, d = w.N, w.H, w.d
    if w.model_dim > 0:
        if w.sharp or w.k_offset_std > 0:
            raise ValueError("projection workloads draw plain hidden states")
        D = w.model_dim
        x = _normal_bf16(gen[8], (N, D))
        w_qkv = np.empty((3 * H * d, D), dtype=np.uint16)
        for r0 in range(0, 3 * H * d, 1024):
            r1 = min(3 * H * d, r0 + 1024)
            w_qkv[r0:r1] = bf16_bits_from_f32(
                gen[9].standard_normal((r1 - r0, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D)))
        norm_w = (1.0 + 0.1 * gen[3].standard_normal((2, H, d))).astype(np.float32)
        return {"x": x, "w_qkv": w_qkv, "norm_w": norm_w, "k_offset": np.zeros((H, d), dtype=np.float32),
                "cu_seqlens": w.cu_seqlens()}
    k_offset = np.zeros((H, d), dtype=np.float32)
    if w.k_offset_std > 0:
        k_offset = (gen[4].standard_normal((H, d)) * w.k_offset_std).astype(np.float32)
    q_scale = k_scale = None
    if w.sharp:
        # per-token magnitudes log-uniform in [0.1, 10] exercise the RMSNorm step
        q_scale = np.exp(gen[5].uniform(np.log(0.1), np.log(10.0), N)).astype(np.float32)
        k_scale = np.exp(gen[6].uniform(np.log(0.1), np.log(10.0), N)).astype(np.float32)
    q = _normal_bf16(gen[0], (N, H, d), row_scale=q_scale)
    k = _normal_bf16(gen[1], (N, H, d), offset=k_offset if w.k_offset_std > 0 else None,
                     row_scale=k_scale)
    v = _normal_bf16(gen[2], (N, H, d))
    if w.sharp:
        norm_w = (2.0 + 0.2 * gen[3].standard_normal((2, H, d))).astype(np.float32)
    else:
        norm_w = (1.0 + 0.1 * gen[3].standard_normal((2, H, d))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "norm_w": norm_w, "k_offset": k_offset,
            "cu_seqlens": w.cu_seqlens()}


def generate_out(w: Workload) -> Dict[str, np.ndarray]:
    """Inputs of the output projection with its gated residual for workload
    ``w`` (independent child streams of the workload seed; the draws of
    ``generate`` are unchanged): a stand-in attention output attn ~ 0.1 N(0, 1)
    [N, H*d] (the size of the attention outputs of these workloads), the
    weight w_o ~ N(0, 1/(H*d)) [D, H*d] and the residual resid ~ N(0, 1)
    [N, D], all bf16 bits, and one fp32 gate per sequence and channel,
    gate ~ 1 + 0.5 N(0, 1) [S, D].  D is the model dimension (H*d without one)."""
    kids = np.random.SeedSequence(w.seed).spawn(14)[10:]
    gen = [np.random.Generator(np.random.Philox(k)) for k in kids]
    N, hd = w.N, w.H * w.d
    D = w.model_dim if w.model_dim > 0 else hd
    attn = np.empty((N, hd), dtype=np.uint16)
    for r0 in range(0, N, 1 << 15):
        r1 = min(N, r0 + (1 << 15))
        attn[r0:r1] = bf16_bits_from_f32(gen[0].standard_normal((r1 - r0, hd), dtype=np.float32) * np.float32(0.1))
    w_o = bf16_bits_from_f32(gen[1].standard_normal((D, hd), dtype=np.float32) * np.float32(1.0 / np.sqrt(hd)))
    resid = _normal_bf16(gen[2], (N, D))
    gate = (1.0 + 0.5 * gen[3].standard_normal((w.S, D))).astype(np.float32)
    return {"attn": attn, "w_o": w_o, "resid": resid, "gate": gate, "cu_seqlens": w.cu_seqlens()}


def sample_rows(w: Workload, n_rows: int, seed: int | None = None) -> np.ndarray:
    """Seeded (token, head) query rows, encoded as token * H + head (int64, sorted).

    Always includes the first and last token of every non-empty sequence and
    the first and last audio token (for one seeded head each); the rest are
    drawn uniformly without replacement.  ``n_rows >= N*H`` returns all rows.
    """
    total = w.N * w.H
    if n_rows >= total:
        return np.arange(total, dtype=np.int64)
    rng = np.random.Generator(np.random.Philox(np.random.SeedSequence(
        (w.seed if seed is None else seed) + 7777)))
    forced: List[int] = []
    start = 0
    for s in w.seqs:
        if s.n > 0:
            for tok in (start, start + s.n - 1):
                forced.append(tok * w.H + int(rng.integers(w.H)))
            if s.n_audio > 0:
                for tok in (start + s.n_video, start + s.n - 1):
                    forced.append(tok * w.H + int(rng.integers(w.H)))
        start += s.n
    chosen = set(forced)
    need = n_rows - len(chosen)
    while need > 0:
        cand = rng.integers(0, total, size=2 * need + 16, dtype=np.int64)
        for c in cand.tolist():
            if c not in chosen:
                chosen.add(c)
                need -= 1
                if need == 0:
                    break
    return np.array(sorted(chosen), dtype=np.int64)
