"""ctypes front end of the fp64 CPU oracle (``h3_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its binding) never loads it.

The oracle evaluates, in fp64 from the same bf16 input bits the GPU reads,
per-head RMSNorm of q and k, interleaved-pair RoPE (3D t/h/w sections for
video tokens, one section over all dims for audio tokens) and block-diagonal
non-causal softmax attention; see the C file's header for the definitions and
the pages they follow.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "h3_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
# H3_ORACLE_LIB points at another build of h3_oracle.c (a sanitized one in the tests).
_LIB_PATH = os.environ.get("H3_ORACLE_LIB") or os.path.join(_BUILD, "liboracle.so")

# Query rows sharing one block-sparse tile list.  The pages credit a sparse
# attention backend with the refine's speed-up ("Open-H3-Regenerate-2K", "Speed
# on one B200 (GB200)", per-module table) but fix no algorithm and no block
# size; this definition takes blocks of 256 query rows (the granularity at which
# the attention kernel streams keys) by 64-key tiles, the softmax exactly over
# the kept keys.
SPARSE_BLOCK = 256


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                               "-Wall", "-Wno-unused-function", src, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, out)
    return out


class _Seq(C.Structure):
    _fields_ = [("T", C.c_int32), ("Hg", C.c_int32), ("Wg", C.c_int32), ("n_audio", C.c_int32)]


class _Problem(C.Structure):
    _fields_ = [("H", C.c_int32), ("d", C.c_int32), ("S", C.c_int32), ("rope", C.c_int32),
                ("split", C.c_int32 * 3), ("pad", C.c_int32),
                ("theta", C.c_double), ("eps", C.c_double), ("scale", C.c_double),
                ("cu", C.POINTER(C.c_int32)), ("seqs", C.POINTER(_Seq)),
                ("q", C.POINTER(C.c_uint16)), ("k", C.POINTER(C.c_uint16)),
                ("v", C.POINTER(C.c_uint16)),
                ("q_stride", C.c_int64), ("k_stride", C.c_int64), ("v_stride", C.c_int64),
                ("norm_w", C.POINTER(C.c_float)),
                ("qf", C.POINTER(C.c_double)), ("kf", C.POINTER(C.c_double)),
                ("vf", C.POINTER(C.c_double))]


_lib = None


def lib(path: Optional[str] = None):
    """Load (building if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(C.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(C.CDLL(_LIB_PATH))
    return _lib


def _bind(L):
    P = C.POINTER
    L.orc_bf16_to_f64.restype = C.c_double
    L.orc_bf16_to_f64.argtypes = [C.c_uint16]
    L.orc_token_pos.argtypes = [P(_Problem), C.c_int64, P(C.c_int32), P(C.c_int32), P(C.c_int32)]
    L.orc_rope_angles.argtypes = [P(_Problem), C.c_int32, P(C.c_int32), P(C.c_double)]
    L.orc_rmsnorm.argtypes = [P(C.c_uint16), P(C.c_float), C.c_int, C.c_double, P(C.c_double)]
    L.orc_rmsnorm_f64.argtypes = [P(C.c_double), P(C.c_float), C.c_int, C.c_double, P(C.c_double)]
    L.orc_rope_rotate.argtypes = [P(C.c_double), P(C.c_double), C.c_int, P(C.c_double)]
    L.orc_prologue_rows.argtypes = [P(_Problem), C.c_int, P(C.c_int64), C.c_int64,
                                    P(C.c_double), C.c_int]
    L.orc_attention_core.argtypes = [P(C.c_double), C.c_int64, P(C.c_double), P(C.c_double),
                                     C.c_int64, C.c_int, C.c_double, P(C.c_double)]
    L.orc_attention_rows.argtypes = [P(_Problem), P(C.c_int64), C.c_int64, P(C.c_double), C.c_int]
    L.orc_default_threads.restype = C.c_int
    L.orc_q8_kmean.argtypes = [P(_Problem), P(C.c_double), C.c_int]
    L.orc_q8_block_quant.argtypes = [P(_Problem), C.c_int, C.c_int32, C.c_int32, C.c_int32,
                                     P(C.c_double), P(C.c_double), P(C.c_double), P(C.c_int8)]
    L.orc_q8_v_quant.argtypes = [P(_Problem), C.c_int32, C.c_int32, P(C.c_double),
                                 P(C.c_double), P(C.c_uint8)]
    L.orc_q8_softmax_pv.argtypes = [P(C.c_double), C.c_int64, P(C.c_double), C.c_int, P(C.c_double)]
    L.orc_q8_attention_rows.restype = C.c_int
    L.orc_q8_attention_rows.argtypes = [P(_Problem), P(C.c_int64), C.c_int64, P(C.c_double),
                                        P(C.c_double), C.c_int]
    L.orc_e2m1_encode.restype = C.c_uint8
    L.orc_e2m1_encode.argtypes = [C.c_double]
    L.orc_e2m1_decode.restype = C.c_double
    L.orc_e2m1_decode.argtypes = [C.c_uint8]
    L.orc_mx_scale_exp.restype = C.c_int
    L.orc_mx_scale_exp.argtypes = [C.c_double]
    L.orc_mx_block.restype = C.c_int
    L.orc_mx_block.argtypes = [P(C.c_double), C.c_int, P(C.c_uint8)]
    L.orc_mx_qk_quant.restype = C.c_int
    L.orc_mx_qk_quant.argtypes = [P(_Problem), C.c_int, C.c_int32, C.c_int32, P(C.c_double),
                                  P(C.c_uint8), P(C.c_int32), C.c_int]
    L.orc_mx_v_quant.restype = C.c_int
    L.orc_mx_v_quant.argtypes = [P(_Problem), C.c_int32, C.c_int32, P(C.c_uint8), P(C.c_int32)]
    L.orc_mx_softmax_pv.argtypes = [P(C.c_double), C.c_int64, P(C.c_double), C.c_int, P(C.c_double)]
    L.orc_mx_attention_rows.restype = C.c_int
    L.orc_mx_attention_rows.argtypes = [P(_Problem), P(C.c_int64), C.c_int64, P(C.c_double),
                                        P(C.c_double), C.c_int]
    L.orc_e4m3_encode.restype = C.c_uint8
    L.orc_e4m3_encode.argtypes = [C.c_double]
    L.orc_e4m3_decode.restype = C.c_double
    L.orc_e4m3_decode.argtypes = [C.c_uint8]
    return L


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(C.POINTER(t))


class Problem:
    """One oracle problem; keeps the numpy buffers it points into alive.

    ``seqs`` is a list of (T, Hg, Wg, n_audio); q, k, v are uint16 bf16 bits
    [N, H, d] or float64 values [N, H, d] (the fp64 outputs of a QKV
    projection, see ``project``); any token stride is taken from the array's
    first stride.  norm_w is float32 [2, H, d].
    """

    def __init__(self, H: int, d: int, seqs: Sequence, split, q, k, v, norm_w,
                 theta: float = 10000.0, eps: float = 1e-6, scale: Optional[float] = None,
                 rope: bool = True, library=None):
        self.L = library or lib()
        self.H, self.d = int(H), int(d)
        seqs = [tuple(int(x) for x in (s if not hasattr(s, "T") else (s.T, s.Hg, s.Wg, s.n_audio)))
                for s in seqs]
        self.seqs_py = seqs
        n = [s[0] * s[1] * s[2] + s[3] for s in seqs]
        self.cu = np.zeros(len(seqs) + 1, dtype=np.int32)
        self.cu[1:] = np.cumsum(n)
        self.N = int(self.cu[-1])
        self._seqs = (_Seq * max(1, len(seqs)))(*[_Seq(*s) for s in seqs])
        self.q, self.k, self.v = (self._prep(x) for x in (q, k, v))
        self.norm_w = np.ascontiguousarray(norm_w, dtype=np.float32)
        assert self.norm_w.shape == (2, self.H, self.d)
        self.scale = float(scale) if scale is not None else 1.0 / np.sqrt(self.d)
        pr = _Problem()
        pr.H, pr.d, pr.S, pr.rope = self.H, self.d, len(seqs), 1 if rope else 0
        pr.split[:] = list(split)
        pr.theta, pr.eps, pr.scale = float(theta), float(eps), self.scale
        pr.cu = _ptr(self.cu, C.c_int32)
        pr.seqs = self._seqs
        bits = [x if x.dtype == np.uint16 else None for x in (self.q, self.k, self.v)]
        vals = [x if x.dtype == np.float64 else None for x in (self.q, self.k, self.v)]
        pr.q, pr.k, pr.v = (_ptr(x, C.c_uint16) if x is not None else None for x in bits)
        pr.qf, pr.kf, pr.vf = (_ptr(x, C.c_double) if x is not None else None for x in vals)
        pr.q_stride, pr.k_stride, pr.v_stride = (x.strides[0] // x.itemsize for x in (self.q, self.k, self.v))
        pr.norm_w = _ptr(self.norm_w, C.c_float)
        self.pr = pr

    def _prep(self, x):
        x = np.asarray(x)
        assert x.dtype in (np.uint16, np.float64) and x.ndim == 3 and x.shape[1:] == (self.H, self.d)
        if x.strides[1] != self.d * x.itemsize or x.strides[2] != x.itemsize:
            x = np.ascontiguousarray(x)
        return x

    @classmethod
    def from_workload(cls, w, inputs, **kw):
        return cls(w.H, w.d, w.seqs, w.split, inputs["q"], inputs["k"], inputs["v"],
                   inputs["norm_w"], theta=w.theta, eps=w.eps, **kw)

    @classmethod
    def from_projection(cls, w, inputs, proj=None, round_v: bool = False, **kw):
        """The problem whose q, k, v are the fp64 QKV projection of the
        hidden states inputs["x"] by inputs["w_qkv"] (``project``); ``proj``
        may pass that projection in when it is already computed.  With
        ``round_v`` v is that projection rounded to bf16 (to nearest, ties to
        even): the quantised projection path stores v in bf16 before coding it
        in FP8, and its FP8 coding takes bf16 v like the quantised path's."""
        if proj is None:
            proj = project(inputs["x"], inputs["w_qkv"])
        hd = w.H * w.d
        assert proj.shape == (w.N, 3 * hd)
        q, k, v = (proj[:, i * hd:(i + 1) * hd].reshape(w.N, w.H, w.d) for i in range(3))
        if round_v:
            v = _bf16_bits_rne(v)
        return cls(w.H, w.d, w.seqs, w.split, q, k, v, inputs["norm_w"], theta=w.theta, eps=w.eps, **kw)

    # -- queries -----------------------------------------------------------
    def attention_rows(self, rows, nthreads: int = 0) -> np.ndarray:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.zeros((len(rows), self.d), dtype=np.float64)
        st = self.L.orc_attention_rows(C.byref(self.pr), _ptr(rows, C.c_int64), len(rows),
                                       _ptr(out, C.c_double), int(nthreads))
        if st != 0:
            raise ValueError("oracle: row outside every sequence")
        return out

    def prologue_rows(self, which: int, rows, nthreads: int = 0) -> np.ndarray:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.zeros((len(rows), self.d), dtype=np.float64)
        st = self.L.orc_prologue_rows(C.byref(self.pr), int(which), _ptr(rows, C.c_int64),
                                      len(rows), _ptr(out, C.c_double), int(nthreads))
        if st != 0:
            raise ValueError("oracle: row outside every sequence")
        return out

    # -- block-sparse attention (kept 64-key tiles per SPARSE_BLOCK-row query block) --
    def sparse_items(self):
        """(sequence, head, query block) work items in the order block-sparse
        tile lists are laid out: sequence-major, then head, then SPARSE_BLOCK-row
        block."""
        items = []
        for s in range(len(self.cu) - 1):
            n = int(self.cu[s + 1] - self.cu[s])
            for hh in range(self.H):
                for qb in range((n + SPARSE_BLOCK - 1) // SPARSE_BLOCK):
                    items.append((s, hh, qb))
        return items

    def sparse_attention_rows(self, rows, tiles, tiles_per_block: int, nthreads: int = 0) -> np.ndarray:
        """Attention of the rows (token * H + head) over only the keys of the
        64-key tiles kept for their SPARSE_BLOCK-row query block: tiles is int32
        [items, tiles_per_block] (items as sparse_items()); of an item's row
        the first min(tiles_per_block, ceil(n_s / 64)) entries are tile
        indices within the sequence, the rest are ignored.  The softmax runs
        over the kept keys only (exactly the plain definition restricted to
        them); a row with no kept key gets 0."""
        rows = np.asarray(rows, dtype=np.int64)
        tiles = np.asarray(tiles)
        items = self.sparse_items()
        index = {it: i for i, it in enumerate(items)}
        out = np.zeros((len(rows), self.d), dtype=np.float64)
        groups = {}
        for r_i, r in enumerate(rows.tolist()):
            tok, hh = divmod(r, self.H)
            s = int(np.searchsorted(self.cu, tok, side="right") - 1)
            qb = (tok - int(self.cu[s])) // SPARSE_BLOCK
            groups.setdefault((s, hh, qb), []).append(r_i)
        for (s, hh, qb), idx in groups.items():
            n = int(self.cu[s + 1] - self.cu[s])
            L = min(tiles_per_block, (n + 63) // 64)
            kept = sorted(set(int(t) for t in tiles[index[(s, hh, qb)], :L]))
            keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, n)) for t in kept]) + int(self.cu[s]) \
                if kept else np.zeros(0, dtype=np.int64)
            krows = keys.astype(np.int64) * self.H + hh
            qrows = rows[idx]
            if len(keys) == 0:
                continue
            khat = self.prologue_rows(1, krows, nthreads)
            vv = self.value_rows(krows)
            qhat = self.prologue_rows(0, qrows, nthreads)
            out[idx] = attention_core(qhat, khat, vv, self.scale, library=self.L)
        return out

    def value_rows(self, rows) -> np.ndarray:
        """v of the rows (token * H + head), fp64."""
        rows = np.asarray(rows, dtype=np.int64)
        tok, hh = rows // self.H, rows % self.H
        vv = self.v[tok, hh]
        return vv.astype(np.float64) if vv.dtype == np.float64 else _bf16_bits_to_f64(vv)

    def sparse_select(self, tiles_per_block: int) -> np.ndarray:
        """Top-k kept tiles per (sequence, head, SPARSE_BLOCK-row query block) by pooled
        score: qbar = mean of the block's qhat' rows (qhat * scale * log2 e),
        kbar_t = mean of tile t's khat rows, both from the values rounded to bf16
        as the attention path stores them, score_t = qbar . kbar_t (fp64).  The
        min(tiles_per_block, ceil(n_s / 64)) best tiles (ties to the lower index)
        in ascending order, the rest of the row -1.  Returns (tiles [items, k],
        scores: list of per-item fp64 score vectors) for checking a selection."""
        items = self.sparse_items()
        out = -np.ones((len(items), tiles_per_block), dtype=np.int32)
        scores = []
        mult = self.scale / np.log(2.0)
        cache = {}
        for i, (s, hh, qb) in enumerate(items):
            n = int(self.cu[s + 1] - self.cu[s])
            if (s, hh) not in cache:
                rr = (np.arange(n, dtype=np.int64) + int(self.cu[s])) * self.H + hh
                kh = _round_bf16(self.prologue_rows(1, rr))
                qh = _round_bf16(self.prologue_rows(0, rr) * mult)
                nt = (n + 63) // 64
                kbar = np.stack([kh[64 * t:64 * t + 64].mean(axis=0) for t in range(nt)])
                cache = {(s, hh): (qh, kbar)}
            qh, kbar = cache[(s, hh)]
            qbar = qh[SPARSE_BLOCK * qb:SPARSE_BLOCK * (qb + 1)].mean(axis=0)
            sc = kbar @ qbar
            L = min(tiles_per_block, len(sc))
            order = sorted(range(len(sc)), key=lambda t: (-sc[t], t))[:L]
            out[i, :L] = sorted(order)
            scores.append(sc)
        return out, scores

    def token_pos(self, token: int):
        s, a = C.c_int32(), C.c_int32()
        pos = (C.c_int32 * 3)()
        self.L.orc_token_pos(C.byref(self.pr), int(token), C.byref(s), C.byref(a), pos)
        return s.value, bool(a.value), tuple(pos)

    def rope_angles(self, is_audio: bool, pos) -> np.ndarray:
        p = (C.c_int32 * 3)(*[int(x) for x in (list(pos) + [0, 0, 0])[:3]])
        out = np.zeros(self.d // 2, dtype=np.float64)
        self.L.orc_rope_angles(C.byref(self.pr), 1 if is_audio else 0, p, _ptr(out, C.c_double))
        return out

    # -- quantised-path stages ---------------------------------------------
    def q8_kmean(self, nthreads: int = 0) -> np.ndarray:
        out = np.zeros((len(self.seqs_py), self.H, self.d), dtype=np.float64)
        self.L.orc_q8_kmean(C.byref(self.pr), _ptr(out, C.c_double), int(nthreads))
        return out

    def q8_block_quant(self, which: int, seq: int, head: int, block: int, kmean=None):
        rows_max = 64
        ratio = np.zeros((rows_max, self.d), dtype=np.float64)
        codes = np.zeros((rows_max, self.d), dtype=np.int8)
        scale = C.c_double()
        km = np.ascontiguousarray(kmean if kmean is not None else
                                  np.zeros((len(self.seqs_py), self.H, self.d)), dtype=np.float64)
        rows = self.L.orc_q8_block_quant(C.byref(self.pr), int(which), int(seq), int(head),
                                         int(block), _ptr(km, C.c_double), C.byref(scale),
                                         _ptr(ratio, C.c_double), _ptr(codes, C.c_int8))
        if rows < 0:
            raise ValueError("oracle: bad quantisation block")
        return scale.value, ratio[:rows], codes[:rows]

    def q8_attention_rows(self, rows, nthreads: int = 0, kmean=None) -> np.ndarray:
        """Output rows of the quantised path taken step by step (orc_q8_attention_rows)."""
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        km = np.ascontiguousarray(self.q8_kmean(nthreads) if kmean is None else kmean, dtype=np.float64)
        out = np.zeros((len(rows), self.d), dtype=np.float64)
        st = self.L.orc_q8_attention_rows(C.byref(self.pr), _ptr(rows, C.c_int64), len(rows),
                                          _ptr(km, C.c_double), _ptr(out, C.c_double), int(nthreads))
        if st != 0:
            raise ValueError("oracle: row outside every sequence")
        return out

    def q8_v_quant(self, seq: int, head: int):
        n = int(self.cu[seq + 1] - self.cu[seq])
        scale = np.zeros(self.d, dtype=np.float64)
        ratio = np.zeros((max(n, 1), self.d), dtype=np.float64)
        codes = np.zeros((max(n, 1), self.d), dtype=np.uint8)
        self.L.orc_q8_v_quant(C.byref(self.pr), int(seq), int(head), _ptr(scale, C.c_double),
                              _ptr(ratio, C.c_double), _ptr(codes, C.c_uint8))
        return scale, ratio[:n], codes[:n]

    # -- MXFP4 path stages --------------------------------------------------
    def mx_qk_quant(self, which: int, seq: int, head: int, kmean=None, nthreads: int = 0):
        """MXFP4 codes [n, d] (uint8, one code per byte) and scale exponents
        [n, d/32] of qhat (which 0) or khat - kmean (which 1) of one sequence
        and head (orc_mx_qk_quant)."""
        n = int(self.cu[seq + 1] - self.cu[seq])
        codes = np.zeros((max(n, 1), self.d), dtype=np.uint8)
        exps = np.zeros((max(n, 1), self.d // 32), dtype=np.int32)
        km = None
        if which == 1:
            km = np.ascontiguousarray(self.q8_kmean(nthreads) if kmean is None else kmean, dtype=np.float64)
        st = self.L.orc_mx_qk_quant(C.byref(self.pr), int(which), int(seq), int(head),
                                    _ptr(km, C.c_double) if km is not None else None,
                                    _ptr(codes, C.c_uint8), _ptr(exps, C.c_int32), int(nthreads))
        if st < 0:
            raise ValueError("oracle: bad MXFP4 quantisation request")
        return codes[:n], exps[:n]

    def mx_v_quant(self, seq: int, head: int):
        """MXFP4 codes [n, d] and scale exponents [ceil(n/32), d] of raw v of
        one sequence and head, blocks of 32 tokens (orc_mx_v_quant)."""
        n = int(self.cu[seq + 1] - self.cu[seq])
        nb = (n + 31) // 32
        codes = np.zeros((max(n, 1), self.d), dtype=np.uint8)
        exps = np.zeros((max(nb, 1), self.d), dtype=np.int32)
        st = self.L.orc_mx_v_quant(C.byref(self.pr), int(seq), int(head), _ptr(codes, C.c_uint8),
                                   _ptr(exps, C.c_int32))
        if st < 0:
            raise ValueError("oracle: bad MXFP4 quantisation request")
        return codes[:n], exps[:nb]

    def mx_attention_rows(self, rows, nthreads: int = 0, kmean=None) -> np.ndarray:
        """Output rows of the FP4 path taken step by step (orc_mx_attention_rows)."""
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        km = np.ascontiguousarray(self.q8_kmean(nthreads) if kmean is None else kmean, dtype=np.float64)
        out = np.zeros((len(rows), self.d), dtype=np.float64)
        st = self.L.orc_mx_attention_rows(C.byref(self.pr), _ptr(rows, C.c_int64), len(rows),
                                          _ptr(km, C.c_double), _ptr(out, C.c_double), int(nthreads))
        if st != 0:
            raise ValueError("oracle: row outside every sequence")
        return out


def mx_softmax_pv(x, vdec, library=None) -> np.ndarray:
    """The FP4 path's softmax and P.V for one row: log2-unit scores x [n],
    decoded V [n, d] (see orc_mx_softmax_pv)."""
    L = library or lib()
    x = np.ascontiguousarray(x, dtype=np.float64)
    vdec = np.ascontiguousarray(vdec, dtype=np.float64)
    n, d = vdec.shape
    out = np.zeros(d, dtype=np.float64)
    L.orc_mx_softmax_pv(_ptr(x, C.c_double), n, _ptr(vdec, C.c_double), d, _ptr(out, C.c_double))
    return out


def e2m1_encode(x: float, library=None) -> int:
    return int((library or lib()).orc_e2m1_encode(float(x)))


def e2m1_decode(c: int, library=None) -> float:
    return float((library or lib()).orc_e2m1_decode(int(c)))


def mx_scale_exp(amax: float, library=None) -> int:
    return int((library or lib()).orc_mx_scale_exp(float(amax)))


def mx_block(x, library=None):
    """(X, codes) of one MX block of values x (orc_mx_block)."""
    L = library or lib()
    x = np.ascontiguousarray(x, dtype=np.float64)
    codes = np.zeros(max(len(x), 1), dtype=np.uint8)
    X = L.orc_mx_block(_ptr(x, C.c_double), len(x), _ptr(codes, C.c_uint8))
    return int(X), codes[:len(x)]


def q8_softmax_pv(x, vdec, library=None) -> np.ndarray:
    """The quantised path's softmax and P.V for one row: log2-unit scores x [n],
    decoded V [n, d] (see orc_q8_softmax_pv)."""
    L = library or lib()
    x = np.ascontiguousarray(x, dtype=np.float64)
    vdec = np.ascontiguousarray(vdec, dtype=np.float64)
    n, d = vdec.shape
    out = np.zeros(d, dtype=np.float64)
    L.orc_q8_softmax_pv(_ptr(x, C.c_double), n, _ptr(vdec, C.c_double), d, _ptr(out, C.c_double))
    return out


def project(x_bits, w_bits, rows=None, chunk: int = 8192) -> np.ndarray:
    """QKV projection of hidden states: y[t, f] = sum_c x[t, c] * W[f, c].

    The attention layer's input projection that the page "H3 Runtime Current
    State" names ("attention QKV" under its tensor-parallel GEMMs) and that the
    GEMM share in question 4 of "Buyer Questions: Current Evidence Status"
    measures; the pages print no formula, so this is the textbook linear map
    without bias, W in the [out_features, in_features] layout with the q, k and
    v features in that order, each head-major.  x: uint16 bf16 bits [N, D];
    W: uint16 bf16 bits [F, D]; the result is fp64 [len(rows) or N, F].  Every
    product of two bf16 values is exact in fp64; the matrix product (numpy's,
    a library primitive) sums them in fp64.
    """
    x = np.asarray(x_bits)
    wt = np.asarray(w_bits)
    assert x.dtype == np.uint16 and wt.dtype == np.uint16 and x.shape[1] == wt.shape[1]
    wf = _bf16_bits_to_f64(wt).T.copy()
    idx = np.arange(x.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(idx), wt.shape[0]), dtype=np.float64)
    for i0 in range(0, len(idx), chunk):
        out[i0:i0 + chunk] = _bf16_bits_to_f64(x[idx[i0:i0 + chunk]]) @ wf
    return out


def out_proj(attn, w_o, cu_seqlens, gate=None, resid=None, rows=None, chunk: int = 8192) -> np.ndarray:
    """Output projection with the gated residual of a DiT-style block:
    y[t, c] = resid[t, c] + gate[s(t), c] * sum_k attn[t, k] * W_o[c, k].

    The page "Buyer Questions: Current Evidence Status" (question 4) counts the
    block's GEMMs and its "gates" apart from attention, and the page
    "Open-H3-Regenerate-2K" lists an adaLN table among the model files; the
    pages give no formula, so this is the plain reading: the bias-free linear
    map W_o ([D, H*d], nn.Linear layout) of the attention output, scaled per
    channel by the gate of the token's sequence and added to the residual.
    attn: uint16 bf16 bits or float64 [N, H*d]; w_o: uint16 bf16 bits [D, H*d];
    gate: float32 [S, D] (None: 1); resid: uint16 bf16 bits [N, D] (None: 0);
    cu_seqlens: [S+1].  Returns fp64 [len(rows) or N, D]; the matrix product
    (numpy's, a library step) sums exact products in fp64.
    """
    a = np.asarray(attn)
    w = _bf16_bits_to_f64(np.asarray(w_o)).T.copy()
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.arange(a.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    seq = np.searchsorted(cu, idx, side="right") - 1
    assert np.all((seq >= 0) & (seq < len(cu) - 1) & (idx < cu[-1])), "token outside every sequence"
    out = np.empty((len(idx), w.shape[1]), dtype=np.float64)
    for i0 in range(0, len(idx), chunk):
        sl = idx[i0:i0 + chunk]
        ai = a[sl]
        ai = _bf16_bits_to_f64(ai) if ai.dtype == np.uint16 else np.asarray(ai, dtype=np.float64)
        y = ai @ w
        if gate is not None:
            y *= np.asarray(gate, dtype=np.float64)[seq[i0:i0 + chunk]]
        if resid is not None:
            y += _bf16_bits_to_f64(np.asarray(resid)[sl])
        out[i0:i0 + chunk] = y
    return out


def _bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bits of fp64 values rounded to nearest, ties to even (via fp32)."""
    f = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((f + np.uint32(0x7FFF) + ((f >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to bf16 (to nearest, ties to even) and back, via fp32."""
    return _bf16_bits_to_f64(_bf16_bits_rne(x))


def _bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_core(qhat, khat, v, scale: float, library=None) -> np.ndarray:
    """Softmax attention of fp64 rows qhat [nq, d] over keys khat, v [nk, d]."""
    L = library or lib()
    qhat, khat, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (qhat, khat, v))
    nq, d = qhat.shape
    out = np.zeros((nq, d), dtype=np.float64)
    L.orc_attention_core(_ptr(qhat, C.c_double), nq, _ptr(khat, C.c_double),
                         _ptr(v, C.c_double), khat.shape[0], d, float(scale),
                         _ptr(out, C.c_double))
    return out


def rmsnorm(x_bf16, w, eps: float, library=None) -> np.ndarray:
    L = library or lib()
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    out = np.zeros(x.shape[-1], dtype=np.float64)
    L.orc_rmsnorm(_ptr(x, C.c_uint16), _ptr(w, C.c_float), x.shape[-1], float(eps),
                  _ptr(out, C.c_double))
    return out


def rope_rotate(x, phi, library=None) -> np.ndarray:
    L = library or lib()
    x = np.ascontiguousarray(x, dtype=np.float64)
    phi = np.ascontiguousarray(phi, dtype=np.float64)
    out = np.zeros_like(x)
    L.orc_rope_rotate(_ptr(x, C.c_double), _ptr(phi, C.c_double), x.shape[-1],
                      _ptr(out, C.c_double))
    return out


def e4m3_encode(x: float, library=None) -> int:
    return int((library or lib()).orc_e4m3_encode(float(x)))


def e4m3_decode(c: int, library=None) -> float:
    return float((library or lib()).orc_e4m3_decode(int(c)))


def default_threads(library=None) -> int:
    return int((library or lib()).orc_default_threads())
