"""Thin ctypes binding of libh3attn.so (include/h3attn.h), same names as the C ABI.

Argument marshalling only: tensors supply device pointers and the current
HIP stream; every step of the computation runs in the library's kernels.  The
library must have been built (``python -m audio_diffusion_transformer_amd.build``);
loading fails loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# H3ATTN_LIB points the binding at another build of the same sources (the
# tests use it for a build with host-side sanitizers).
LIB_PATH = os.environ.get("H3ATTN_LIB") or os.path.join(_HERE, "libh3attn.so")

H3ATTN_OK = 0
H3ATTN_ERR_INVALID_ARG = 1
H3ATTN_ERR_UNSUPPORTED = 2
H3ATTN_ERR_WORKSPACE = 3
H3ATTN_ERR_DEVICE = 4
H3ATTN_ERR_HIP = 5
H3ATTN_MAX_SEQS = 64
H3ATTN_VERSION = 2                 # the ABI version of include/h3attn.h this binding follows
H3ATTN_STATIC_WORKSPACE_BYTES = 128 << 20
SPARSE_BLOCK_ROWS = 256            # query rows per block-sparse tile list

EXPORTED = ("h3attn_workspace_size", "h3attn_fwd", "h3attn_fwd_stages", "h3attn_fwd_q8",
            "h3attn_fwd_q8_stages", "h3attn_prologue", "h3attn_fwd_proj", "h3attn_fwd_proj_stages",
            "h3attn_proj_prologue", "h3attn_fwd_proj_q8", "h3attn_fwd_proj_q8_stages", "h3attn_proj_q8_prologue",
            "h3attn_out_proj", "h3attn_fwd_sparse", "h3attn_fwd_sparse_stages",
            "h3attn_q8_prologue", "h3attn_fwd_mx", "h3attn_fwd_mx_stages", "h3attn_mx_prologue",
            "h3attn_fwd_static", "h3attn_mfma_ceiling", "h3attn_rope_fill_video", "h3attn_rope_fill_audio",
            "h3attn_checked", "h3attn_status_string", "h3attn_last_error", "h3attn_version")


class H3AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (status_string(status), msg))
        self.status = status


class h3attn_params(C.Structure):
    _fields_ = [("num_heads", C.c_int32), ("head_dim", C.c_int32), ("num_seqs", C.c_int32),
                ("flags", C.c_int32), ("q_stride", C.c_int64), ("k_stride", C.c_int64),
                ("v_stride", C.c_int64), ("o_stride", C.c_int64), ("eps", C.c_float),
                ("softmax_scale", C.c_float)]


_lib = None


def lib():
    """Load libh3attn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libh3attn.so is not built (%s); run "
                               "`python -m audio_diffusion_transformer_amd.build`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        P, vp = C.POINTER, C.c_void_p
        L.h3attn_workspace_size.restype = C.c_size_t
        L.h3attn_workspace_size.argtypes = [P(h3attn_params), P(C.c_int32), C.c_int]
        fwd_args = [P(h3attn_params), vp, vp, vp, vp, vp, P(C.c_int32), vp, vp, C.c_size_t, vp]
        for name in ("h3attn_fwd", "h3attn_fwd_q8", "h3attn_fwd_mx"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = fwd_args
        for name in ("h3attn_fwd_stages", "h3attn_fwd_q8_stages", "h3attn_fwd_mx_stages"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = fwd_args + [C.c_int]
        L.h3attn_checked.restype = C.c_int
        L.h3attn_checked.argtypes = [vp, C.c_int, C.c_uint32]
        L.h3attn_mfma_ceiling.restype = C.c_int
        L.h3attn_mfma_ceiling.argtypes = [C.c_int, C.c_int, C.c_int, vp, vp]
        L.h3attn_fwd_static.restype = C.c_int
        L.h3attn_fwd_static.argtypes = [P(h3attn_params), vp, vp, vp, vp, vp, P(C.c_int32), vp, vp]
        proj_args = [P(h3attn_params), C.c_int32, vp, C.c_int64, vp, vp, vp, P(C.c_int32), vp, vp,
                     C.c_size_t, vp]
        for name in ("h3attn_fwd_proj", "h3attn_fwd_proj_q8"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = proj_args
        for name in ("h3attn_fwd_proj_stages", "h3attn_fwd_proj_q8_stages"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = proj_args + [C.c_int]
        L.h3attn_proj_q8_prologue.restype = C.c_int
        L.h3attn_proj_q8_prologue.argtypes = [P(h3attn_params), C.c_int32, vp, C.c_int64, vp, vp, vp,
                                              P(C.c_int32), vp, C.c_size_t, vp, vp, vp, vp, vp, vp, vp, vp]
        L.h3attn_proj_prologue.restype = C.c_int
        L.h3attn_proj_prologue.argtypes = [P(h3attn_params), C.c_int32, vp, C.c_int64, vp, vp, vp,
                                           P(C.c_int32), vp, vp, vp, vp]
        sparse_args = [P(h3attn_params), vp, vp, vp, vp, vp, P(C.c_int32), C.c_int32, vp, vp, vp, C.c_size_t, vp]
        L.h3attn_fwd_sparse.restype = C.c_int
        L.h3attn_fwd_sparse.argtypes = sparse_args
        L.h3attn_fwd_sparse_stages.restype = C.c_int
        L.h3attn_fwd_sparse_stages.argtypes = sparse_args + [C.c_int]
        L.h3attn_out_proj.restype = C.c_int
        L.h3attn_out_proj.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, P(C.c_int32), vp, C.c_int64,
                                      vp, vp, vp, C.c_int64, vp, C.c_int64, vp]
        L.h3attn_prologue.restype = C.c_int
        L.h3attn_prologue.argtypes = [P(h3attn_params), vp, vp, vp, vp, P(C.c_int32), vp, vp, vp]
        L.h3attn_q8_prologue.restype = C.c_int
        L.h3attn_q8_prologue.argtypes = [P(h3attn_params), vp, vp, vp, vp, vp, P(C.c_int32), vp,
                                         C.c_size_t, vp, vp, vp, vp, vp, vp, vp, vp]
        L.h3attn_mx_prologue.restype = C.c_int
        L.h3attn_mx_prologue.argtypes = [P(h3attn_params), vp, vp, vp, vp, vp, P(C.c_int32), vp,
                                         C.c_size_t, vp, vp, vp, vp, vp, vp, vp, vp]
        L.h3attn_rope_fill_video.restype = C.c_int
        L.h3attn_rope_fill_video.argtypes = [C.c_int32] * 6 + [C.c_double, P(C.c_float)]
        L.h3attn_rope_fill_audio.restype = C.c_int
        L.h3attn_rope_fill_audio.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_double, P(C.c_float)]
        L.h3attn_status_string.restype = C.c_char_p
        L.h3attn_status_string.argtypes = [C.c_int]
        L.h3attn_last_error.restype = C.c_char_p
        L.h3attn_version.restype = C.c_int
        got = int(L.h3attn_version())
        if got != H3ATTN_VERSION:
            # the array layouts this binding allocates (tile lists, workspaces) are
            # those of its own ABI version; another build would read and write past them
            raise RuntimeError("%s reports ABI version %d; this binding is for version %d (rebuild with "
                               "`python -m audio_diffusion_transformer_amd.build`)" % (LIB_PATH, got, H3ATTN_VERSION))
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().h3attn_status_string(int(status)).decode()


def last_error() -> str:
    return lib().h3attn_last_error().decode()


def version() -> int:
    return int(lib().h3attn_version())


def _check(status: int):
    if status != H3ATTN_OK:
        raise H3AttnError(status, last_error())


def make_params(num_heads: int, head_dim: int, num_seqs: int, q_stride: int, k_stride: int,
                v_stride: int, o_stride: int, eps: float = 1e-6, softmax_scale: float = 0.0,
                flags: int = 0) -> h3attn_params:
    return h3attn_params(num_heads, head_dim, num_seqs, flags, q_stride, k_stride, v_stride,
                         o_stride, eps, softmax_scale)


def _cu_array(cu_seqlens) -> np.ndarray:
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(cu_seqlens, dtype=np.int32)


def _cu_ptr(cu: np.ndarray):
    return cu.ctypes.data_as(C.POINTER(C.c_int32))


def _mode(quantized) -> int:
    """False/0: bf16; True/1: INT8/FP8; 2: bf16 plus the sparse selection; "mx"/3: MXFP4;
    4: the projection's INT8/FP8 path (h3attn_fwd_proj_q8)."""
    if isinstance(quantized, str):
        if quantized != "mx":
            raise ValueError("quantized must be a bool, 0..4 or 'mx' (got %r)" % quantized)
        return 3
    return int(quantized)


def h3attn_workspace_size(params: h3attn_params, cu_seqlens, quantized=False) -> int:
    """Workspace bytes: quantized False/0 bf16, True/1 INT8/FP8, 2 bf16 plus the
    sparse selection, "mx"/3 MXFP4, 4 the projection's INT8/FP8 path."""
    cu = _cu_array(cu_seqlens)
    n = int(lib().h3attn_workspace_size(C.byref(params), _cu_ptr(cu), _mode(quantized)))
    if n == 0:
        raise H3AttnError(H3ATTN_ERR_INVALID_ARG, last_error())
    return n


# ---------------------------------------------------------------- raw calls

def fwd_raw(params, q, k, v, norm_w, rope_tables, cu_seqlens, out, workspace, workspace_bytes,
            stream, quantized=False, stages: int = 3) -> int:
    """Direct call with integer device pointers; returns the status code.
    ``quantized`` picks h3attn_fwd (False), h3attn_fwd_q8 (True) or
    h3attn_fwd_mx ("mx"); ``stages`` (1 prologue, 2 attention, 3 both) selects
    the matching *_stages entry point when it is not 3."""
    cu = _cu_array(cu_seqlens)
    args = (C.byref(params), q, k, v, norm_w, rope_tables, _cu_ptr(cu), out, workspace,
            workspace_bytes, stream)
    name = {0: "h3attn_fwd", 1: "h3attn_fwd_q8", 3: "h3attn_fwd_mx"}.get(_mode(quantized))
    if name is None:
        raise ValueError("quantized must be False, True or 'mx'")
    if stages != 3:
        return int(getattr(lib(), name + "_stages")(*args, int(stages)))
    return int(getattr(lib(), name)(*args))


# ------------------------------------------------------------ torch helpers

def _dev_ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _empty(stream, shape, dtype, device):
    """torch.empty on the launch stream: memory allocated while a stream is
    current belongs to that stream in torch's caching allocator, so a buffer
    the kernels on ``stream`` use is not handed to other streams' work before
    those kernels are done with it."""
    import torch
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def params_for(q, k, v, out, num_seqs: int, eps: float = 1e-6, softmax_scale: float = 0.0):
    """Params from [N, H, d] bf16 tensors (any token stride, unit channel stride)."""
    N, H, d = q.shape
    for t in (q, k, v, out):
        if t.dim() != 3 or t.shape[1:] != (H, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("q/k/v/out must be [N, H, d] with contiguous heads and channels")
    return make_params(H, d, num_seqs, q.stride(0), k.stride(0), v.stride(0), out.stride(0),
                       eps, softmax_scale)


def workspace_for(q, cu_seqlens, quantized: bool = False, eps: float = 1e-6):
    import torch
    N, H, d = q.shape
    cu = _cu_array(cu_seqlens)
    p = make_params(H, d, len(cu) - 1, H * d, H * d, H * d, H * d, eps)
    n = h3attn_workspace_size(p, cu, quantized)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def h3attn_fwd(q, k, v, norm_w, rope_tables, cu_seqlens, out=None, workspace=None,
               eps: float = 1e-6, softmax_scale: float = 0.0, stream=None, quantized: bool = False,
               stages: int = 3):
    """out[N, H, d] (bf16) = fused RMSNorm + RoPE + attention of bf16 q, k, v [N, H, d].

    norm_w: fp32 [2, H, d] on the device; rope_tables: fp32 [N, d/2, 2] on the
    device; cu_seqlens: int32 [S+1] (host array or CPU tensor)."""
    import torch
    if out is None:
        out = _empty(stream, q.shape, q.dtype, q.device)
    cu = _cu_array(cu_seqlens)
    params = params_for(q, k, v, out, len(cu) - 1, eps, softmax_scale)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, quantized),), torch.uint8, q.device)
    _check(fwd_raw(params, _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(norm_w),
                   _dev_ptr(rope_tables), cu, _dev_ptr(out), _dev_ptr(workspace),
                   workspace.numel() * workspace.element_size(), _stream_ptr(stream), quantized,
                   stages))
    return out


H3ATTN_CHECK_KINDS = 4


def checked(clear: bool = True, jitter_seed: int = 0) -> np.ndarray:
    """Checked build only (H3ATTN_LIB=.../libh3attn_checked.so): the attention
    kernels' invariant flag words (cleared after reading when ``clear``), and
    the timing-jitter seed for later launches (0: none).  Raises on the
    product library."""
    flags = np.zeros(H3ATTN_CHECK_KINDS, dtype=np.uint32)
    _check(lib().h3attn_checked(flags.ctypes.data, 1 if clear else 0, int(jitter_seed)))
    return flags


def mfma_ceiling_raw(mix: int, workgroups: int, iters: int, out, stream) -> int:
    """Direct call of h3attn_mfma_ceiling (device pointer `out`); returns the status."""
    return int(lib().h3attn_mfma_ceiling(int(mix), int(workgroups), int(iters), out, stream))


def static_raw(params, q, k, v, norm_w, rope_tables, cu_seqlens, out, stream) -> int:
    """Direct call of h3attn_fwd_static with integer device pointers; returns the status."""
    cu = _cu_array(cu_seqlens)
    return int(lib().h3attn_fwd_static(C.byref(params), q, k, v, norm_w, rope_tables, _cu_ptr(cu), out, stream))


def h3attn_fwd_static(q, k, v, norm_w, rope_tables, cu_seqlens, out, eps: float = 1e-6,
                      softmax_scale: float = 0.0, stream=None):
    """h3attn_fwd with the library's static device workspace (include/h3attn.h):
    allocates nothing, so ``out`` must be given."""
    cu = _cu_array(cu_seqlens)
    params = params_for(q, k, v, out, len(cu) - 1, eps, softmax_scale)
    _check(static_raw(params, _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(norm_w), _dev_ptr(rope_tables),
                      cu, _dev_ptr(out), _stream_ptr(stream)))
    return out


def h3attn_fwd_q8(q, k, v, norm_w, rope_tables, cu_seqlens, out=None, workspace=None,
                  eps: float = 1e-6, softmax_scale: float = 0.0, stream=None):
    return h3attn_fwd(q, k, v, norm_w, rope_tables, cu_seqlens, out, workspace, eps,
                      softmax_scale, stream, quantized=True)


def h3attn_fwd_mx(q, k, v, norm_w, rope_tables, cu_seqlens, out=None, workspace=None,
                  eps: float = 1e-6, softmax_scale: float = 0.0, stream=None, stages: int = 3):
    return h3attn_fwd(q, k, v, norm_w, rope_tables, cu_seqlens, out, workspace, eps,
                      softmax_scale, stream, quantized="mx", stages=stages)


def h3attn_prologue(q, k, norm_w, rope_tables, cu_seqlens, q_hat=None, k_hat=None,
                    eps: float = 1e-6, stream=None):
    import torch
    q_hat = _empty(stream, q.shape, torch.bfloat16, q.device) if q_hat is None else q_hat
    k_hat = _empty(stream, q.shape, torch.bfloat16, q.device) if k_hat is None else k_hat
    cu = _cu_array(cu_seqlens)
    params = params_for(q, k, q, q_hat, len(cu) - 1, eps)
    _check(lib().h3attn_prologue(C.byref(params), _dev_ptr(q), _dev_ptr(k), _dev_ptr(norm_w),
                                 _dev_ptr(rope_tables), _cu_ptr(cu), _dev_ptr(q_hat),
                                 _dev_ptr(k_hat), _stream_ptr(stream)))
    return q_hat, k_hat


def proj_raw(params, model_dim: int, x, x_stride: int, w_qkv, norm_w, rope_tables, cu_seqlens, out,
             workspace, workspace_bytes, stream, stages: int = 3, quantized: bool = False) -> int:
    """Direct call of h3attn_fwd_proj (h3attn_fwd_proj_q8 when ``quantized``;
    _stages when ``stages`` is not 3) with integer device pointers; returns
    the status code."""
    cu = _cu_array(cu_seqlens)
    args = (C.byref(params), int(model_dim), x, int(x_stride), w_qkv, norm_w, rope_tables, _cu_ptr(cu),
            out, workspace, workspace_bytes, stream)
    name = "h3attn_fwd_proj_q8" if quantized else "h3attn_fwd_proj"
    if stages != 3:
        return int(getattr(lib(), name + "_stages")(*args, int(stages)))
    return int(getattr(lib(), name)(*args))


def _proj_params(x, w_qkv, num_heads: int, head_dim: int, num_seqs: int, o_stride: int, eps, softmax_scale):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [N, D] with contiguous channels")
    hd = num_heads * head_dim
    if w_qkv.dim() != 2 or tuple(w_qkv.shape) != (3 * hd, x.shape[1]) or not w_qkv.is_contiguous():
        raise ValueError("w_qkv must be a contiguous [3*H*d, D] tensor")
    return make_params(num_heads, head_dim, num_seqs, hd, hd, hd, o_stride, eps, softmax_scale)


def h3attn_fwd_proj(x, w_qkv, norm_w, rope_tables, cu_seqlens, num_heads: int, head_dim: int, out=None,
                    workspace=None, eps: float = 1e-6, softmax_scale: float = 0.0, stream=None,
                    stages: int = 3, quantized: bool = False):
    """out[N, H, d] (bf16) = attention of the fused QKV projection of hidden
    states x [N, D] (bf16) by w_qkv [3*H*d, D] (bf16), with the RMSNorm + RoPE
    prologue (include/h3attn.h, h3attn_fwd_proj); with ``quantized`` the
    INT8/FP8 path with its prologue in the projection (h3attn_fwd_proj_q8)."""
    import torch
    N, D = x.shape
    if out is None:
        out = _empty(stream, (N, num_heads, head_dim), torch.bfloat16, x.device)
    cu = _cu_array(cu_seqlens)
    params = _proj_params(x, w_qkv, num_heads, head_dim, len(cu) - 1, out.stride(0), eps, softmax_scale)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, 4 if quantized else 0),), torch.uint8,
                           x.device)
    _check(proj_raw(params, D, _dev_ptr(x), x.stride(0), _dev_ptr(w_qkv), _dev_ptr(norm_w),
                    _dev_ptr(rope_tables), cu, _dev_ptr(out), _dev_ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream_ptr(stream), stages, quantized))
    return out


def h3attn_proj_prologue(x, w_qkv, norm_w, rope_tables, cu_seqlens, num_heads: int, head_dim: int,
                         eps: float = 1e-6, stream=None):
    """Stage 1 of h3attn_fwd_proj in natural layouts: (q_hat, k_hat, v), each bf16 [N, H, d]."""
    import torch
    N, D = x.shape
    cu = _cu_array(cu_seqlens)
    res = [_empty(stream, (N, num_heads, head_dim), torch.bfloat16, x.device) for _ in range(3)]
    params = _proj_params(x, w_qkv, num_heads, head_dim, len(cu) - 1, num_heads * head_dim, eps, 0.0)
    _check(lib().h3attn_proj_prologue(C.byref(params), D, _dev_ptr(x), x.stride(0), _dev_ptr(w_qkv),
                                      _dev_ptr(norm_w), _dev_ptr(rope_tables), _cu_ptr(cu),
                                      *[_dev_ptr(t) for t in res], _stream_ptr(stream)))
    return tuple(res)


def h3attn_proj_q8_prologue(x, w_qkv, norm_w, rope_tables, cu_seqlens, num_heads: int, head_dim: int,
                            workspace=None, eps: float = 1e-6, stream=None):
    """Stage 1 of h3attn_fwd_proj_q8 exported like h3attn_q8_prologue (see include/h3attn.h)."""
    import torch
    N, D = x.shape
    cu = _cu_array(cu_seqlens)
    S = len(cu) - 1
    H, d = num_heads, head_dim
    nblocks = int(sum((int(cu[s + 1] - cu[s]) + 63) // 64 for s in range(S)))
    params = _proj_params(x, w_qkv, H, d, S, H * d, eps, 0.0)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, 4),), torch.uint8, x.device)
    dev = x.device
    res = _q8_outputs(stream, N, H, d, S, nblocks, dev)
    _check(lib().h3attn_proj_q8_prologue(
        C.byref(params), D, _dev_ptr(x), x.stride(0), _dev_ptr(w_qkv), _dev_ptr(norm_w), _dev_ptr(rope_tables),
        _cu_ptr(cu), _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
        *[_dev_ptr(res[n]) for n in ("q8", "k8", "q_scale", "k_scale", "k_mean", "v8", "v_scale")],
        _stream_ptr(stream)))
    return res


def sparse_items(cu_seqlens, num_heads: int) -> int:
    """Rows of the block-sparse tile lists: sum over sequences of H * ceil(n_s / SPARSE_BLOCK_ROWS)."""
    cu = _cu_array(cu_seqlens)
    B = SPARSE_BLOCK_ROWS
    return int(sum(num_heads * ((int(cu[s + 1] - cu[s]) + B - 1) // B) for s in range(len(cu) - 1)))


def sparse_raw(params, q, k, v, norm_w, rope_tables, cu_seqlens, tiles_per_block: int, block_tiles, out,
               workspace, workspace_bytes, stream, stages: int = 7) -> int:
    """Direct call of h3attn_fwd_sparse_stages with integer device pointers; returns the status."""
    cu = _cu_array(cu_seqlens)
    return int(lib().h3attn_fwd_sparse_stages(C.byref(params), q, k, v, norm_w, rope_tables, _cu_ptr(cu),
                                              int(tiles_per_block), block_tiles, out, workspace, workspace_bytes,
                                              stream, int(stages)))


def h3attn_fwd_sparse(q, k, v, norm_w, rope_tables, cu_seqlens, tiles_per_block: int, block_tiles=None,
                      select: bool = True, out=None, workspace=None, eps: float = 1e-6, softmax_scale: float = 0.0,
                      stream=None):
    """Block-sparse attention (include/h3attn.h).  With select, the kept tiles
    are chosen by pooled score and written to block_tiles (allocated when
    None); otherwise block_tiles [items, tiles_per_block] (int32, device) is
    the caller's list.  Returns (out, block_tiles)."""
    import torch
    if out is None:
        out = _empty(stream, q.shape, q.dtype, q.device)
    cu = _cu_array(cu_seqlens)
    params = params_for(q, k, v, out, len(cu) - 1, eps, softmax_scale)
    N, H, d = q.shape
    if block_tiles is None:
        if not select:
            raise ValueError("block_tiles is needed when select is False")
        block_tiles = _empty(stream, (sparse_items(cu, H), tiles_per_block), torch.int32, q.device)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, 2 if select else 0),), torch.uint8, q.device)
    _check(sparse_raw(params, _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(norm_w), _dev_ptr(rope_tables), cu,
                      tiles_per_block, _dev_ptr(block_tiles), _dev_ptr(out), _dev_ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream_ptr(stream), 7 if select else 5))
    return out, block_tiles


def out_proj_raw(num_heads: int, head_dim: int, model_dim: int, cu_seqlens, attn, attn_stride: int, w_o, gate,
                 resid, resid_stride: int, out, out_stride: int, stream) -> int:
    """Direct call of h3attn_out_proj with integer device pointers (0 for NULL); returns the status."""
    cu = _cu_array(cu_seqlens)
    return int(lib().h3attn_out_proj(int(num_heads), int(head_dim), int(model_dim), len(cu) - 1, _cu_ptr(cu),
                                     attn, int(attn_stride), w_o, gate, resid, int(resid_stride), out,
                                     int(out_stride), stream))


def h3attn_out_proj(attn, w_o, cu_seqlens, gate=None, resid=None, out=None, stream=None):
    """out[N, D] (bf16) = resid + gate[seq] * (attn . w_o^T): attn [N, H, d] or [N, H*d] bf16,
    w_o [D, H*d] bf16, gate fp32 [S, D] or None, resid [N, D] bf16 or None; out may be resid."""
    import torch
    N = attn.shape[0]
    if attn.dim() == 3:
        H, d = attn.shape[1], attn.shape[2]
        if attn.stride(2) != 1 or attn.stride(1) != d:
            raise ValueError("attn must have contiguous heads and channels")
    else:
        raise ValueError("attn must be [N, H, d]")
    D = w_o.shape[0]
    if not w_o.is_contiguous() or w_o.shape[1] != H * d:
        raise ValueError("w_o must be a contiguous [D, H*d] tensor")
    if out is None:
        out = _empty(stream, (N, D), torch.bfloat16, attn.device)
    for t in (out, resid):
        if t is not None and (t.dim() != 2 or t.shape[1] != D or t.stride(1) != 1):
            raise ValueError("out / resid must be [N, D] with contiguous channels")
    cu = _cu_array(cu_seqlens)
    _check(out_proj_raw(H, d, D, cu, _dev_ptr(attn), attn.stride(0), _dev_ptr(w_o), _dev_ptr(gate),
                        _dev_ptr(resid), resid.stride(0) if resid is not None else 0, _dev_ptr(out),
                        out.stride(0), _stream_ptr(stream)))
    return out


def _q8_outputs(stream, N: int, H: int, d: int, S: int, nblocks: int, dev):
    import torch
    return {
        "q8": _empty(stream, (N, H, d), torch.int8, dev),
        "k8": _empty(stream, (N, H, d), torch.int8, dev),
        "q_scale": _empty(stream, (H, nblocks), torch.float32, dev),
        "k_scale": _empty(stream, (H, nblocks), torch.float32, dev),
        "k_mean": _empty(stream, (S, H, d), torch.float32, dev),
        "v8": _empty(stream, (N, H, d), torch.uint8, dev),
        "v_scale": _empty(stream, (S, H, d), torch.float32, dev),
    }


def h3attn_q8_prologue(q, k, v, norm_w, rope_tables, cu_seqlens, workspace=None,
                       eps: float = 1e-6, stream=None):
    """Quantised prologue exported in natural layouts (see include/h3attn.h)."""
    import torch
    N, H, d = q.shape
    cu = _cu_array(cu_seqlens)
    S = len(cu) - 1
    nblocks = int(sum((int(cu[s + 1] - cu[s]) + 63) // 64 for s in range(S)))
    params = params_for(q, k, v, q, S, eps)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, True),), torch.uint8, q.device)
    res = _q8_outputs(stream, N, H, d, S, nblocks, q.device)
    _check(lib().h3attn_q8_prologue(
        C.byref(params), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(norm_w),
        _dev_ptr(rope_tables), _cu_ptr(cu), _dev_ptr(workspace),
        workspace.numel() * workspace.element_size(),
        *[_dev_ptr(res[n]) for n in ("q8", "k8", "q_scale", "k_scale", "k_mean", "v8", "v_scale")],
        _stream_ptr(stream)))
    return res


def h3attn_mx_prologue(q, k, v, norm_w, rope_tables, cu_seqlens, workspace=None,
                       eps: float = 1e-6, stream=None):
    """FP4 prologue exported in natural layouts, one code per byte (see include/h3attn.h)."""
    import torch
    N, H, d = q.shape
    cu = _cu_array(cu_seqlens)
    S = len(cu) - 1
    nvb = int(sum((int(cu[s + 1] - cu[s]) + 31) // 32 for s in range(S)))
    params = params_for(q, k, v, q, S, eps)
    if workspace is None:
        workspace = _empty(stream, (h3attn_workspace_size(params, cu, "mx"),), torch.uint8, q.device)
    dev = q.device
    res = {
        "q_codes": _empty(stream, (N, H, d), torch.uint8, dev),
        "q_exp": _empty(stream, (N, H, d // 32), torch.uint8, dev),
        "k_codes": _empty(stream, (N, H, d), torch.uint8, dev),
        "k_exp": _empty(stream, (N, H, d // 32), torch.uint8, dev),
        "k_mean": _empty(stream, (S, H, d), torch.float32, dev),
        "v_codes": _empty(stream, (N, H, d), torch.uint8, dev),
        "v_exp": _empty(stream, (nvb, H, d), torch.uint8, dev),
    }
    _check(lib().h3attn_mx_prologue(
        C.byref(params), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(norm_w),
        _dev_ptr(rope_tables), _cu_ptr(cu), _dev_ptr(workspace),
        workspace.numel() * workspace.element_size(),
        *[_dev_ptr(res[n]) for n in ("q_codes", "q_exp", "k_codes", "k_exp", "k_mean", "v_codes", "v_exp")],
        _stream_ptr(stream)))
    return res


# ------------------------------------------------------------- RoPE tables

def h3attn_rope_fill_video(T: int, Hg: int, Wg: int, dt: int, dh: int, dw: int,
                           theta: float = 10000.0) -> np.ndarray:
    out = np.zeros((T * Hg * Wg, (dt + dh + dw) // 2, 2), dtype=np.float32)
    _check(lib().h3attn_rope_fill_video(T, Hg, Wg, dt, dh, dw, float(theta),
                                        out.ctypes.data_as(C.POINTER(C.c_float))))
    return out


def h3attn_rope_fill_audio(n: int, pos0: int, dim: int, theta: float = 10000.0) -> np.ndarray:
    out = np.zeros((n, dim // 2, 2), dtype=np.float32)
    _check(lib().h3attn_rope_fill_audio(n, pos0, dim, float(theta),
                                        out.ctypes.data_as(C.POINTER(C.c_float))))
    return out


def rope_table(seqs: Sequence, split, d: int, theta: float = 10000.0) -> np.ndarray:
    """Packed RoPE table [N, d/2, 2] for sequences given as (T, Hg, Wg, n_audio):
    each sequence's video grid rows followed by its audio rows (positions from 0)."""
    parts = []
    for s in seqs:
        T, Hg, Wg, na = (s.T, s.Hg, s.Wg, s.n_audio) if hasattr(s, "T") else tuple(s)
        if T * Hg * Wg > 0:
            parts.append(h3attn_rope_fill_video(T, Hg, Wg, *split, theta=theta))
        if na > 0:
            parts.append(h3attn_rope_fill_audio(na, 0, d, theta=theta))
    if not parts:
        return np.zeros((0, d // 2, 2), dtype=np.float32)
    return np.ascontiguousarray(np.concatenate(parts, axis=0))
