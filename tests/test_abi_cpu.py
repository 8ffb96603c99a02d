"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every function include/h3attn.h declares;
every argument error must be reported, with a message, before any HIP call;
the host RoPE table helpers must agree with the oracle's independently
computed fp64 angles.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3attn_\w+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = h.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), "libh3attn.so does not export %s" % n
    assert set(names) == set(h.EXPORTED)
    assert h.version() == h.H3ATTN_VERSION == 2


def test_status_strings():
    for code, name in [(0, "H3ATTN_OK"), (1, "H3ATTN_ERR_INVALID_ARG"), (2, "H3ATTN_ERR_UNSUPPORTED"),
                       (3, "H3ATTN_ERR_WORKSPACE"), (4, "H3ATTN_ERR_DEVICE"), (5, "H3ATTN_ERR_HIP")]:
        assert h.status_string(code) == name


FAKE = 1 << 20          # aligned fake device address; never dereferenced on a failing path


def _params(**kw):
    base = dict(num_heads=24, head_dim=128, num_seqs=1, q_stride=3072, k_stride=3072,
                v_stride=3072, o_stride=3072, eps=1e-6, softmax_scale=0.0, flags=0)
    base.update(kw)
    return h.make_params(**base)


def _call(params=None, cu=(0, 1000), ws_bytes=1 << 40, ptrs=None, quantized=False, stages=3):
    params = params if params is not None else _params()
    p = dict(q=FAKE, k=FAKE, v=FAKE, norm_w=FAKE, rope=FAKE, out=FAKE, ws=FAKE * 256)
    p.update(ptrs or {})
    return h.fwd_raw(params, p["q"], p["k"], p["v"], p["norm_w"], p["rope"], np.array(cu, np.int32),
                     p["out"], p["ws"], ws_bytes, None, quantized, stages)


@pytest.mark.parametrize("kw,msg", [
    (dict(num_heads=0), "num_heads"),
    (dict(head_dim=96), "head_dim"),
    (dict(num_seqs=0), "num_seqs"),
    (dict(num_seqs=65), "num_seqs"),
    (dict(flags=1), "flags"),
    (dict(q_stride=3064), "q_stride"),
    (dict(k_stride=3073), "k_stride"),
    (dict(v_stride=100), "v_stride"),
    (dict(o_stride=3076), "o_stride"),
    (dict(eps=0.0), "eps"),
    (dict(eps=float("nan")), "eps"),
    (dict(softmax_scale=float("inf")), "softmax_scale"),
])
def test_invalid_params_rejected_before_any_hip_call(kw, msg):
    st = _call(_params(**kw))
    assert st in (h.H3ATTN_ERR_INVALID_ARG, h.H3ATTN_ERR_UNSUPPORTED)
    assert msg in h.last_error()


@pytest.mark.parametrize("cu,msg", [((1, 10), "cu_seqlens[0]"), ((0, 10, 5), "decreases")])
def test_invalid_cu_seqlens(cu, msg):
    st = _call(_params(num_seqs=len(cu) - 1), cu=cu)
    assert st == h.H3ATTN_ERR_INVALID_ARG and msg in h.last_error()


@pytest.mark.parametrize("name", ["q", "k", "v", "norm_w", "rope", "out"])
def test_null_and_misaligned_pointers(name):
    assert _call(ptrs={name: 0}) == h.H3ATTN_ERR_INVALID_ARG
    assert "NULL" in h.last_error()
    assert _call(ptrs={name: FAKE + 8}) == h.H3ATTN_ERR_INVALID_ARG
    assert "aligned" in h.last_error()


def test_workspace_errors():
    need = h.h3attn_workspace_size(_params(), [0, 1000])
    assert _call(ws_bytes=need - 1) == h.H3ATTN_ERR_WORKSPACE and "needs" in h.last_error()
    assert _call(ptrs={"ws": 0}) == h.H3ATTN_ERR_WORKSPACE
    assert _call(ptrs={"ws": FAKE * 256 + 128}) == h.H3ATTN_ERR_WORKSPACE
    assert _call(stages=0) == h.H3ATTN_ERR_INVALID_ARG and "stages" in h.last_error()
    assert _call(stages=4) == h.H3ATTN_ERR_INVALID_ARG


def test_workspace_size_layout():
    # three head-major bf16 copies and one fp32 key-norm per 64-token tile and
    # head; every sequence padded to 256 tokens, every region to 256 bytes
    p = _params()
    cu = [0, 18144, 63394, 70594]
    got = h.h3attn_workspace_size(_params(num_seqs=3), cu)
    npad = sum(-(-(cu[i + 1] - cu[i]) // 256) * 256 for i in range(3))
    assert got == 3 * 24 * npad * 128 * 2 + -(-(24 * (npad // 64) * 4) // 256) * 256
    assert h.h3attn_workspace_size(p, [0, 0]) == 256     # empty input is valid; 0 means error
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(_params(head_dim=80), [0, 10])
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(_params(head_dim=64, num_heads=2, q_stride=128, k_stride=128,
                                        v_stride=128, o_stride=128), [0, 10], quantized=True)


@pytest.mark.parametrize("d", [64, 128])
def test_sequence_longer_than_the_descriptor_range(d):
    """One (sequence, head) slice of the bf16 K/V copies must stay below 2 GiB:
    the kernels' buffer descriptors take 32-bit sizes and offsets."""
    hd = 24 * d
    p = _params(head_dim=d, q_stride=hd, k_stride=hd, v_stride=hd, o_stride=hd)
    limit = (2 ** 31 // (2 * d)) // 64 * 64 - 64
    assert (limit + 64) * d * 2 <= 2 ** 31
    p2 = _params(head_dim=d, num_seqs=2, q_stride=hd, k_stride=hd, v_stride=hd, o_stride=hd)
    for cu in ([0, limit + 1], [0, 5, limit + 6]):
        prm = p if len(cu) == 2 else p2
        assert _call(prm, cu=cu) == h.H3ATTN_ERR_UNSUPPORTED
        assert "at most %d" % limit in h.last_error()
        with pytest.raises(h.H3AttnError):
            h.h3attn_workspace_size(prm, cu)
    assert h.h3attn_workspace_size(p, [0, limit]) > 3 * 24 * limit * d * 2


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device error path; a GPU is present")
def test_valid_call_without_gpu_reports_device_error():
    assert _call() == h.H3ATTN_ERR_DEVICE
    assert "device" in h.last_error().lower()


def test_error_message_is_thread_local():
    import threading
    _call(_params(num_heads=0))
    msgs = []

    def other():
        msgs.append(h.last_error())
        _call(_params(head_dim=3))
        msgs.append(h.last_error())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert msgs[0] == "" and "head_dim" in msgs[1]
    assert "num_heads" in h.last_error()


# ----------------------------------------------------------- RoPE tables

def _oracle_angles(seqs, split, d):
    N = sum(s[0] * s[1] * s[2] + s[3] for s in seqs)
    z = np.zeros((N, 1, d), np.uint16)
    p = oracle.Problem(1, d, seqs, split, z, z, z, np.ones((2, 1, d), np.float32))
    out = np.zeros((N, d // 2))
    for t in range(N):
        _, aud, pos = p.token_pos(t)
        out[t] = p.rope_angles(aud, pos)
    return out


@pytest.mark.parametrize("seqs,split,d", [
    ([(4, 8, 8, 0)], (16, 24, 24), 64),
    ([(3, 7, 9, 250), (2, 5, 5, 0), (0, 1, 1, 4)], (32, 48, 48), 128),
    # unit grid extents (each section is filled once per coordinate and copied)
    ([(2, 1, 5, 0), (3, 4, 1, 2), (1, 1, 1, 0), (5, 1, 1, 3)], (32, 48, 48), 128),
])
def test_rope_tables_match_oracle_angles(seqs, split, d):
    tab = h.rope_table(seqs, split, d)
    phi = _oracle_angles(seqs, split, d)
    assert tab.shape == (phi.shape[0], d // 2, 2) and tab.dtype == np.float32
    np.testing.assert_allclose(tab[..., 0], np.cos(phi), atol=1e-7, rtol=0)
    np.testing.assert_allclose(tab[..., 1], np.sin(phi), atol=1e-7, rtol=0)


def test_rope_fill_argument_errors():
    out = (ctypes.c_float * 64)()
    L = h.lib()
    assert L.h3attn_rope_fill_video(1, 1, 1, 3, 2, 2, 1e4, out) == h.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_fill_video(1, 0, 1, 2, 2, 2, 1e4, out) == h.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_fill_video(1, 1, 1, 2, 2, 2, 0.5, out) == h.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_fill_audio(2, -1, 8, 1e4, out) == h.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_fill_audio(2, 0, 7, 1e4, out) == h.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_fill_audio(2, 0, 8, 1e4, None) == h.H3ATTN_ERR_INVALID_ARG


def test_synth_is_seeded_and_bf16_rounding_is_nearest_even():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.generate(w), synth.generate(w)
    for key in ("q", "k", "v", "norm_w"):
        np.testing.assert_array_equal(a[key], b[key])
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.5], np.float32)   # ties -> even
    np.testing.assert_array_equal(synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(x)),
                                  [1.0, 1.0 + 2 ** -6, -1.5])
    rows = synth.sample_rows(synth.WORKLOADS["ragged"], 4096)
    assert len(rows) == 4096 and len(np.unique(rows)) == 4096
    H = 24
    toks = set((rows // H).tolist())
    for t in (0, 18143, 18144, 18144 + 45000, 63393, 63394, 70593):
        assert t in toks


def test_quantised_path_argument_errors():
    small = _params(num_heads=2, head_dim=64, q_stride=128, k_stride=128, v_stride=128, o_stride=128)
    assert _call(small, quantized=True) == h.H3ATTN_ERR_UNSUPPORTED
    assert "head_dim 128" in h.last_error()
    need = h.h3attn_workspace_size(_params(), [0, 1000], quantized=True)
    assert need < h.h3attn_workspace_size(_params(), [0, 1000])
    assert _call(ws_bytes=need - 1, quantized=True) == h.H3ATTN_ERR_WORKSPACE
    assert _call(quantized=True, stages=5) == h.H3ATTN_ERR_INVALID_ARG
    assert _call(ptrs={"v": 0}, quantized=True) == h.H3ATTN_ERR_INVALID_ARG


def test_fp4_path_argument_errors():
    small = _params(num_heads=2, head_dim=64, q_stride=128, k_stride=128, v_stride=128, o_stride=128)
    assert _call(small, quantized="mx") == h.H3ATTN_ERR_UNSUPPORTED
    assert "head_dim 128" in h.last_error()
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(small, [0, 1000], quantized="mx")
    need = h.h3attn_workspace_size(_params(), [0, 1000], quantized="mx")
    # FP4 codes (d/2 bytes per row of q, k and v) and scale bytes are smaller than the INT8/FP8 copies
    assert need < h.h3attn_workspace_size(_params(), [0, 1000], quantized=True)
    assert need == h.h3attn_workspace_size(_params(), [0, 1000], quantized=3)
    assert _call(ws_bytes=need - 1, quantized="mx") == h.H3ATTN_ERR_WORKSPACE
    assert _call(ptrs={"ws": FAKE * 256 + 16}, quantized="mx") == h.H3ATTN_ERR_WORKSPACE
    assert _call(quantized="mx", stages=0) == h.H3ATTN_ERR_INVALID_ARG
    assert _call(quantized="mx", stages=4) == h.H3ATTN_ERR_INVALID_ARG
    assert _call(ptrs={"k": 0}, quantized="mx") == h.H3ATTN_ERR_INVALID_ARG
    assert _call(ptrs={"out": FAKE + 2}, quantized="mx") == h.H3ATTN_ERR_INVALID_ARG
    # empty input: nothing read, written or launched
    assert _call(cu=(0, 0), ptrs={"q": 0, "k": 0, "v": 0, "out": 0, "ws": 0}, quantized="mx") == h.H3ATTN_OK
    # a valid call reaches the device check (only where no GPU is present)
    if not _gpu_present():
        assert _call(quantized="mx") == h.H3ATTN_ERR_DEVICE
    with pytest.raises(ValueError):
        h.fwd_raw(_params(), FAKE, FAKE, FAKE, FAKE, FAKE, np.array([0, 10], np.int32), FAKE, FAKE * 256,
                  1 << 40, None, "fp4")


def test_fp4_prologue_export_errors():
    import ctypes as C
    L = h.lib()
    cu = np.array([0, 1000], np.int32)
    outs = [FAKE] * 7
    args = lambda o: (C.byref(_params()), FAKE, FAKE, FAKE, FAKE, FAKE, cu.ctypes.data_as(C.POINTER(C.c_int32)),
                      FAKE * 256, 1 << 40, *o, None)
    names = ("q_codes", "q_exp", "k_codes", "k_exp", "k_mean", "v_codes", "v_exp")
    for i in range(7):      # every output is checked before any device call
        o = list(outs)
        o[i] = 0
        assert L.h3attn_mx_prologue(*args(o)) == h.H3ATTN_ERR_INVALID_ARG
        assert names[i] in h.last_error() and "NULL" in h.last_error()


def _proj_call(params=None, model_dim=3072, x_stride=3072, cu=(0, 1000), ws_bytes=1 << 40, ptrs=None,
               stages=3, quantized=False):
    params = params if params is not None else _params()
    p = dict(x=FAKE, w=FAKE, norm_w=FAKE, rope=FAKE, out=FAKE, ws=FAKE * 256)
    p.update(ptrs or {})
    return h.proj_raw(params, model_dim, p["x"], x_stride, p["w"], p["norm_w"], p["rope"], np.array(cu, np.int32),
                      p["out"], p["ws"], ws_bytes, None, stages, quantized)


@pytest.mark.parametrize("kw,msg,code", [
    (dict(model_dim=0), "model_dim", h.H3ATTN_ERR_INVALID_ARG),
    (dict(model_dim=3000), "model_dim", h.H3ATTN_ERR_INVALID_ARG),
    (dict(x_stride=3064), "x_stride", h.H3ATTN_ERR_INVALID_ARG),
    (dict(x_stride=3076), "x_stride", h.H3ATTN_ERR_INVALID_ARG),
    (dict(x_stride=1 << 23), "x_stride", h.H3ATTN_ERR_UNSUPPORTED),
    (dict(model_dim=1 << 23, x_stride=1 << 23), "too large", h.H3ATTN_ERR_UNSUPPORTED),
    (dict(stages=0), "stages", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"x": 0}), "NULL", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"w": FAKE + 4}), "aligned", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"ws": 0}), "workspace", h.H3ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=4096), "needs", h.H3ATTN_ERR_WORKSPACE),
    (dict(params=_params(num_heads=0)), "num_heads", h.H3ATTN_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("quantized", [False, True])
def test_projection_argument_errors(kw, msg, code, quantized):
    assert _proj_call(quantized=quantized, **kw) == code
    assert msg in h.last_error()


@pytest.mark.parametrize("quantized", [False, True])
def test_projection_ignores_qkv_strides_and_accepts_empty_input(quantized):
    # the q/k/v strides of the params are not read by the projection entry points
    p = _params(q_stride=8, k_stride=8, v_stride=8)
    assert _proj_call(p, cu=(0, 0), quantized=quantized) == h.H3ATTN_OK
    assert _proj_call(p, cu=(0, 0), ptrs={"x": 0, "w": 0}, quantized=quantized) == h.H3ATTN_OK


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device error path; a GPU is present")
@pytest.mark.parametrize("quantized", [False, True])
def test_projection_valid_call_without_gpu_reports_device_error(quantized):
    assert _proj_call(quantized=quantized) == h.H3ATTN_ERR_DEVICE


def test_quantised_projection_workspace_and_head_dim():
    """h3attn_fwd_proj_q8 takes workspace mode 4: the INT8/FP8 regions plus
    fp32 khat and bf16 v of every padded token; head_dim 128 only."""
    p = _params()
    q8 = h.h3attn_workspace_size(p, [0, 1000], True)
    q8p = h.h3attn_workspace_size(p, [0, 1000], 4)
    assert q8p - q8 >= 24 * 1024 * 128 * (4 + 2)
    assert _proj_call(ws_bytes=q8, quantized=True) == h.H3ATTN_ERR_WORKSPACE and "needs" in h.last_error()
    p64 = _params(head_dim=64, q_stride=1536, k_stride=1536, v_stride=1536, o_stride=1536)
    assert _proj_call(p64, quantized=True) == h.H3ATTN_ERR_UNSUPPORTED and "head_dim 128" in h.last_error()
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(p64, [0, 1000], 4)
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(p, [0, 1000], 5)


def test_quantised_projection_prologue_export_errors():
    import ctypes as C
    L = h.lib()
    cu = np.array([0, 1000], np.int32)
    outs = [FAKE] * 7
    args = lambda o: (C.byref(_params()), 3072, FAKE, 3072, FAKE, FAKE, FAKE, cu.ctypes.data_as(C.POINTER(C.c_int32)),
                      FAKE * 256, 1 << 40, *o, None)
    names = ("q8", "k8", "q_scale", "k_scale", "k_mean", "v8", "v_scale")
    for i in range(7):      # every output is checked before any device call
        o = list(outs)
        o[i] = 0
        assert L.h3attn_proj_q8_prologue(*args(o)) == h.H3ATTN_ERR_INVALID_ARG
        assert names[i] in h.last_error() and "NULL" in h.last_error()


def _out_call(H=24, d=128, D=3072, cu=(0, 1000), attn_stride=3072, resid_stride=3072, out_stride=3072,
              ptrs=None):
    p = dict(attn=FAKE, w=FAKE, gate=FAKE, resid=FAKE * 4, out=FAKE * 64)
    p.update(ptrs or {})
    return h.out_proj_raw(H, d, D, np.array(cu, np.int32), p["attn"], attn_stride, p["w"], p["gate"], p["resid"],
                          resid_stride, p["out"], out_stride, None)


@pytest.mark.parametrize("kw,msg,code", [
    (dict(H=0), "num_heads", h.H3ATTN_ERR_INVALID_ARG),
    (dict(d=96), "head_dim", h.H3ATTN_ERR_UNSUPPORTED),
    (dict(D=3000), "model_dim", h.H3ATTN_ERR_INVALID_ARG),
    (dict(D=64), "model_dim", h.H3ATTN_ERR_INVALID_ARG),
    (dict(cu=(1, 10)), "cu_seqlens[0]", h.H3ATTN_ERR_INVALID_ARG),
    (dict(cu=(0, 10, 5)), "decreases", h.H3ATTN_ERR_INVALID_ARG),
    (dict(attn_stride=3064), "attn_stride", h.H3ATTN_ERR_INVALID_ARG),
    (dict(out_stride=3076), "out_stride", h.H3ATTN_ERR_INVALID_ARG),
    (dict(resid_stride=8), "resid_stride", h.H3ATTN_ERR_INVALID_ARG),
    (dict(attn_stride=1 << 23), "attn_stride", h.H3ATTN_ERR_UNSUPPORTED),
    (dict(ptrs={"w": 0}), "NULL", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"attn": FAKE + 2}), "aligned", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"gate": FAKE + 4}), "aligned", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"out": FAKE * 4 + 1024}), "overlaps", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"out": FAKE * 4}, out_stride=3080), "stride", h.H3ATTN_ERR_INVALID_ARG),
])
def test_out_proj_argument_errors(kw, msg, code):
    assert _out_call(**kw) == code
    assert msg in h.last_error()


def test_out_proj_empty_input_and_null_gate_residual():
    assert _out_call(cu=(0, 0), ptrs={"attn": 0, "w": 0, "out": 0}) == h.H3ATTN_OK
    if not _gpu_present():
        assert _out_call(ptrs={"gate": 0, "resid": 0}) == h.H3ATTN_ERR_DEVICE   # valid up to the device check


def _sparse_call(params=None, cu=(0, 1000), tpb=4, ws_bytes=1 << 40, ptrs=None, stages=7):
    params = params if params is not None else _params()
    p = dict(q=FAKE, k=FAKE, v=FAKE, norm_w=FAKE, rope=FAKE, out=FAKE, ws=FAKE * 256, tiles=FAKE * 8)
    p.update(ptrs or {})
    return h.sparse_raw(params, p["q"], p["k"], p["v"], p["norm_w"], p["rope"], np.array(cu, np.int32), tpb,
                        p["tiles"], p["out"], p["ws"], ws_bytes, None, stages)


@pytest.mark.parametrize("kw,msg,code", [
    (dict(tpb=0), "tiles_per_block", h.H3ATTN_ERR_INVALID_ARG),
    (dict(tpb=2049), "tiles_per_block", h.H3ATTN_ERR_INVALID_ARG),
    (dict(cu=(0, 131073)), "at most", h.H3ATTN_ERR_UNSUPPORTED),
    (dict(stages=0), "stages", h.H3ATTN_ERR_INVALID_ARG),
    (dict(stages=8), "stages", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"tiles": 0}), "block_tiles", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"tiles": FAKE + 2}), "aligned", h.H3ATTN_ERR_INVALID_ARG),
    (dict(ptrs={"ws": 0}), "workspace", h.H3ATTN_ERR_WORKSPACE),
    (dict(ptrs={"q": 0}), "NULL", h.H3ATTN_ERR_INVALID_ARG),
])
def test_sparse_argument_errors(kw, msg, code):
    assert _sparse_call(**kw) == code
    assert msg in h.last_error()


def test_sparse_workspace_sizes():
    p = _params()
    dense = h.h3attn_workspace_size(p, [0, 1000])
    with_select = h.h3attn_workspace_size(p, [0, 1000], 2)
    npad, tiles = 1024, 16
    assert with_select - dense >= 2 * 24 * tiles * 128 * 4 + tiles * 4     # pooled k means, q sums, counts
    # the selection stage needs the larger workspace, the others the bf16 one
    assert _sparse_call(ws_bytes=dense, stages=2) == h.H3ATTN_ERR_WORKSPACE and "needs" in h.last_error()
    if not _gpu_present():
        assert _sparse_call(ws_bytes=dense, stages=5) == h.H3ATTN_ERR_DEVICE
    assert h.sparse_items([0, 1000, 1000, 1129], 24) == 24 * 4 + 24 * 1     # 256-row blocks
    assert h.SPARSE_BLOCK_ROWS == oracle.SPARSE_BLOCK
    with pytest.raises(h.H3AttnError):
        h.h3attn_workspace_size(p, [0, 1000], 5)


def test_injected_launch_failure_reports_hip_error(monkeypatch):
    """H3ATTN_FAULT=launch: a call that passes its argument checks makes no
    HIP call and reports its first launch as failed, with a message naming
    it; argument errors still come first, and the binding raises."""
    monkeypatch.setenv("H3ATTN_FAULT", "launch")
    cases = [
        (lambda: _call(), "prologue launch"),
        (lambda: _call(stages=2), "attention launch"),
        (lambda: _call(quantized=True), "quantised prologue launch"),
        (lambda: _call(quantized=True, stages=2), "quantised attention launch"),
        (lambda: _call(quantized="mx"), "FP4 prologue launch"),
        (lambda: _call(quantized="mx", stages=2), "FP4 attention launch"),
        (lambda: _proj_call(), "projection launch"),
        (lambda: _proj_call(quantized=True), "projection launch"),
        (lambda: _proj_call(quantized=True, stages=2), "quantised attention launch"),
        (lambda: _out_call(), "output projection launch"),
        (lambda: _sparse_call(), "prologue launch"),
        (lambda: _sparse_call(stages=4), "sparse attention launch"),
    ]
    for fn, what in cases:
        assert fn() == h.H3ATTN_ERR_HIP, what
        msg = h.last_error()
        assert msg.startswith(what) and "injected" in msg, msg
    assert _call(_params(num_heads=0)) == h.H3ATTN_ERR_INVALID_ARG
    assert _call(cu=(0, 0), ptrs={"q": 0, "k": 0, "v": 0, "out": 0, "ws": 0}) == h.H3ATTN_OK   # nothing to launch
    with pytest.raises(h.H3AttnError, match="injected") as err:
        h._check(_call())
    assert err.value.status == h.H3ATTN_ERR_HIP
    monkeypatch.setenv("H3ATTN_FAULT", "")
    if not _gpu_present():
        assert _call() == h.H3ATTN_ERR_DEVICE     # switched off again: back to the device check


def _static_call(params=None, cu=(0, 1000), ptrs=None):
    params = params if params is not None else _params()
    p = dict(q=FAKE, k=FAKE, v=FAKE, norm_w=FAKE, rope=FAKE, out=FAKE)
    p.update(ptrs or {})
    return h.static_raw(params, p["q"], p["k"], p["v"], p["norm_w"], p["rope"], np.array(cu, np.int32), p["out"],
                        None)


def test_static_workspace_entry_point_limits():
    """h3attn_fwd_static takes shapes whose bf16 workspace fits the static
    array and rejects larger ones, before any HIP call; argument errors are
    those of h3attn_fwd."""
    cap = h.H3ATTN_STATIC_WORKSPACE_BYTES
    assert h.h3attn_workspace_size(_params(), [0, 7168]) <= cap < h.h3attn_workspace_size(_params(), [0, 7169])
    assert _static_call(cu=(0, 7169)) == h.H3ATTN_ERR_WORKSPACE
    assert "static workspace holds %d" % cap in h.last_error()
    p3 = _params(num_heads=3, q_stride=384, k_stride=384, v_stride=384, o_stride=384)
    assert _static_call(p3, cu=(0, 58113)) == h.H3ATTN_ERR_WORKSPACE
    assert _static_call(_params(num_heads=0)) == h.H3ATTN_ERR_INVALID_ARG
    assert _static_call(ptrs={"out": 0}) == h.H3ATTN_ERR_INVALID_ARG and "out" in h.last_error()
    assert _static_call(cu=(0, 0), ptrs={"q": 0, "k": 0, "v": 0, "out": 0}) == h.H3ATTN_OK
    if not _gpu_present():
        assert _static_call(cu=(0, 7168)) == h.H3ATTN_ERR_DEVICE
        assert _static_call(p3, cu=(0, 58112)) == h.H3ATTN_ERR_DEVICE


def test_static_workspace_entry_point_injected_failure(monkeypatch):
    monkeypatch.setenv("H3ATTN_FAULT", "launch")
    assert _static_call() == h.H3ATTN_ERR_HIP and "injected" in h.last_error()
    assert _static_call(cu=(0, 7169)) == h.H3ATTN_ERR_WORKSPACE       # the size check comes first


def test_mfma_ceiling_argument_errors(monkeypatch):
    for args, msg in [((6, 256, 10), "mix"), ((-1, 256, 10), "mix"), ((0, 0, 10), "workgroups"), ((0, 1 << 21, 10), "workgroups"),
                      ((0, 256, 0), "iters"), ((1, 256, 1 << 21), "iters")]:
        assert h.mfma_ceiling_raw(*args, FAKE, None) == h.H3ATTN_ERR_INVALID_ARG
        assert msg in h.last_error()
    assert h.mfma_ceiling_raw(0, 256, 10, 0, None) == h.H3ATTN_ERR_INVALID_ARG and "NULL" in h.last_error()
    assert h.mfma_ceiling_raw(0, 256, 10, FAKE + 2, None) == h.H3ATTN_ERR_INVALID_ARG
    if not _gpu_present():
        assert h.mfma_ceiling_raw(0, 256, 10, FAKE, None) == h.H3ATTN_ERR_DEVICE
    monkeypatch.setenv("H3ATTN_FAULT", "launch")
    assert h.mfma_ceiling_raw(1, 256, 10, FAKE, None) == h.H3ATTN_ERR_HIP and "mfma ceiling" in h.last_error()


def test_binding_refuses_another_abi_version(tmp_path):
    """A library of another ABI version lays out its tile lists and workspaces
    differently (version 1 kept one block-sparse list per 128 query rows), so
    the arrays this binding allocates would be too small for it: the binding
    refuses to load it instead of letting its kernels write past them."""
    import subprocess
    import sys
    src = tmp_path / "stub.c"
    names = [n for n in h.EXPORTED if n != "h3attn_version"]
    src.write_text("".join("int %s(void) { return 0; }\n" % n for n in names) +
                   "int h3attn_version(void) { return 1; }\n")
    so = tmp_path / "libstub.so"
    subprocess.run(["gcc", "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    code = ("import audio_diffusion_transformer_amd.h3attn as h\n"
            "try:\n    h.lib()\n    print('LOADED')\nexcept RuntimeError as e:\n    print('REFUSED', e)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       env=dict(os.environ, H3ATTN_LIB=str(so)))
    assert "REFUSED" in r.stdout and "ABI version 1" in r.stdout, r.stdout + r.stderr


def test_checked_entry_point_and_checked_build():
    """h3attn_checked is a diagnostic of the checked build: the product library
    refuses it before touching a device; the checked library (same sources with
    H3ATTN_CHECKED) exports exactly the same symbols and the same ABI version."""
    import ctypes as C
    from audio_diffusion_transformer_amd import build as B
    with pytest.raises(h.H3AttnError) as e:
        h.checked()
    assert e.value.status == h.H3ATTN_ERR_UNSUPPORTED and "without checks" in str(e.value)
    assert os.path.exists(B.LIB_CHECKED), "libh3attn_checked.so is not built"
    L = C.CDLL(B.LIB_CHECKED)
    for n in h.EXPORTED:
        assert hasattr(L, n), n
    L.h3attn_version.restype = C.c_int
    assert L.h3attn_version() == h.H3ATTN_VERSION
    if not _gpu_present():
        L.h3attn_checked.restype = C.c_int
        L.h3attn_checked.argtypes = [C.c_void_p, C.c_int, C.c_uint32]
        assert L.h3attn_checked(None, 0, 0) == h.H3ATTN_ERR_DEVICE     # past the build check, no device here
