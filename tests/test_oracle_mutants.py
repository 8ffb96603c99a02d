"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Every mutant is compiled from a textual edit of ``oracle/h3_oracle.c`` into a
temporary directory (the committed oracle is never touched) and the pin
functions of ``test_oracle_pins.py`` are run against it.  A mutant that
survives every pin means the pins cannot tell that mistake from the right
arithmetic.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "h3_oracle.c")

MUTANTS = {
    "rmsnorm_drops_eps": ("1.0 / sqrt(ss / d + eps)", "1.0 / sqrt(ss / d)"),
    "rmsnorm_sum_not_mean": ("1.0 / sqrt(ss / d + eps)", "1.0 / sqrt(ss + eps)"),
    "rmsnorm_drops_weight": ("* r * (double)w[c]", "* r"),
    "rope_sign_first": ("y[2 * j] = a * c - b * s;", "y[2 * j] = a * c + b * s;"),
    "rope_sign_second": ("y[2 * j + 1] = a * s + b * c;", "y[2 * j + 1] = -a * s + b * c;"),
    "rope_half_split_pairs": ("double a = x[2 * j], b = x[2 * j + 1];",
                              "double a = x[j], b = x[j + d / 2];"),
    "rope_freq_uses_head_dim": ("phi[off / 2 + j] = (double)pos[a] * pow(p->theta, -2.0 * j / (double)D);",
                                "phi[off / 2 + j] = (double)pos[a] * pow(p->theta, -2.0 * j / (double)d);"),
    "rope_freq_exponent": ("phi[off / 2 + j] = (double)pos[a] * pow(p->theta, -2.0 * j / (double)D);",
                           "phi[off / 2 + j] = (double)pos[a] * pow(p->theta, -1.0 * j / (double)D);"),
    "rope_section_order": ("phi[off / 2 + j] = (double)pos[a] *", "phi[off / 2 + j] = (double)pos[2 - a] *"),
    "raster_swapped": ("pos[1] = (int32_t)((i / g->Wg) % g->Hg);", "pos[1] = (int32_t)((i / g->Hg) % g->Wg);"),
    "audio_position_absolute": ("pos[0] = (int32_t)(i - nv);", "pos[0] = (int32_t)(i);"),
    "audio_freq_section": ("phi[j] = (double)pos[0] * pow(p->theta, -2.0 * j / (double)d);",
                           "phi[j] = (double)pos[0] * pow(p->theta, -2.0 * j / (double)p->split[0]);"),
    "k_uses_q_weights": ("p->norm_w + ((int64_t)which * p->H + head) * d", "p->norm_w + ((int64_t)head) * d"),
    "softmax_scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "output_not_normalised": ("oi[c] = nk > 0 ? oi[c] / l : 0.0;", "oi[c] = nk > 0 ? oi[c] : 0.0;"),
    "value_channel_index": ("oi[c] += pj * v[j * d + c];", "oi[c] += pj * v[j * d + (d - 1 - c)];"),
    "sequence_boundary": ("if (token >= p->cu[s] && token < p->cu[s + 1]) return s;",
                          "if (token >= p->cu[s] && token <= p->cu[s + 1]) return s;"),
    "kmean_divisor": ("acc[c2] / (double)n", "acc[c2] / (double)(n + 1)"),
    "int8_scale_128": ("amax > 0 ? amax / 127.0 : 1.0", "amax > 0 ? amax / 128.0 : 1.0"),
    "int8_round_half_up": ("double q = nearbyint(r);", "double q = floor(r + 0.5);"),
    "e4m3_round_half_up": ("double mant = nearbyint((2.0 * f - 1.0) * 8.0);",
                           "double mant = floor((2.0 * f - 1.0) * 8.0 + 0.5);"),
    "e4m3_subnormal_step": ("double q = nearbyint(a / ldexp(1.0, -9));", "double q = nearbyint(a / ldexp(1.0, -10));"),
    "v_scale_fnuz_max": ("scale_out[c] = amax > 0 ? amax / 448.0 : 1.0;",
                         "scale_out[c] = amax > 0 ? amax / 240.0 : 1.0;"),
    "lazy_rescale_on_any_rise": ("if (mx - *m > 1.0) {", "if (mx - *m > 0.0) {"),
    "q8_rowsum_unquantised": ("\n            l += P;\n", "\n            l += 224.0 * exp2(x[j] - m);\n"),
    "q8_p_scale_448": ("orc_e4m3_encode(224.0 * exp2(x[j] - m))", "orc_e4m3_encode(448.0 * exp2(x[j] - m))"),
    "q8_score_natural_log": ("x->qscale[qi / 64] * p->scale / log(2.0)", "x->qscale[qi / 64] * p->scale"),
    "projected_k_from_q": ("const double *xf = which == 0 ? p->qf : p->kf;",
                           "const double *xf = which == 0 ? p->qf : p->qf;"),
    "projected_v_channel": ("p->vf ? p->vf[at + c] :", "p->vf ? p->vf[at + (c ^ 1)] :"),
    "e2m1_round_half_up": ("double mant = nearbyint((2.0 * f - 1.0) * 2.0);",
                           "double mant = floor((2.0 * f - 1.0) * 2.0 + 0.5);"),
    "e2m1_subnormal_half_up": ("double q = nearbyint(a / 0.5);", "double q = floor(a / 0.5 + 0.5);"),
    "mx_scale_offset": ("int X = e - 1 - 2;", "int X = e - 1 - 1;"),
    "mx_scale_low_limit": ("if (X < -126) X = -126;", "if (X < -127) X = -127;"),
    "mx_k_first_block_scale": ("kx[j * nb + c / 32]", "kx[j * nb]"),
    "mx_v_scale_of_first_block": ("vx[(j / 32) * d + c]", "vx[c]"),
    "mx_score_natural_log": ("double qs = p->scale / log(2.0);\n    for (int c = 0; c < p->d; ++c) row[c] *= qs;",
                             "double qs = p->scale;\n    for (int c = 0; c < p->d; ++c) row[c] *= qs;"),
    "mx_rowsum_unquantised": ("                l += P;\n", "                l += exp2(x[b0 + i] - m);\n"),
    "mx_query_from_k": ("prologue_one(p, 0, sel[i] / p->H, h, row);", "prologue_one(p, 1, sel[i] / p->H, h, row);"),
    "q8_first_block_qscale": ("double qs = x->qscale[qi / 64] * p->scale / log(2.0);",
                              "double qs = x->qscale[0] * p->scale / log(2.0);"),
    "q8_qscale_of_next_block": ("double qs = x->qscale[qi / 64] * p->scale / log(2.0);",
                                "double qs = x->qscale[(qi + 1) / 64] * p->scale / log(2.0);"),
    "q8_v_scale_of_first_channel": ("vdec[j * d + c] = orc_e4m3_decode(vc[j * d + c]) * vsc[c];",
                                    "vdec[j * d + c] = orc_e4m3_decode(vc[j * d + c]) * vsc[0];"),
    "q8_v_scale_channel_reversed": ("vdec[j * d + c] = orc_e4m3_decode(vc[j * d + c]) * vsc[c];",
                                    "vdec[j * d + c] = orc_e4m3_decode(vc[j * d + c]) * vsc[d - 1 - c];"),
    "q8_first_block_kscale": ("s[j] = (double)dot * qs * x->kscale[j / 64];",
                              "s[j] = (double)dot * qs * x->kscale[0];"),
}


def _pin_functions():
    return [f for n, f in sorted(inspect.getmembers(pins, inspect.isfunction))
            if n.startswith("test_") and not inspect.signature(f).parameters]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation pattern must occur exactly once: %r" % old
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mut_src), out=so)
    pins.LIB = oracle.lib(so)
    caught = []
    try:
        for fn in _pin_functions():
            try:
                fn()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(fn.__name__)
                break
    finally:
        pins.LIB = None
    assert caught, "no pin caught mutant %s" % name


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = str(tmp_path / "libcopy.so")
    oracle.build(force=True, src=SRC, out=so)
    pins.LIB = oracle.lib(so)
    try:
        for fn in _pin_functions():
            fn()
    finally:
        pins.LIB = None
