"""Build libh3attn.so in-tree with hipcc for gfx950.

Run ``python -m audio_diffusion_transformer_amd.build``; the library lands next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libh3attn.so")
# The same sources with the attention kernels' invariant checks and timing
# jitter compiled in (H3ATTN_CHECKED); loaded only through H3ATTN_LIB.
LIB_CHECKED = os.path.join(HERE, "libh3attn_checked.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-variable",
    # no NaNs reach the kernels' arithmetic: lets fmaxf lower to plain v_max/v_max3
    # without canonicalising each operand first (infinities are still honoured)
    "-fno-honor-nans",
    # no packed-fp32 VALU forms (v_pk_{add,mul,fma}_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + list(extra) + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % out)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
    if verbose and msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False):
    """The product library and its checked build."""
    return build(verbose), build(verbose, out=LIB_CHECKED, extra=("-DH3ATTN_CHECKED",))


if __name__ == "__main__":
    print(build_all(verbose=True))
