"""Cases of the checked-build comparison (tests/test_gpu_checked.py), and the
runner that executes them in a process whose binding loads another library
(H3ATTN_LIB).  Run as ``python -m tests.checked_run OUT.npz SEED [SEED ...]``:
computes every case's attention output once per jitter seed and saves the
bf16 bits and the checked build's flag words."""
import sys

import numpy as np

from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

Seq = synth.Seq
CASES = {
    # head_dim 128: the eight-wave kernel, dense (ragged batch, a long sequence, sharp inputs that take
    # the lazily rescaled running maximum) and block-sparse with caller lists
    "ragged_d128": synth.Workload("chk_ragged_d128", H=2, d=128, seqs=(Seq(3, 10, 11, 7), Seq(0, 1, 1),
                                                                   Seq(1, 4, 5, 70)), split=(32, 48, 48), seed=71),
    "long_d128": synth.Workload("chk_long_d128", H=2, d=128, seqs=(Seq(6, 20, 25, 40),), split=(32, 48, 48),
                                seed=72),
    "sharp_d128": synth.Workload("chk_sharp_d128", H=2, d=128, seqs=(Seq(4, 10, 15, 100),), split=(32, 48, 48),
                                 seed=73, sharp=True),
    # head_dim 64: the four-wave kernel
    "long_d64": synth.Workload("chk_long_d64", H=2, d=64, seqs=(Seq(5, 16, 20, 33), Seq(1, 3, 3)),
                               split=(16, 24, 24), seed=74),
}
SPARSE = {"long_d128": 7, "long_d64": 5}      # cases also run block-sparse, with this many tiles per list
QUANT = {"long_d128": (True, "mx"), "ragged_d128": (True, "mx")}   # cases also run on the INT8/FP8 and MXFP4 paths


def random_lists(w, tpb, seed, bad=False):
    """Caller tile lists (distinct valid tiles, random order); with ``bad`` one
    entry per sequence is out of range, which the kernels clamp and the
    checked build flags."""
    rng = np.random.default_rng(seed)
    rows = []
    for s in w.seqs:
        nt = (s.n + 63) // 64
        for _ in range(w.H):
            for qb in range((s.n + h.SPARSE_BLOCK_ROWS - 1) // h.SPARSE_BLOCK_ROWS):
                L = min(tpb, nt)
                row = np.full(tpb, -1, dtype=np.int32)
                row[:L] = rng.choice(nt, L, replace=False)
                if bad and qb == 0:
                    row[0] = nt + 3
                rows.append(row)
    return np.stack(rows)


def run_all(torch):
    """Every case's output bits, dense and block-sparse."""
    res = {}
    for name, w in CASES.items():
        inp = synth.generate(w)
        t = G.to_device(inp, w)
        res[name] = G.bits(G.run(w, t, label="checked-comparison " + name))
        for mode in QUANT.get(name, ()):
            tag = "q8" if mode is True else mode
            res["%s_%s" % (name, tag)] = G.bits(G.run(w, t, quantized=mode, label="checked-comparison %s %s" % (
                name, tag)))
        if name in SPARSE:
            tpb = SPARSE[name]
            bt = torch.from_numpy(random_lists(w, tpb, seed=tpb)).to("cuda:0")
            G.announce("checked-comparison %s block-sparse tpb=%d" % (name, tpb))
            out, _ = h.h3attn_fwd_sparse(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], tpb,
                                         block_tiles=bt, select=False, eps=w.eps)
            torch.cuda.synchronize()
            res[name + "_sparse"] = G.bits(out)
    return res


def main(argv):
    import torch
    out_path, seeds = argv[0], [int(x) for x in argv[1:]]
    saved = {}
    for seed in seeds:
        h.checked(clear=True, jitter_seed=seed)
        for name, bits in run_all(torch).items():
            saved["%s@%d" % (name, seed)] = bits
        saved["flags@%d" % seed] = h.checked(clear=True, jitter_seed=0)
    # the jitter is live: the long head_dim-128 case takes longer with delays than without
    w = CASES["long_d128"]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    # (the best of three batches of 20 calls each, so a stray slow batch cannot decide it)
    for seed in (0, 1):
        h.checked(clear=False, jitter_seed=seed)
        h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], eps=w.eps)
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                h.h3attn_fwd(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], eps=w.eps)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 20)
        saved["ms@%d" % seed] = np.array([best])
    h.checked(clear=True, jitter_seed=0)
    # a list entry out of range: clamped by the kernel, recorded in flag word 3
    bt = torch.from_numpy(random_lists(w, 7, seed=7, bad=True)).to("cuda:0")
    G.announce("checked build: block-sparse list with an out-of-range entry")
    h.h3attn_fwd_sparse(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], 7, block_tiles=bt, select=False,
                        eps=w.eps)
    torch.cuda.synchronize()
    saved["flags@bad_list"] = h.checked(clear=True, jitter_seed=0)
    np.savez(out_path, **saved)
    print("checked run done: %d arrays" % len(saved), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
