#!/usr/bin/env python3
"""Benchmark of the fused RMSNorm + RoPE + attention hot path on one MI355X.

One step = one h3attn_fwd pass (the prologue kernel, then the attention
kernel) over the joint video+audio workload: one packed sequence of a
t31 x h48 x w84 video grid (124,992 tokens) plus 250 audio tokens, H = 24,
d = 128, bf16 inputs already resident in HBM.  The step is issued as its two
stages (h3attn_fwd_stages 1 then 2, exactly what h3attn_fwd does) with HIP
events between them on the launch stream, so each kernel's average duration
is measured live over the timed region.

Prints one JSON line: whole-step attention TFLOP/s (4 * sum n_i^2 * d * H per
step), the attention kernel's roofline against the bf16 dense MFMA peak, and
the CPU oracle's throughput on a bounded sample of the same workload.

With a projection workload (``--workload proj_joint``) a step starts from the
hidden states: the fused QKV projection + prologue kernel, then the attention
kernel (h3attn_fwd_proj_stages 1 and 2), then the output projection with its
gated residual; the step's FLOP count adds the projections' 2 * N * D * 3*H*d
and 2 * N * H*d * D, and the line also reports the projection kernel beside
the vendor-library GEMM plus the separate prologue.  ``--workload
proj_q8_joint`` runs the same layer on the quantised path
(h3attn_fwd_proj_q8_stages: the projection with the INT8/FP8 prologue, then
the INT8/FP8 attention).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from audio_diffusion_transformer_amd.h3attn import SPARSE_BLOCK_ROWS  # noqa: E402  (no library load)

MI355X_BF16_DENSE_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense, no sparsity)
MI355X_FP8_DENSE_TFLOPS = 5033.2
MI355X_FP4_DENSE_TFLOPS = 10066.4     # FP4 (and FP6) dense MFMA
MI355X_HBM_GBPS = 8000.0
# performance gate of the attention kernel: this fraction of its datasheet peak
PERF_GATE_FRAC = 0.60
METRIC = "attention TFLOP/s and % of bf16 MFMA peak at N=125k packed tokens, H=24, d=128"


def kernel_source_sha(name: str) -> str:
    path = os.path.join(ROOT, "audio_diffusion_transformer_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_source_sha(kernel_file):
        return None
    return float(t.group(1))


def _sha256_file(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for blk in iter(lambda: f.read(1 << 20), b""):
            h.update(blk)
    return h.hexdigest()


def _input_digest(arrays) -> str:
    """xxh3-64 (blake2b when xxhash is absent) over the input arrays' bytes, in order."""
    try:
        import xxhash
        h, kind = xxhash.xxh3_64(), "xxh3_64"
    except ImportError:
        h, kind = hashlib.blake2b(digest_size=8), "blake2b-64"
    for a in arrays:
        h.update(memoryview(np.ascontiguousarray(a)).cast("B"))
    return "%s:%s" % (kind, h.hexdigest())


def provenance(torch, h, w, inputs) -> dict:
    """What the line was measured on and with: device, ROCm/HIP and torch
    versions, the library file and ABI, the sources it was built from, the
    command line, the workload seed and a digest of the generated inputs."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    csrc = os.path.join(ROOT, "audio_diffusion_transformer_amd", "csrc")
    src = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        src.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            src.update(f.read())
    keys = [k for k in ("q", "k", "v", "x", "w_qkv", "norm_w", "cu_seqlens") if k in inputs]
    return {
        "gpu": torch.cuda.get_device_name(0),
        "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "rocm": rocm,
        "hip_runtime": torch.version.hip,
        "torch": torch.__version__,
        "library": {"file": os.path.relpath(h.LIB_PATH, ROOT), "sha256": _sha256_file(h.LIB_PATH),
                    "abi_version": h.version()},
        "sources_sha256": src.hexdigest(),
        "argv": sys.argv[1:],
        "workload_seed": w.seed,
        "inputs": keys,
        "inputs_digest": _input_digest([inputs[k] for k in keys]),
    }


def parity_metrics(got: np.ndarray, ref: np.ndarray, against: str) -> dict:
    """The run's own output rows against the oracle's rows for the same queries."""
    d = got - ref
    nr = float(np.linalg.norm(ref))
    return {"rows": int(got.shape[0]), "against": against,
            "max_abs": float(np.abs(d).max()), "mean_abs": float(np.abs(d).mean()),
            "rel_l2": float(np.linalg.norm(d) / max(nr, 1e-300)),
            "cosine": float(np.sum(got * ref) / max(np.linalg.norm(got) * nr, 1e-300))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads():
    """Threads for the CPU oracle: every CPU this process may run on, limited
    to the job's CPU share when OMP_NUM_THREADS states one (a one-GPU job on a
    shared host gets a slice of its cores).  Returns (threads, host facts)."""
    host_cpus = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = host_cpus
    share = os.environ.get("OMP_NUM_THREADS", "").strip()
    threads = affinity
    if share.isdigit() and int(share) > 0:
        threads = min(affinity, int(share))
    return max(1, threads), {"host_cpus": host_cpus, "affinity_cpus": affinity,
                             "job_cpu_share": int(share) if share.isdigit() else None}


def device_copy_rate(torch, dev, mib: int = 1024, reps: int = 5) -> float:
    """GB/s (read + write bytes) of a plain device-to-device copy, the practical
    rate of mixed HBM traffic the prologue is compared with."""
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def mfma_ceiling(torch, h, dev, stream, path: str = "bf16", target_ms: float = 120.0):
    """Sustained matrix-core rate of this device (h3attn_mfma_ceiling):
    register-only MFMA streams on changing operands on all 256 CUs, alone and
    with the vector work the attention adds beside its MFMAs.  bf16 (mixes 0,
    1): v_mfma_f32_32x32x16_bf16, then with one v_exp_f32 + one FMA per MFMA.
    Quantised (mixes 2, 3): v_mfma_i32_32x32x32_i8, then with two FMAs, two
    v_exp_f32, one FP8 pack and one max per MFMA (the quantised kernel's
    ratio).  MXFP4 (mixes 4, 5): the scaled FP4 MFMA, then with four v_exp_f32,
    two FP4 packs, two max3 and one FMA per MFMA.  Each launch runs ~target_ms, long enough for the clock to settle
    where the power limit holds it; one warm-up launch, then two timed.
    Returns the rates (TFLOP/s or TOP/s) of both mixes (after the timed region)."""
    wg = 256
    out = torch.empty(512 * wg, dtype=torch.float32, device=dev)
    sp = int(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(mix, iters, reps):
        e0.record(stream)
        for _ in range(reps):
            st = h.mfma_ceiling_raw(mix, wg, iters, out.data_ptr(), sp)
            if st != 0:
                raise RuntimeError("%s: %s" % (h.status_string(st), h.last_error()))
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    mixes, ops_per_mfma = {
        "bf16": (((0, "mfma_only_TFLOPs"), (1, "mfma_with_exp_fma_TFLOPs")), 32768.0),
        "q8": (((2, "int8_mfma_only_TOPs"), (3, "int8_mfma_with_q8_vector_work_TOPs")), 65536.0),
        "mx": (((4, "fp4_mfma_only_TFLOPs"), (5, "fp4_mfma_with_mx_vector_work_TFLOPs")), 131072.0),
    }[path]
    flop_per_iter = ops_per_mfma * 8 * 8 * wg
    res = {}
    for mix, key in mixes:
        probe = 20000
        ms = timed(mix, probe, 1)
        iters = int(max(1, min(1 << 20, probe * target_ms / max(ms, 1e-3))))
        timed(mix, iters, 1)                      # warm-up at the full length
        ms = timed(mix, iters, 2)
        res[key] = round(flop_per_iter * iters / (ms * 1e-3) / 1e12, 1)
    del out
    return res


def one_head_problem(w, inputs, head: int):
    """The oracle problem of one head of a projection workload: its q, k, v
    rows of W_qkv, projected in fp64 (heads are independent)."""
    import oracle
    hd = w.H * w.d
    sel = np.concatenate([part * hd + head * w.d + np.arange(w.d) for part in range(3)])
    w1 = w.replace(H=1)
    sub = {"x": inputs["x"], "w_qkv": np.ascontiguousarray(inputs["w_qkv"][sel]),
           "norm_w": np.ascontiguousarray(inputs["norm_w"][:, [head]])}
    return w1, oracle.Problem.from_projection(w1, sub)


def cpu_baseline_sparse(w, inputs, seconds: float, threads: int, gpu_rows=None, gpu_lists=None):
    """Time the fp64 CPU oracle of the block-sparse path on one head: its own
    tile selection for that head, then sampled query rows over their kept keys.
    With gpu_rows / gpu_lists (the GPU's output rows and tile lists of that
    head) the timed rows of blocks whose lists agree are also compared."""
    import oracle
    rng = np.random.default_rng(w.seed + 99)
    head = int(rng.integers(w.H))
    sub = {key: np.ascontiguousarray(inputs[key][:, [head]]) for key in ("q", "k", "v")}
    sub["norm_w"] = np.ascontiguousarray(inputs["norm_w"][:, [head]])
    p = oracle.Problem.from_workload(w.replace(H=1), sub)
    t0 = time.perf_counter()
    tiles, _ = p.sparse_select(w.keep_tiles)
    sel_s = time.perf_counter() - t0
    n = w.seqs[0].n
    nt = (n + 63) // 64
    keys_per_block = [int(np.minimum(64, n - 64 * tiles[qb, :min(w.keep_tiles, nt)].astype(np.int64)).sum())
                      for qb in range(tiles.shape[0])]

    B = oracle.SPARSE_BLOCK
    nqb = (n + B - 1) // B

    def run(nblocks):
        # whole query blocks: the kept keys' khat is formed once per block, as in a full run
        blocks = np.sort(rng.choice(nqb, size=nblocks, replace=False))
        toks = np.concatenate([np.arange(B * qb, min(B * qb + B, n)) for qb in blocks]).astype(np.int64)
        t1 = time.perf_counter()
        vals = p.sparse_attention_rows(toks, tiles, w.keep_tiles, nthreads=threads)
        return time.perf_counter() - t1, toks, vals

    t_probe, _, _ = run(1)
    nb = int(max(1, min(nqb, seconds / max(t_probe, 1e-6))))
    t, toks, vals = run(nb)
    nrows = len(toks)
    flops = sum(4.0 * w.d * keys_per_block[int(tk) // B] for tk in toks)
    t += sel_s * nrows / n                 # the head's selection, spread over its rows
    value = flops / t / 1e12
    res = {
        "value": round(value, 6), "unit": "TFLOP/s", "cores": threads, "cpu_model": cpu_model(),
        "extrapolated_full_s": round(sparse_total_flops_estimate(w, keys_per_block) / (value * 1e12), 1),
        "kind": "oracle",
        "sample": "%d query rows (%d whole %d-row blocks) of head %d (of %d x %d rows), each over the keys of "
                  "the %d tiles the oracle keeps for its block; fp64; the head's pooled-score selection (%.1f s) "
                  "spread over its rows; %.1f s" % (nrows, nb, B, head, w.N, w.H, w.keep_tiles, sel_s, t),
    }
    if gpu_rows is not None and gpu_lists is not None:
        same = np.all(gpu_lists(head) == tiles, axis=1)           # blocks whose kept tiles agree
        keep = same[toks // B]
        if keep.any():
            res["parity"] = parity_metrics(gpu_rows(toks[keep], head), vals[keep],
                                           "fp64 oracle over the same kept tiles (blocks whose lists agree: "
                                           "%d of %d)" % (int(same.sum()), len(same)))
    return res


def sparse_total_flops_estimate(w, keys_per_block) -> float:
    n, B = w.seqs[0].n, SPARSE_BLOCK_ROWS
    return float(sum(4.0 * w.d * min(B, n - B * qb) * k for qb, k in enumerate(keys_per_block))) * w.H


def cpu_baseline(w, inputs, seconds: float, threads: int, gpu_rows=None, gpu_lists=None):
    """Time the fp64 CPU oracle on sampled query rows of one head (full key
    set).  With gpu_rows (token indices, head -> the GPU output rows) the
    oracle rows of the timed run are also compared with this run's output."""
    import oracle
    if w.keep_tiles > 0:
        return cpu_baseline_sparse(w, inputs, seconds, threads, gpu_rows, gpu_lists)
    rng = np.random.default_rng(w.seed + 99)
    head = int(rng.integers(w.H))
    n = w.seqs[0].n
    flops_per_row = 4.0 * n * w.d
    proj_s = 0.0
    if w.model_dim > 0:
        # the one head's fp64 projection of every token is part of the timed work
        t0 = time.perf_counter()
        w1, p = one_head_problem(w, inputs, head)
        proj_s = time.perf_counter() - t0
        H_rows, head_row = 1, 0
        flops_per_row += 2.0 * w.model_dim * 3 * w.d        # the row's share of the projection
    else:
        p = oracle.Problem.from_workload(w, inputs)
        H_rows, head_row = w.H, head

    rows_fn = p.mx_attention_rows if w.fp4 else p.attention_rows

    last = {}

    def run(nrows):
        toks = np.sort(rng.choice(n, size=nrows, replace=False)).astype(np.int64)
        rows = toks * H_rows + head_row
        t0 = time.perf_counter()
        last["vals"] = rows_fn(rows, nthreads=threads)
        last["toks"] = toks
        return time.perf_counter() - t0

    # fixed cost (the keys' prologue, and for the FP4 emulation their
    # quantisation) + per-row cost, from two probes far enough apart that the
    # per-row part stands out of the fixed part, the larger one big enough to
    # see the memory-bound rate of many rows streaming the keys at once
    probe = 2 * threads
    t1 = run(probe)
    t2 = run(20 * probe)
    per_row = max((t2 - t1) / (19 * probe), 1e-6)
    fixed = max(t1 - per_row * probe, 0.0)
    nrows = int(max(probe, min(n, (seconds - fixed) / per_row)))
    t = run(nrows)
    if w.model_dim > 0:
        # the head's projection time is spread over all n of its rows
        t += proj_s * nrows / n
    value = nrows * flops_per_row / t / 1e12
    sample = ("%d query rows of head %d (of %d x %d rows), each over all %d keys; fp64; "
              "the keys' RMSNorm+RoPE included; %.1f s" % (nrows, head, w.N, w.H, n, t))
    if w.fp4:
        sample += "; the step-by-step MXFP4 emulation (codes of q, k, v, FP4 probabilities)"
    if w.model_dim > 0:
        sample += ("; plus the head's fp64 QKV projection of all tokens (%.1f s, %.0f%% of it "
                   "charged to the sampled rows)" % (proj_s, 100.0 * nrows / n))
    res = {
        "value": round(value, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "extrapolated_full_s": round((w.flops() + w.proj_flops()) / (value * 1e12), 1),
        "kind": "oracle",
        "sample": sample,
    }
    if gpu_rows is not None:
        res["parity"] = parity_metrics(gpu_rows(last["toks"], head), last["vals"],
                                       "fp64 MXFP4 emulation" if w.fp4 else "exact fp64 attention")
    return res


def library_gemm_then_prologue(torch, h, w, x, wq, norm_w, rope, cu, ws, ws_bytes, stream, reps: int = 5):
    """The unfused alternative, timed after the timed region: the QKV product on
    the vendor library (torch.mm, hipBLASLt) into a bf16 [N, 3*H*d] buffer,
    then this library's prologue (the quantised one for a quantised workload)
    reading q, k and v as strided views of it."""
    hd = w.H * w.d
    y = torch.empty((w.N, 3 * hd), dtype=torch.bfloat16, device=x.device)
    wt = wq.t()
    q, k, v = (y[:, i * hd:(i + 1) * hd].view(w.N, w.H, w.d) for i in range(3))
    out = torch.empty((w.N, w.H, w.d), dtype=torch.bfloat16, device=x.device)
    params = h.params_for(q, k, v, out, len(cu) - 1, w.eps)
    ptrs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), norm_w.data_ptr(), rope.data_ptr()]
    assert ws_bytes >= h.h3attn_workspace_size(params, cu, w.quantized)

    def prologue():
        st = h.fwd_raw(params, *ptrs, cu, out.data_ptr(), ws.data_ptr(), ws_bytes, int(stream.cuda_stream),
                       w.quantized, 1)
        if st != 0:
            raise RuntimeError(h.last_error())

    torch.mm(x, wt, out=y)
    prologue()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    gemm, pro = [], []
    for _ in range(reps):
        ev[0].record(stream)
        torch.mm(x, wt, out=y)
        ev[1].record(stream)
        prologue()
        ev[2].record(stream)
        torch.cuda.synchronize()
        gemm.append(ev[0].elapsed_time(ev[1]))
        pro.append(ev[1].elapsed_time(ev[2]))
    del y, out
    g, p = float(np.mean(gemm)), float(np.mean(pro))
    return {"library_gemm_ms": round(g, 4),
            "library_gemm_TFLOPs": round(w.proj_flops() / (g * 1e-3) / 1e12, 1),
            "unfused_prologue_ms": round(p, 4),
            "unfused_total_ms": round(g + p, 4)}


def sparse_flops(w, tiles) -> float:
    """4 * d * (query rows) * (kept keys) summed over the (sequence, head, query
    block) items of the tile lists: the attention work the sparse kernel does."""
    total, it = 0.0, 0
    for s in w.seqs:
        n = s.n
        nt = (n + 63) // 64
        L = min(w.keep_tiles, nt)
        for _ in range(w.H):
            for qb in range((n + SPARSE_BLOCK_ROWS - 1) // SPARSE_BLOCK_ROWS):
                rows = min(SPARSE_BLOCK_ROWS, n - SPARSE_BLOCK_ROWS * qb)
                kept = tiles[it, :L].astype(np.int64)
                keys = np.minimum(64, n - 64 * kept).sum()
                total += 4.0 * w.d * rows * float(keys)
                it += 1
    return total


def dense_attention_ms(torch, h, w, params, ptrs, cu, out, ws, ws_bytes, stream, reps: int = 3) -> float:
    """The dense attention kernel on the same inputs (after the timed region),
    for the speed-up of the block-sparse one."""
    def run():
        st = h.fwd_raw(params, *ptrs, cu, out.data_ptr(), ws.data_ptr(), ws_bytes, int(stream.cuda_stream), False, 2)
        if st != 0:
            raise RuntimeError(h.last_error())
    h.fwd_raw(params, *ptrs, cu, out.data_ptr(), ws.data_ptr(), ws_bytes, int(stream.cuda_stream), False, 1)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def library_out_proj(torch, w, attn, w_o, gate, resid, stream, reps: int = 5):
    """The unfused output projection, timed after the timed region: torch.mm
    (hipBLASLt) of the attention output by W_o^T, then the gated residual as
    one torch elementwise kernel (the workload has one sequence, so its gate
    row broadcasts)."""
    a2 = attn.view(w.N, w.H * w.d)
    wt = w_o.t()
    g = gate[0].to(torch.bfloat16)
    y = torch.mm(a2, wt)
    z = torch.addcmul(resid, y, g)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    mm, ew = [], []
    for _ in range(reps):
        ev[0].record(stream)
        torch.mm(a2, wt, out=y)
        ev[1].record(stream)
        torch.addcmul(resid, y, g, out=z)
        ev[2].record(stream)
        torch.cuda.synchronize()
        mm.append(ev[0].elapsed_time(ev[1]))
        ew.append(ev[1].elapsed_time(ev[2]))
    del y, z
    m_, e_ = float(np.mean(mm)), float(np.mean(ew))
    return {"library_out_gemm_ms": round(m_, 4), "library_gated_residual_ms": round(e_, 4),
            "unfused_out_total_ms": round(m_ + e_, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="joint")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB "
                         "(reference kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from audio_diffusion_transformer_amd import h3attn as h
    from audio_diffusion_transformer_amd import synth

    w = synth.WORKLOADS[args.workload]
    proj = w.model_dim > 0
    sparse = w.keep_tiles > 0
    t0 = time.time()
    inp = synth.generate(w)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    norm_w = torch.from_numpy(inp["norm_w"]).to(dev)
    rope = torch.from_numpy(h.rope_table(w.seqs, w.split, w.d, w.theta)).to(dev)
    cu = inp["cu_seqlens"]
    out = torch.empty((w.N, w.H, w.d), dtype=torch.bfloat16, device=dev)
    if proj:
        x, wq = up(inp["x"]), up(inp["w_qkv"])
        params = h._proj_params(x, wq, w.H, w.d, len(cu) - 1, out.stride(0), w.eps, 0.0)
        gout = synth.generate_out(w)
        w_o, resid = up(gout["w_o"]), up(gout["resid"])
        gate = torch.from_numpy(gout["gate"]).to(dev)
        y = torch.empty((w.N, w.model_dim), dtype=torch.bfloat16, device=dev)
        del gout
    else:
        q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
        params = h.params_for(q, k, v, out, len(cu) - 1, w.eps)
        ptrs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), norm_w.data_ptr(), rope.data_ptr()]
    mode = "mx" if w.fp4 else w.quantized
    ws_bytes = h.h3attn_workspace_size(params, cu, 2 if sparse else 4 if (proj and w.quantized) else mode)
    if sparse:
        tiles = torch.empty((h.sparse_items(cu, w.H), w.keep_tiles), dtype=torch.int32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    torch.cuda.synchronize()
    print("[bench] inputs ready for %s (N=%d) in %.1f s" % (w.name, w.N, time.time() - t0),
          file=sys.stderr, flush=True)

    if args.calib_copy_mb > 0:
        nb = args.calib_copy_mb << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: %d bytes read, %d bytes written" % (nb, nb),
              file=sys.stderr, flush=True)
        del src, dst

    def stage(sid):
        if sparse:
            # 1 prologue, 2 tile selection, 4 attention over the kept tiles
            st = h.sparse_raw(params, *ptrs, cu, w.keep_tiles, tiles.data_ptr(), out.data_ptr(), ws.data_ptr(),
                              ws_bytes, sp, sid)
        elif proj and sid == 4:
            st = h.out_proj_raw(w.H, w.d, w.model_dim, cu, out.data_ptr(), out.stride(0), w_o.data_ptr(),
                                gate.data_ptr(), resid.data_ptr(), resid.stride(0), y.data_ptr(), y.stride(0), sp)
        elif proj:
            st = h.proj_raw(params, w.model_dim, x.data_ptr(), x.stride(0), wq.data_ptr(), norm_w.data_ptr(),
                            rope.data_ptr(), cu, out.data_ptr(), ws.data_ptr(), ws_bytes, sp, sid, w.quantized)
        else:
            st = h.fwd_raw(params, *ptrs, cu, out.data_ptr(), ws.data_ptr(), ws_bytes, sp, mode, sid)
        if st != 0:
            raise RuntimeError("%s: %s" % (h.status_string(st), h.last_error()))

    # launches per step: projection or prologue, [tile selection,] attention, [output projection]
    nst = 3 if (proj or sparse) else 2
    seq_ids = (1, 2, 4) if sparse else (1, 2, 4) if proj else (1, 2)

    def step_launch(i=None):
        for k_, sid in enumerate(seq_ids):
            stage(sid)
            if i is not None:
                ev[i][k_ + 1].record(stream)

    for _ in range(args.warmup):
        step_launch()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step_launch(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev[0][0].elapsed_time(ev[K - 1][nst])
    pro_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    ai = 2 if sparse else 1                 # events bracketing the attention launch
    att_ms = [ev[i][ai].elapsed_time(ev[i][ai + 1]) for i in range(K)]
    ms_step = total_ms / K
    att_avg = float(np.mean(att_ms))
    pro_avg = float(np.mean(pro_ms))
    outp_avg = float(np.mean([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)])) if proj else 0.0
    sel_avg = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])) if sparse else 0.0
    step_ms = [ev[i][0].elapsed_time(ev[i][nst]) for i in range(K)]
    # the output of the last timed step, kept for the parity figures (the dense
    # attention run after the block-sparse one writes `out`)
    out_final = out.clone() if sparse else out
    copy_gbps = device_copy_rate(torch, dev)        # after the timed region
    ceiling = mfma_ceiling(torch, h, dev, stream, path="mx" if w.fp4 else "q8" if w.quantized else "bf16")
    print("[bench] %d steps: %.3f ms/step (attention %.3f, %s %.3f), wall %.3f s" % (
        K, ms_step, att_avg, "projection" if proj else "prologue", pro_avg, wall), file=sys.stderr, flush=True)
    unfused = library_gemm_then_prologue(torch, h, w, x, wq, norm_w, rope, cu, ws, ws_bytes, stream) if proj else None
    if proj:
        unfused.update(library_out_proj(torch, w, out, w_o, gate, resid, stream))
    out_flops = 2.0 * w.N * w.H * w.d * w.model_dim if proj else 0.0
    attn_flops = w.flops()
    dense_att = None
    if sparse:
        attn_flops = sparse_flops(w, tiles.cpu().numpy())
        dense_att = dense_attention_ms(torch, h, w, params, ptrs, cu, out, ws, ws_bytes, stream)

    flops = attn_flops + w.proj_flops() + out_flops
    value = flops / (ms_step * 1e-3) / 1e12
    peak = (MI355X_FP4_DENSE_TFLOPS if w.fp4 else MI355X_FP8_DENSE_TFLOPS if w.quantized
            else MI355X_BF16_DENSE_TFLOPS)
    achieved = attn_flops / (att_avg * 1e-3) / 1e12
    kname = "mx" if w.fp4 else "q8" if w.quantized else "bf16"
    kernel_file = {"mx": "mx.hip", "q8": "q8.hip", "bf16": "attn_bf16.hip"}[kname]
    summary = "attn_%s_%s_pmc.md" % (kname, w.name)
    traffic = measured_traffic(kernel_file, summary)
    N, H, d = w.N, w.H, w.d
    if w.fp4:
        # pass 1 reads q, k and the table and writes FP4 q; pass 3 re-reads k, v and
        # the table and writes FP4 k and v; one scale byte per 32 values
        pro_bytes = 4 * N * H * d * 2 + 2 * N * (d // 2) * 8 + 3 * N * H * d // 2 + 3 * N * H * d // 32
        metric = ("attention TFLOP/s (MXFP4 QK and PV) and %% of fp4 MFMA peak at N=%d packed tokens, "
                  "H=%d, d=%d" % (N, H, d))
    elif w.quantized and proj:
        # the projection reads x, W and the table and writes q8, fp32 khat and bf16 v;
        # pass 1 and pass 3 each read khat and v, pass 3 writes k8 and v8
        pro_bytes = (N * w.model_dim * 2 + 3 * H * d * w.model_dim * 2 + N * (d // 2) * 8
                     + N * H * d * (1 + 4 + 2) + 2 * N * H * d * (4 + 2) + 2 * N * H * d)
        metric = ("attention layer on the quantised path (QKV projection with the INT8/FP8 prologue, INT8/FP8 "
                  "attention, output projection with gated residual; D=%d) TFLOP/s at N=%d packed tokens, "
                  "H=%d, d=%d" % (w.model_dim, N, H, d))
    elif w.quantized:
        # pass 1 reads q, k, v and the table and writes q8; pass 3 re-reads k, v and the
        # table and writes k8 and v8 (per-tile scales and sums are negligible)
        pro_bytes = 5 * N * H * d * 2 + 3 * N * H * d + 2 * N * (d // 2) * 8
        metric = ("attention TFLOP/s (INT8 QK, FP8 PV) and %% of fp8 MFMA peak at N=%d packed tokens, "
                  "H=%d, d=%d" % (N, H, d))
    elif proj:
        # read x, W and the table; write qhat, khat and the transposed V copy
        pro_bytes = N * w.model_dim * 2 + 3 * H * d * w.model_dim * 2 + N * (d // 2) * 8 + 3 * N * H * d * 2
        metric = ("attention layer (QKV projection + RMSNorm/RoPE, attention, output projection with gated "
                  "residual; D=%d) TFLOP/s at N=%d packed tokens, H=%d, d=%d" % (w.model_dim, N, H, d))
    else:
        # read q, k, v and the table; write qhat, khat and the transposed V copy
        pro_bytes = 3 * N * H * d * 2 + 3 * N * H * d * 2 + N * (d // 2) * 8
        metric = METRIC if w.name == "joint" else (
            "attention TFLOP/s and %% of bf16 MFMA peak at N=%d packed tokens, H=%d, d=%d" % (N, H, d))
        if sparse:
            metric = ("block-sparse attention TFLOP/s of the computed (kept) work, %d of the 64-key tiles kept "
                      "per %d-row query block, at N=%d packed tokens, H=%d, d=%d" % (
                          w.keep_tiles, SPARSE_BLOCK_ROWS, N, H, d))
    res = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mx": "mxfp4", "q8": "int8/fp8", "bf16": "bf16"}[kname],
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": N, "heads": H,
                   "head_dim": d, "seq_lens": [s.n for s in w.seqs], "parallelism": "none"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": {"mx": "attn_mx_kernel", "q8": "attn_q8_kernel",
                                "bf16": "attn_bf16_pp_kernel<128, false>"}[kname],
                     "avg_ms": round(att_avg, 4)},
        # the attention kernel against 60% of its datasheet peak: the result is reported on every
        # run, met or not, with the kernel time that would meet it
        "perf_gate": {"target_frac": PERF_GATE_FRAC, "frac": round(achieved / peak, 4),
                      "met": bool(achieved >= PERF_GATE_FRAC * peak),
                      "attention_ms_at_target": round(attn_flops / (PERF_GATE_FRAC * peak * 1e12) * 1e3, 3)},
        # the same box's sustained matrix-core rate for this path's MFMA type, alone and with the
        # path's vector work beside it (h3attn_mfma_ceiling), beside the datasheet peak
        "measured_mfma_ceiling": None,
        "step_ms": {"p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p50": round(float(np.percentile(step_ms, 50)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "kernels": {"prologue_avg_ms": round(pro_avg, 4),
                    "prologue_GBps": round(pro_bytes / (pro_avg * 1e-3) / 1e9, 1),
                    "prologue_hbm_frac": round(pro_bytes / (pro_avg * 1e-3) / 1e9 / MI355X_HBM_GBPS, 4),
                    "device_copy_GBps": round(copy_gbps, 1),
                    "prologue_copy_frac": round(pro_bytes / (pro_avg * 1e-3) / 1e9 / copy_gbps, 4),
                    "attention_avg_ms": round(att_avg, 4)},
        "cpu_baseline": None,
    }
    if ceiling is not None:
        for key in list(ceiling):
            ceiling["attention_frac_of_" + key.rsplit("_", 1)[0]] = round(achieved / ceiling[key], 4)
        res["measured_mfma_ceiling"] = ceiling
    if sparse:
        res["kernels"].update({
            "selection_avg_ms": round(sel_avg, 4),
            "kept_fraction": round(attn_flops / w.flops(), 4),
            "dense_attention_ms": round(dense_att, 4),
            "speedup_vs_dense_step": round((pro_avg + dense_att) / ms_step, 3)})
        res["roofline"]["kernel"] = "attn_bf16_pp_kernel<128, true>"
        res["roofline"]["traffic"] = None
        res["config"]["keep_tiles"] = w.keep_tiles
    if proj:
        pf = w.proj_flops() / (pro_avg * 1e-3) / 1e12
        kern = res["kernels"]
        for key in ("prologue_avg_ms", "prologue_GBps", "prologue_hbm_frac", "prologue_copy_frac"):
            kern.pop(key)
        of = out_flops / (outp_avg * 1e-3) / 1e12
        kern.update({"projection_avg_ms": round(pro_avg, 4), "projection_TFLOPs": round(pf, 1),
                     "projection_frac": round(pf / MI355X_BF16_DENSE_TFLOPS, 4),
                     "projection_min_bytes": pro_bytes,
                     "out_proj_avg_ms": round(outp_avg, 4), "out_proj_TFLOPs": round(of, 1),
                     "out_proj_frac": round(of / MI355X_BF16_DENSE_TFLOPS, 4)})
        kern.update(unfused)
        res["config"]["model_dim"] = w.model_dim
    res["provenance"] = provenance(torch, h, w, inp)
    if not args.no_cpu_baseline:
        threads, host = oracle_threads()
        print("[bench] timing the CPU oracle on %d threads (%s)" % (threads, host), file=sys.stderr, flush=True)
        out_rows = out_final.view(torch.int16)

        def gpu_rows(toks, head):
            b = out_rows[torch.from_numpy(np.asarray(toks, dtype=np.int64)).to(dev), head].cpu().numpy()
            return (b.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

        def gpu_lists(head):
            nqb = (w.seqs[0].n + SPARSE_BLOCK_ROWS - 1) // SPARSE_BLOCK_ROWS
            return tiles[head * nqb:(head + 1) * nqb].cpu().numpy()

        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, threads, gpu_rows,
                                           gpu_lists if sparse else None)
        res["cpu_baseline"].update(host)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
