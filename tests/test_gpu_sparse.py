"""GPU parity of the block-sparse attention (h3attn_fwd_sparse_stages).

- Every tile kept: the sparse kernel visits the same tiles in the same order
  as the dense one, so its output is bit-identical to h3attn_fwd (and meets
  the oracle's bf16 gates).
- Caller lists (the oracle's inputs, from a seeded generator): random subsets
  of tiles per (sequence, head, 256-row query block), in random order, including the
  sequence's partial last tile, compared on every row with the oracle's
  softmax over exactly the kept keys.
- Selection: the tiles the GPU keeps against the oracle's pooled-score top-k.
  The GPU scores in fp32 and the oracle in fp64 from the same stored bf16
  values, so a tile may differ only where the oracle's scores of the two
  tiles involved are within 1e-3 relative of each other (a near tie); the
  attention over the GPU's selection is then checked on the rows whose lists
  agree.
- The 125,242-token joint shape with 25% of the tiles kept, on two heads.
- The longest sequence the path accepts (131,072 tokens, 2,048 tiles) with
  every tile selected: lists of the maximum length, bit-identical to dense.
"""
import numpy as np
import pytest

import oracle
from audio_diffusion_transformer_amd import h3attn as h
from audio_diffusion_transformer_amd import synth
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu
B = oracle.SPARSE_BLOCK            # query rows per tile list
Seq = synth.Seq

SMALL = {
    "sparse_ragged": synth.Workload("sparse_ragged", H=2, d=128, seqs=(Seq(3, 10, 11, 7), Seq(0, 1, 1), Seq(1, 4, 5, 70)),
                                    split=(32, 48, 48), k_offset_std=0.5, seed=51),
    "sparse_long_d64": synth.Workload("sparse_long_d64", H=2, d=64, seqs=(Seq(5, 16, 20, 33),), split=(16, 24, 24),
                                      seed=52),
}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _run_sparse(torch, w, t, tpb, tiles=None, select=True, label=""):
    G.announce("sparse %s N=%d H=%d d=%d tiles_per_block=%d select=%s" % (label, w.N, w.H, w.d, tpb, select))
    bt = None if tiles is None else torch.from_numpy(np.ascontiguousarray(tiles, dtype=np.int32)).to("cuda:0")
    out, bt = h.h3attn_fwd_sparse(t["q"], t["k"], t["v"], t["norm_w"], t["rope"], t["cu"], tpb, block_tiles=bt,
                                  select=select, eps=w.eps)
    torch.cuda.synchronize()
    return G.bits(out), bt.cpu().numpy()


def _random_lists(w, tpb, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for s in w.seqs:
        n = s.n
        nt = (n + 63) // 64
        for _ in range(w.H):
            for _ in range((n + B - 1) // B):
                L = min(tpb, nt)
                pick = rng.choice(nt, L, replace=False)
                if nt - 1 not in pick and L > 1 and rng.random() < 0.5:
                    pick[rng.integers(L)] = nt - 1           # often include the partial last tile
                row = np.full(tpb, -1, dtype=np.int32)
                row[:L] = pick                                # random order
                rows.append(row)
    return np.stack(rows) if rows else np.zeros((0, tpb), np.int32)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_all_tiles_kept_is_dense_attention(torch_dev, name):
    w = SMALL[name]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    dense = G.bits(G.run(w, t, label=name + " dense"))
    nt_max = max((s.n + 63) // 64 for s in w.seqs)
    items = h.sparse_items(inp["cu_seqlens"], w.H)
    tiles = np.tile(np.arange(nt_max, dtype=np.int32), (items, 1))
    got, _ = _run_sparse(torch_dev, w, t, nt_max, tiles=tiles, select=False, label=name + " all tiles")
    assert np.array_equal(got, dense)
    rows = np.arange(w.N * w.H, dtype=np.int64)
    ref = oracle.Problem.from_workload(w, inp).attention_rows(rows, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), ref), G.BF16_GATE, name + " all tiles")


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("tpb", [1, 3])
def test_caller_lists_all_rows(torch_dev, name, tpb):
    w = SMALL[name]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    tiles = _random_lists(w, tpb, seed=tpb * 100 + len(name))
    got, _ = _run_sparse(torch_dev, w, t, tpb, tiles=tiles, select=False, label="%s caller lists" % name)
    rows = np.arange(w.N * w.H, dtype=np.int64)
    ref = oracle.Problem.from_workload(w, inp).sparse_attention_rows(rows, tiles, tpb, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), ref), G.BF16_GATE, "%s tpb=%d" % (name, tpb))


def _compare_selection(gpu, ref, scores, label):
    """Identical lists except near ties; returns the mask of items whose lists agree."""
    same = np.all(gpu == ref, axis=1)
    for i in np.nonzero(~same)[0]:
        g = set(int(x) for x in gpu[i] if x >= 0)
        r = set(int(x) for x in ref[i] if x >= 0)
        assert len(g) == len(r), "%s item %d: %d tiles against %d" % (label, i, len(g), len(r))
        sc = scores[i]
        worst_kept = min(sc[t] for t in r)
        for t in g - r:                       # the GPU kept t, the oracle a tile scoring at least as well
            assert sc[t] >= worst_kept - 1e-3 * max(abs(worst_kept), 1e-30), \
                "%s item %d: tile %d (score %.6g) kept, oracle's k-th score %.6g" % (label, i, t, sc[t], worst_kept)
    assert same.mean() > 0.9, "%s: only %.3f of the lists agree" % (label, same.mean())
    return same


@pytest.mark.parametrize("name", sorted(SMALL))
def test_selection_and_attention_over_it(torch_dev, name):
    w = SMALL[name]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    tpb = 2
    got, lists = _run_sparse(torch_dev, w, t, tpb, select=True, label=name + " select")
    p = oracle.Problem.from_workload(w, inp)
    ref_lists, scores = p.sparse_select(tpb)
    same = _compare_selection(lists, ref_lists, scores, name)
    items = p.sparse_items()
    rows = np.array([tok * w.H + hh for i, (s, hh, qb) in enumerate(items) if same[i]
                     for tok in range(int(p.cu[s]) + B * qb, min(int(p.cu[s]) + B * qb + B, int(p.cu[s + 1])))],
                    dtype=np.int64)
    ref = p.sparse_attention_rows(rows, ref_lists, tpb, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), ref), G.BF16_GATE, name + " selected")


def test_full_size_two_heads(torch_dev):
    w = synth.WORKLOADS["sparse_joint"]
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    got, lists = _run_sparse(torch_dev, w, t, w.keep_tiles, select=True, label="sparse_joint")
    del t
    heads = [3, 17]
    sub = {key: np.ascontiguousarray(inp[key][:, heads]) for key in ("q", "k", "v")}
    sub["norm_w"] = np.ascontiguousarray(inp["norm_w"][:, heads])
    ws = w.replace(H=len(heads))
    p = oracle.Problem.from_workload(ws, sub)
    ref_lists, scores = p.sparse_select(w.keep_tiles)
    nqb = (w.N + B - 1) // B
    gl = np.concatenate([lists[hh * nqb:(hh + 1) * nqb] for hh in heads])
    same = _compare_selection(gl, ref_lists, scores, "sparse_joint")
    rng = np.random.default_rng(12)
    items = np.nonzero(same)[0]
    pick = np.sort(rng.choice(items, 64, replace=False))
    rows = []
    for i in pick:
        j, qb = divmod(int(i), nqb)
        toks = rng.choice(np.arange(B * qb, min(B * qb + B, w.N)), 8, replace=False)
        rows += [int(tk) * len(heads) + j for tk in toks]
    rows = np.array(sorted(rows), dtype=np.int64)
    ref = p.sparse_attention_rows(rows, ref_lists, w.keep_tiles, nthreads=G.oracle_threads())
    tok, j = rows // len(heads), rows % len(heads)
    gotr = G.decode(got[tok, np.array(heads)[j]])
    G.check(G.metrics(gotr, ref), G.BF16_GATE, "sparse_joint sampled")


def test_full_size_ragged_two_heads(torch_dev):
    """The three-sequence ragged batch at full size (18,144 + 45,250 + 7,200
    tokens) with 177 tiles kept per block, so the last sequence keeps all of
    its 113 tiles: the GPU selection of two heads against the oracle's, then
    sampled rows of agreeing blocks against the oracle's softmax over the
    kept keys."""
    w = synth.WORKLOADS["ragged"].replace(name="sparse_ragged_full", keep_tiles=177)
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    got, lists = _run_sparse(torch_dev, w, t, w.keep_tiles, select=True, label=w.name)
    del t
    heads = [5, 19]
    sub = {key: np.ascontiguousarray(inp[key][:, heads]) for key in ("q", "k", "v")}
    sub["norm_w"] = np.ascontiguousarray(inp["norm_w"][:, heads])
    ws = w.replace(H=len(heads))
    p = oracle.Problem.from_workload(ws, sub)
    ref_lists, scores = p.sparse_select(w.keep_tiles)
    # the GPU's list rows run sequence by sequence, then over all H heads, then query block
    gpu_rows, base = [], 0
    for s in w.seqs:
        nqb = (s.n + B - 1) // B
        for hh in heads:
            gpu_rows += list(range(base + hh * nqb, base + (hh + 1) * nqb))
        base += w.H * nqb
    gl = lists[np.array(gpu_rows)]
    same = _compare_selection(gl, ref_lists, scores, w.name)
    items = p.sparse_items()                  # (sequence, head of the two, block), the order of gl
    rng = np.random.default_rng(13)
    pick = np.sort(rng.choice(np.nonzero(same)[0], 96, replace=False))
    rows = []
    for i in pick:
        s, j, qb = items[int(i)]
        lo = int(p.cu[s]) + B * qb
        hi = min(lo + B, int(p.cu[s + 1]))
        toks = rng.choice(np.arange(lo, hi), min(8, hi - lo), replace=False)
        rows += [int(tk) * len(heads) + j for tk in toks]
    rows = np.array(sorted(rows), dtype=np.int64)
    ref = p.sparse_attention_rows(rows, ref_lists, w.keep_tiles, nthreads=G.oracle_threads())
    tok, j = rows // len(heads), rows % len(heads)
    gotr = G.decode(got[tok, np.array(heads)[j]])
    G.check(G.metrics(gotr, ref), G.BF16_GATE, w.name + " sampled")


@pytest.mark.timeout(400)
def test_caller_lists_ragged_last_sequence_every_row(torch_dev):
    """Full-tensor evidence on the block-sparse path at a full-size workload:
    the three-sequence ragged batch runs whole with 40 seeded caller-given
    tiles per 256-row block, and every row of every head of its 7,200-token
    sequence (172,800 rows) is compared with the oracle's softmax over the
    listed keys."""
    w = synth.WORKLOADS["ragged"].replace(name="sparse_ragged_lists")
    tpb = 40
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    tiles = _random_lists(w, tpb, seed=41)
    got, _ = _run_sparse(torch_dev, w, t, tpb, tiles=tiles, select=False, label=w.name)
    del t
    cu = w.cu_seqlens().astype(np.int64)
    rows = (np.arange(cu[2], cu[3])[:, None] * w.H + np.arange(w.H)[None, :]).reshape(-1)
    G.announce("%s: oracle, %d rows" % (w.name, len(rows)))
    ref = oracle.Problem.from_workload(w, inp).sparse_attention_rows(rows, tiles, tpb, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), ref), G.BF16_GATE, w.name + " last sequence")


def test_longest_sequence_every_tile_selected(torch_dev):
    """The largest sequence the block-sparse path accepts: 131,072 tokens
    (32 x 64 x 64 video grid), i.e. 2,048 tiles, with 2,048 tiles per block,
    the list length's upper bound.  The selection has to keep every tile, so
    each list is 0..2047 in tile order, and the attention over it is the
    dense kernel's, bit for bit; sampled rows also against the oracle."""
    w = synth.Workload("sparse_longest", H=2, d=128, seqs=(Seq(32, 64, 64),), split=(32, 48, 48), seed=53)
    nt = w.N // 64
    assert w.N == 131072 and nt == 2048
    inp = synth.generate(w)
    t = G.to_device(inp, w)
    dense = G.bits(G.run(w, t, label=w.name + " dense"))
    got, lists = _run_sparse(torch_dev, w, t, nt, select=True, label=w.name)
    del t
    assert lists.shape == (h.sparse_items(inp["cu_seqlens"], w.H), nt)
    assert np.array_equal(lists, np.tile(np.arange(nt, dtype=np.int32), (lists.shape[0], 1)))
    assert np.array_equal(got, dense)
    rows = np.sort(np.random.default_rng(14).choice(w.N * w.H, 128, replace=False)).astype(np.int64)
    ref = oracle.Problem.from_workload(w, inp).attention_rows(rows, nthreads=G.oracle_threads())
    G.check(G.metrics(G.gpu_rows(got, rows, w.H), ref), G.BF16_GATE, w.name + " sampled")
