"""GPU parity of the QSA block scorer and top-k selection (through the C ABI)
against the oracle.

Scores: within a float32 bound of the oracle's fp64 scores (each lane sums
n_heads * idx_dim / 16 products with fmas, then four pairwise sums:
|error| <= 64 * 2^-24 * sum |q k| is a safe margin), -inf exactly where the
oracle has -inf.  Selection: the top-k decision is taken on the kernel's
fp32 scores, so the oracle's selection is run on those same scores and the
cell lists must be identical bit for bit; the selection must also be a
valid top-k of the oracle's own scores up to that bound (blocks whose fp64
scores are closer than the bound to the k-th may trade places)."""
import dataclasses
import zlib

import numpy as np
import pytest

import oracle
from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import check, say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def run_qsa(x, k_blocks=None, pad=0):
    """Scores and selection on the GPU: numpy scores [n_inst][n_rows][B],
    sel [n_inst][k R], n_sel [n_inst], plus the device sel and n_sel.  With
    pad > 0 the selection rows are pad entries longer than k R."""
    import torch
    from decode_attention_sparse_amd import api
    k = x.k_blocks if k_blocks is None else k_blocks
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pooled, dead, q, vis = t(x.pooled), t(x.dead), t(x.q_idx), t(x.n_visible)
    scores = torch.full((x.n_inst, x.n_rows, x.max_blocks), float("nan"), device="cuda")
    api.qsa_block_scores(pooled, dead, q, vis, x.block_cells, scores)
    stride = max(k * x.block_cells, 1) + pad
    sel = torch.full((x.n_inst, stride), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((x.n_inst,), -7, dtype=torch.int32, device="cuda")
    api.qsa_select(scores, vis, x.block_cells, k, sel, n_sel)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy(), sel, n_sel


def score_bound(x):
    """64 * 2^-24 * sum_h,d |q| |k| per (instance, row, block)."""
    a = np.abs(x.q_idx.astype(np.float64)).reshape(x.n_inst, x.n_rows, -1)
    b = np.abs(x.pooled.astype(np.float64)).reshape(x.n_inst, x.max_blocks, -1)
    return 64 * U32 * np.einsum("irk,ibk->irb", a, b) + 1e-30


def check_qsa(x, k_blocks=None, what="", pad=0):
    k = x.k_blocks if k_blocks is None else k_blocks
    got, sel, n_sel, _, _ = run_qsa(x, k, pad)
    for i in range(x.n_inst):
        assert (sel[i, n_sel[i]:] == -7).all(), f"{what}: instance {i} written past its list"
    ref = oracle.qsa_scores(x)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf pattern differs"
    assert np.isfinite(got[~ninf]).all(), f"{what}: non-finite scores"
    bound = score_bound(x)
    err = np.abs(got.astype(np.float64) - ref)[~ninf]
    assert np.all(err <= bound[~ninf]), f"{what}: score error {err.max():.3e}"
    # the selection on the kernel's own scores, bit for bit
    rsel, rn = oracle.qsa_select(got.astype(np.float64), x.n_visible, x.block_cells, k)
    assert np.array_equal(n_sel, rn), f"{what}: counts {n_sel[:4]} vs {rn[:4]}"
    for i in range(x.n_inst):
        assert np.array_equal(sel[i, :n_sel[i]], rsel[i, :rn[i]]), f"{what}: instance {i}"
    # and a valid top-k of the oracle's fp64 scores, up to the bound: a live
    # block always has a visible first cell, so the cell list names exactly
    # the selected blocks; a block left out may outscore a selected one only
    # by less than the two blocks' bounds together
    c = ref.max(axis=1)
    cb = np.where(ninf, 0, bound).max(axis=1)
    for i in range(x.n_inst):
        picked = np.unique(sel[i, :n_sel[i]] // x.block_cells)
        live = np.flatnonzero(c[i] > -np.inf)
        assert picked.size == min(k, live.size), f"{what}: instance {i}"
        rest = np.setdiff1d(live, picked)
        if picked.size and rest.size:
            assert np.max(c[i, rest] - cb[i, rest]) <= np.min(c[i, picked] + cb[i, picked]), \
                f"{what}: instance {i} is not a top-k of the oracle's scores"
    say(f"  {what}: max score error {err.max() if err.size else 0:.2e} "
        f"(bound {bound[~ninf].min() if err.size else 0:.1e}..), cells per instance "
        f"{n_sel.min()}..{n_sel.max()}")
    return got, sel, n_sel


def test_qsa_workload():
    """The bench workload: 64 instances x 512 blocks of 256 cells, 2 rows,
    4 x 128 indexer dims, top 64, a partial last block, 2 % dead blocks."""
    say("case: QSA scorer + top-k, 64 x 512 blocks of 256 cells, top 64")
    x = gen.make_qsa("qsa_select_64inst_128k_2q")
    _, _, n_sel = check_qsa(x, what="workload")
    assert n_sel.max() == 64 * 256


GEOMS = {
    # name: (make_qsa overrides, k)
    "one_row_hd64_R16": (dict(n_inst=3, n_rows=1, n_heads=1, idx_dim=64, block_cells=16,
                              max_blocks=300, dead_frac=0.1), 17),
    "three_rows_hd192": (dict(n_inst=2, n_rows=3, n_heads=3, idx_dim=64, block_cells=64,
                              max_blocks=129, dead_frac=0.05), 40),
    "eight_rows_hd1024": (dict(n_inst=2, n_rows=8, n_heads=8, idx_dim=128, block_cells=32,
                               max_blocks=70, dead_frac=0.0), 9),
    "five_rows_hd256_R1024": (dict(n_inst=4, n_rows=5, n_heads=2, idx_dim=128,
                                   block_cells=1024, max_blocks=40, dead_frac=0.2), 7),
    "k_above_live": (dict(n_inst=2, n_rows=2, n_heads=1, idx_dim=128, block_cells=64,
                          max_blocks=50, dead_frac=0.5), 50),
    "k_zero": (dict(n_inst=2, n_rows=2, n_heads=1, idx_dim=64, block_cells=64, max_blocks=50),
               0),
    # 256 or more instances: one selection workgroup each (below that, up
    # to eight share an instance's writes, as in every other case here)
    "many_instances_one_group_each": (dict(n_inst=300, n_rows=2, n_heads=1, idx_dim=64,
                                           block_cells=16, max_blocks=40, dead_frac=0.1), 5),
    "max_blocks_16384": (dict(n_inst=2, n_rows=4, n_heads=1, idx_dim=64, block_cells=16,
                              max_blocks=16384, dead_frac=0.01), 4096),
}


@pytest.mark.parametrize("name", sorted(GEOMS))
def test_qsa_geometries(name):
    kw, k = GEOMS[name]
    say(f"case: QSA {name} {kw} k={k}")
    x = gen.make_qsa(None, seed=zlib.crc32(name.encode()) % 1000, **dict(kw, k_blocks=k))
    check_qsa(x, what=name)


@pytest.mark.parametrize("extent", [4096, 32768, 131072, 262144])
def test_qsa_live_extents(extent):
    """4K..256K live cells under one 256K capacity (1,024 blocks of 256
    cells), rows ending at different cells, so the dead tail starts in
    different blocks for different rows."""
    say(f"case: QSA live extent {extent} of 262,144")
    x = gen.make_qsa(None, seed=extent % 997, n_inst=3, n_rows=4, n_heads=4, idx_dim=64,
                     block_cells=256, max_blocks=1024, k_blocks=32, dead_frac=0.02,
                     context=[extent - 300, extent - 256, extent])
    check_qsa(x, what=f"extent {extent}")


@pytest.mark.parametrize("pad", [0, 1, 3])
def test_qsa_ragged_rows_and_strides(pad):
    """Lists whose rows start off a 16-byte boundary (row stride k R + pad)
    and extents that end inside a block at every remainder mod 4, so the
    cell lists are written both four cells per store and one at a time."""
    say(f"case: QSA ragged extents, selection row stride k R + {pad}")
    ctx = [4317, 4318, 4319, 4320, 4001]
    x = gen.make_qsa(None, seed=11 + pad, n_inst=5, n_rows=2, n_heads=2, idx_dim=64,
                     block_cells=48, max_blocks=90, k_blocks=12, dead_frac=0.05, context=ctx)
    # the block holding each instance's last visible cell live and on top
    pooled, dead = x.pooled.copy(), x.dead.copy()
    for i, c in enumerate(ctx):
        pooled[i, (c - 1) // 48] = 8 * x.q_idx[i, 0]
        dead[i, (c - 1) // 48] = 0
    x = dataclasses.replace(x, pooled=pooled, dead=dead)
    _, sel, n_sel = check_qsa(x, what=f"pad {pad}", pad=pad)
    assert list(n_sel % 4) == [1, 2, 3, 0, 1], n_sel


def test_qsa_equal_keys():
    """Every block has the same pooled key: all live scores tie and the
    lowest-numbered live blocks are taken (dead blocks skipped)."""
    say("case: QSA equal keys")
    x = gen.make_qsa(None, seed=5, n_inst=2, n_rows=3, n_heads=2, idx_dim=64, block_cells=64,
                     max_blocks=100, k_blocks=10, dead_frac=0.2)
    pooled = np.broadcast_to(x.pooled[:, :1], x.pooled.shape).copy()
    x = dataclasses.replace(x, pooled=pooled)
    _, sel, n_sel = check_qsa(x, what="equal keys")
    for i in range(x.n_inst):
        live = np.flatnonzero(x.dead[i] == 0)[:10]
        assert np.array_equal(np.unique(sel[i, :n_sel[i]] // 64), live)


def test_qsa_all_dead_and_empty_extent():
    """No live block: nothing is selected; an extent of 0 likewise."""
    say("case: QSA all dead / empty extent")
    x = gen.make_qsa(None, seed=6, n_inst=3, n_rows=2, n_heads=1, idx_dim=64, block_cells=32,
                     max_blocks=20, k_blocks=5, context=[640, 0, 640])
    dead = x.dead.copy()
    dead[0] = 1
    x = dataclasses.replace(x, dead=dead)
    _, _, n_sel = check_qsa(x, what="all dead")
    assert n_sel[0] == 0 and n_sel[1] == 0 and n_sel[2] == 5 * 32


def test_qsa_feeds_decode_attention():
    """End to end: scores, top-k and the decode attention over the selected
    cells, all on the GPU (the selection goes straight from sda_qsa_select to
    sda_decode_attn_batch); against the oracle's attention over the
    oracle's selection of the same scores."""
    import torch
    from decode_attention_sparse_amd import api
    n_inst, ctx, R, k = 8, 32768, 256, 16
    say(f"case: QSA select -> decode attention, {n_inst} x {ctx}-cell contexts, top {k} of "
        f"{ctx // R} blocks")
    xq = gen.make_qsa(None, seed=7, n_inst=n_inst, n_rows=2, n_heads=4, idx_dim=128,
                      block_cells=R, max_blocks=ctx // R, k_blocks=k, dead_frac=0.02,
                      context=ctx - 50)
    got, sel, n_sel, dsel, dn = run_qsa(xq)
    x = gen.make(None, seed=8, n_inst=n_inst, n_q=2, pool_cells=ctx, n_sel=k * R,
                 sel="uniform", chunk=512)
    pool, dev = api.to_device(x, interleave_scales=True)
    out = torch.full(x.q.shape, float("nan"), device="cuda")
    lse = torch.full(x.q.shape[:3], float("nan"), device="cuda")
    g = torch.full((n_inst, k * R), -7, dtype=torch.int32, device="cuda")
    api.decode_attn_batch(pool, dev["page_table"], dsel, dn, k * R, dev["q"], x.softmax_scale,
                          x.chunk, out, lse, gather_out=g)
    torch.cuda.synchronize()
    rsel, rn = oracle.qsa_select(got.astype(np.float64), xq.n_visible, R, k)
    assert np.array_equal(n_sel, rn)
    xs = dataclasses.replace(x, sel=rsel, n_sel=rn)
    check(xs, out.cpu().numpy(), lse.cpu().numpy(), g.cpu().numpy(), what="select -> decode")
