"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (elementwise, |gpu - oracle| <= atol + rtol*|oracle|): out 1e-3 /
1e-3, per-head lse 1e-4 / 1e-4; gather indices bit-exact; -inf lse and zero
output for instances with no unmasked cell.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import (LSE_ATOL, LSE_RTOL, OUT_ATOL, OUT_RTOL, assert_close, check,
                            run_batch, say, two_pass)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_q", [1])
def test_config0_tiny_single_step(n_q):
    say("case: config 0 (600 cells, 1 q), batch entry point")
    x = gen.make(0)
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what="cfg0")


@pytest.mark.parametrize("n_q", [1, 2, 3, 4])
def test_config1_pages_kernel_point(n_q):
    say(f"case: config 1 (2,051 cells), n_q={n_q}")
    x = gen.make(1).with_n_q(n_q)
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what=f"cfg1 nq{n_q}")


def wide_scales(x, seed, octaves=8):
    """K and V scales spread over 2^-octaves .. 2^octaves times their drawn
    values, independently per cell (rows of very different magnitudes)."""
    rng = np.random.default_rng(seed)
    def spread(bits):
        v = bits.view(np.float16).astype(np.float32)
        v = v * np.exp2(rng.uniform(-octaves, octaves, v.shape)).astype(np.float32)
        return v.astype(np.float16).view(np.uint16)
    return dataclasses.replace(x, k_scales=spread(x.k_scales), v_scales=spread(x.v_scales))


@pytest.mark.parametrize("n_q", [1, 4])
def test_wide_scale_range(n_q):
    """K and V scales spanning 2^16: each tile's probability digits are
    scaled by the row's largest p * v_scale, so the accuracy does not depend
    on how far apart the largest probability and the largest V scale are."""
    say(f"case: scales over 2^16, config 1, n_q={n_q}")
    x = wide_scales(gen.make(1).with_n_q(n_q), 40 + n_q)
    out, lse, g, _ = run_batch(x)
    # scores reach the hundreds here: lse to the relative bound only
    check(x, out, lse, g, what=f"wide scales nq{n_q}", strict_lse=False)
    o2, l2, g2, _ = two_pass(x, 256)
    check(x, o2, l2, g2, what=f"wide scales nq{n_q}, two passes at chunk 256", strict_lse=False)


@pytest.mark.parametrize("cfg", [0, 1])
def test_interleaved_scales(cfg):
    """(K, V) scale pairs interleaved per cell (scale_stride 2) give the
    same result as two scale arrays, bit for bit, and match the oracle."""
    say(f"case: interleaved scales, config {cfg}")
    x = gen.make(cfg)
    o1, l1, g1, _ = run_batch(x)
    o2, l2, g2, _ = run_batch(x, interleave=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(g1, g2)
    check(x, o2, l2, g2, what=f"cfg{cfg} interleaved")


@pytest.mark.parametrize("n_q", [1, 4])
def test_step_entry_matches_batch(n_q):
    """sda_decode_attn_step on one sequence equals the batch entry bit for bit."""
    import torch
    from decode_attention_sparse_amd import api
    say(f"case: step entry, config 1, n_q={n_q}")
    x = gen.make(1).with_n_q(n_q)
    out_b, lse_b, g_b, _ = run_batch(x)
    pool, dev = api.to_device(x)
    out = torch.empty(x.q.shape[1:], device="cuda")
    lse = torch.empty(x.q.shape[1:3], device="cuda")
    g = torch.empty(x.sel.shape[1], dtype=torch.int32, device="cuda")
    api.decode_attn_step(pool, dev["page_table"][0], dev["sel"][0], dev["q"][0], x.softmax_scale,
                         x.chunk, out, lse, gather_out=g)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out_b[0])
    assert np.array_equal(lse.cpu().numpy(), lse_b[0])
    assert np.array_equal(g.cpu().numpy(), g_b[0])


def check_partials(x, ws, chunk, what):
    from decode_attention_sparse_amd import api
    acc, m, l = (t.cpu().numpy() for t in api.partials(ws, x.n_inst, x.n_q, x.n_qheads,
                                                       x.sel.shape[1], chunk))
    racc, rm, rl = oracle.chunk_partials(x, chunk)
    assert racc.shape[1] == acc.shape[1]
    assert_close(m, rm, LSE_ATOL, LSE_RTOL, f"{what} partial m")
    assert_close(l, rl, 0, 1e-3, f"{what} partial l")
    assert_close(acc / l[..., None], racc / rl[..., None], OUT_ATOL, OUT_RTOL, f"{what} partial acc/l")


@pytest.mark.parametrize("cfg,n_q", [(0, 1), (1, 4), (1, 2)])
def test_chunk_partials(cfg, n_q):
    """The partials (acc, m, l) against the oracle's: those sda_chunk_batch
    leaves for the caller's chunk size, and those the fused call leaves for
    the finer chunk it runs (sda_fused_chunk_cells)."""
    import torch
    from decode_attention_sparse_amd import api
    say(f"case: partials, config {cfg}, n_q={n_q}")
    x = gen.make(cfg).with_n_q(n_q)
    max_sel = int(x.sel.shape[1])
    pool, dev = api.to_device(x)
    ws = api.workspace(x.n_inst, n_q, x.n_qheads, max_sel, x.chunk)
    api.chunk_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], max_sel, dev["q"],
                    x.softmax_scale, x.chunk, ws)
    torch.cuda.synchronize()
    check_partials(x, ws, x.chunk, "chunk pass")
    fc = api.fused_chunk_cells(x.n_inst, max_sel, x.chunk)
    assert fc == 64  # one instance: the fused call runs 64-cell chunks
    _, _, _, ws2 = run_batch(x)
    check_partials(x, ws2, fc, "fused call")


EDGE_COUNTS = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("chunk", [64, 256])
@pytest.mark.parametrize("n_q", [1, 2, 3, 4])
def test_edge_counts(n_q, chunk):
    """The pages' 0/1/2/3/63/64/65 selected-cell cases plus chunk edges, one
    instance per count in one batched call (device n_sel per instance)."""
    say(f"case: edge counts {EDGE_COUNTS}, n_q={n_q}, chunk={chunk}")
    k = len(EDGE_COUNTS)
    x = gen.make(None, seed=77 + n_q, n_inst=k, n_q=n_q, pool_cells=1024, n_sel=257,
                 sel="uniform", chunk=chunk)
    x = dataclasses.replace(x, n_sel=np.array(EDGE_COUNTS, np.int32))
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what=f"edges nq{n_q} C{chunk}")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("n_q", [1, 4])
def test_edge_counts_large_grid(n_q):
    """The edge counts again, inside a grid of more than 256 workgroups
    (64-cell chunks; the filler instances use the full count), so that they
    run alongside full chunks on a busy chip."""
    say(f"case: edge counts in a large grid, n_q={n_q}")
    k = 64
    counts = np.full(k, 257, np.int32)
    counts[: len(EDGE_COUNTS)] = EDGE_COUNTS
    x = gen.make(None, seed=91 + n_q, n_inst=k, n_q=n_q, pool_cells=1024, n_sel=257,
                 sel="uniform", chunk=64)
    x = dataclasses.replace(x, n_sel=counts)
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what=f"edges large grid nq{n_q}")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("n_q", [2, 4])
def test_batch_size_independence(n_q):
    """The chunk pass and merge at a given chunk size do not depend on the
    batch: the same instances run in a small grid and in larger ones (which
    the library launches differently: one-tile workgroups, one per 16-row
    group in the smallest grids and one per (instance, chunk) above that,
    the V accumulation split over two waves per row group in small grids,
    several chunks per workgroup in large ones); every instance gets the
    same arithmetic in the same order, so outputs and gather indices agree
    bit for bit.  The fused call chooses its chunk size from the grid
    (sda_fused_chunk_cells), so it is checked against the oracle."""
    say(f"case: batch-size independence, n_q={n_q}")
    spec = dict(n_q=n_q, pool_cells=2048, n_sel=600, sel="uniform", chunk=64)
    tiny = gen.make(None, seed=123, n_inst=5, **spec)     # 5 x 10 chunks: a workgroup per row group
    small = gen.make(None, seed=123, n_inst=20, **spec)   # 20 x 10 chunks
    large = gen.make(None, seed=123, n_inst=30, **spec)   # 30 x 10 chunks
    huge = gen.make(None, seed=123, n_inst=120, **spec)   # 120 x 10: two chunks per workgroup
    assert np.array_equal(small.sel, large.sel[:20]) and np.array_equal(small.q, large.q[:20])
    assert np.array_equal(tiny.sel, small.sel[:5]) and np.array_equal(tiny.q, small.q[:5])
    o0, l0, g0, _ = two_pass(tiny, 64)
    o1, l1, g1, _ = two_pass(small, 64)
    o2, l2, g2, _ = two_pass(large, 64)
    o3, l3, g3, _ = two_pass(huge, 64)
    assert np.array_equal(o0, o1[:5]) and np.array_equal(l0, l1[:5])
    assert np.array_equal(g0, g1[:5])
    for o, l, g_ in ((o2, l2, g2), (o3, l3, g3)):
        assert np.array_equal(o1, o[:20]) and np.array_equal(l1, l[:20])
        assert np.array_equal(g1, g_[:20])
    check(large, o2, l2, g2, inst_ids=[0, 19, 29], what="batch of 30")
    o4, l4, g4, _ = run_batch(huge)
    check(huge, o4, l4, g4, inst_ids=[0, 19, 77, 119], what="fused call, batch of 120")


@pytest.mark.parametrize("n_q,n_qheads", [(1, 12), (1, 17), (2, 12), (1, 33), (4, 12), (4, 16)])
def test_single_tile_forms_bitwise(n_q, n_qheads):
    """One-tile chunks run in three forms, chosen by the grid: a workgroup
    per (instance, chunk, 16-row group) in the smallest grids, all row
    groups in one workgroup up to one workgroup per CU, and the pipelined
    kernel beyond; with a single 16-row group its two waves share the
    scoring through LDS.  The same instances through each form give the
    same outputs, log-sum-exps and gather indices bit for bit (row counts
    12 to 64, one to four row groups), and the smallest grid matches the
    oracle."""
    say(f"case: single-tile forms, n_q={n_q}, n_qheads={n_qheads}")
    spec = dict(n_q=n_q, n_qheads=n_qheads, pool_cells=1024, n_sel=600, sel="uniform", chunk=64)
    res = []
    for n_inst in (2, 25, 60):  # 20, 250 and 600 (instance, chunk) pairs
        x = gen.make(None, seed=311, n_inst=n_inst, **spec)
        res.append((x, two_pass(x, 64)))
    x0, (o0, l0, g0, _) = res[0]
    for x, (o, l, g_, _) in res[1:]:
        assert np.array_equal(x0.sel, x.sel[:2]) and np.array_equal(x0.q, x.q[:2])
        assert np.array_equal(o0, o[:2]) and np.array_equal(l0, l[:2])
        assert np.array_equal(g0, g_[:2])
    check(x0, o0, l0, g0, what=f"single-tile forms R={n_q * n_qheads}")


@pytest.mark.parametrize("n_q", [1, 4])
def test_merge_of_many_chunks(n_q):
    """Rows with far more chunk partials than the merge requests at once
    (up to 48): sda_chunk_batch + sda_merge_batch at chunk 64 over
    12,800-cell lists (200 chunks: several batches per wave, and the maximum
    over chunk maxima past 64 chunks), a ragged second instance (3,001 cells,
    47 chunks) and a third with 65 chunks, against the oracle."""
    say(f"case: merge of 200 chunks, n_q={n_q}")
    x = gen.make(None, seed=77 + n_q, n_inst=3, n_q=n_q, pool_cells=16384, n_sel=12800,
                 sel="uniform", chunk=64)
    x = dataclasses.replace(x, n_sel=np.array([12800, 3001, 4097], np.int32))
    out, lse, g, _ = two_pass(x, 64)
    check(x, out, lse, g, what=f"200-chunk merge nq{n_q}")


def test_many_instances_coarse_chunks():
    """More than 256 instances and 512 (instance, chunk) pairs: the fused
    call takes chunks k times the caller's (300 x 600 cells at chunk 64:
    3,000 pairs, k = 5, 320-cell chunks).  Against the oracle on sampled
    instances, and bit for bit against the two passes at that chunk size."""
    from decode_attention_sparse_amd import api
    say("case: 300 instances, coarse fused chunks")
    x = gen.make(None, seed=61, n_inst=300, n_q=2, pool_cells=1024, n_sel=600, sel="uniform",
                 chunk=64)
    rng = np.random.default_rng(62)
    counts = rng.integers(0, 601, size=300).astype(np.int32)
    counts[[0, 1, 2]] = [600, 0, 321]
    x = dataclasses.replace(x, n_sel=counts)
    fc = api.fused_chunk_cells(300, 600, 64)
    assert fc == 320
    out, lse, g, _ = run_batch(x)
    ids = [0, 1, 2, 150, 299]
    check(x, out, lse, g, inst_ids=ids, what="coarse fused chunks")
    o2, l2, g2, _ = two_pass(x, fc)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2) and np.array_equal(g, g2)


def test_several_chunks_per_workgroup():
    """A grid of 1,600 chunks, so that each workgroup streams several
    consecutive chunks of one instance; ragged per-instance counts put chunk
    ends and instance ends at every position.  Outputs and every chunk's
    partial are checked on sampled instances."""
    from decode_attention_sparse_amd import api
    say("case: several chunks per workgroup")
    x = gen.make(None, seed=31, n_inst=200, n_q=2, pool_cells=1024, n_sel=512, sel="uniform",
                 chunk=64)
    rng = np.random.default_rng(8)
    counts = rng.integers(0, 513, size=200).astype(np.int32)
    counts[[0, 1, 2, 3]] = [512, 0, 65, 449]
    x = dataclasses.replace(x, n_sel=counts)
    ids = [0, 1, 2, 3, 57, 128, 199]
    out, lse, g, ws = two_pass(x, 64)  # the caller's chunk: three chunks per workgroup
    check(x, out, lse, g, inst_ids=ids, what="chunks per workgroup")
    acc, m, l = (t.cpu().numpy() for t in api.partials(ws, 200, 2, 12, 512, 64))
    racc, rm, rl = oracle.chunk_partials(x, 64, 8, inst_ids=ids)
    for k, i in enumerate(ids):
        nch = -(-int(counts[i]) // 64)
        assert_close(m[i, :nch], rm[k, :nch], LSE_ATOL, LSE_RTOL, f"partial m inst {i}")
        assert_close(l[i, :nch], rl[k, :nch], 0, 1e-3, f"partial l inst {i}")
        assert_close(acc[i, :nch] / l[i, :nch, :, None], racc[k, :nch] / rl[k, :nch, :, None],
                     OUT_ATOL, OUT_RTOL, f"partial acc/l inst {i}")


def test_two_row_groups_paired_chunks():
    """Two 16-row groups with one chunk per workgroup run as pairs of chunks
    in one workgroup of two pipelines: an odd chunk count (the last pair's
    second chunk past the list) and ragged counts (instances ending in either
    chunk of a pair, or before the pair).  Every chunk's partial and the
    outputs against the oracle on sampled instances."""
    from decode_attention_sparse_amd import api
    say("case: paired chunks, 24 rows")
    x = gen.make(None, seed=47, n_inst=100, n_q=2, pool_cells=1024, n_sel=320, sel="uniform",
                 chunk=64)
    rng = np.random.default_rng(48)
    counts = rng.integers(0, 321, size=100).astype(np.int32)
    counts[[0, 1, 2, 3, 4, 5]] = [320, 0, 64, 65, 129, 257]
    x = dataclasses.replace(x, n_sel=counts)
    ids = [0, 1, 2, 3, 4, 5, 33, 99]
    out, lse, g, ws = two_pass(x, 64)  # 5 chunks: 3 workgroups per instance
    check(x, out, lse, g, inst_ids=ids, what="paired chunks")
    acc, m, l = (t.cpu().numpy() for t in api.partials(ws, 100, 2, 12, 320, 64))
    racc, rm, rl = oracle.chunk_partials(x, 64, 8, inst_ids=ids)
    for k, i in enumerate(ids):
        nch = -(-int(counts[i]) // 64)
        assert_close(m[i, :nch], rm[k, :nch], LSE_ATOL, LSE_RTOL, f"partial m inst {i}")
        assert_close(l[i, :nch], rl[k, :nch], 0, 1e-3, f"partial l inst {i}")
        assert_close(acc[i, :nch] / l[i, :nch, :, None], racc[k, :nch] / rl[k, :nch, :, None],
                     OUT_ATOL, OUT_RTOL, f"partial acc/l inst {i}")


@pytest.mark.parametrize("n_q", [1, 4])
def test_small_grid_large_page_table(n_q):
    """A small (latency-bound) grid whose page table is too large to be read
    into LDS (8,192 pages), with masked and out-of-range entries."""
    say(f"case: small grid, 8,192-page table, n_q={n_q}")
    x = gen.make(None, seed=41 + n_q, n_inst=2, n_q=n_q, pool_cells=131072, n_sel=700,
                 sel="uniform", chunk=256)
    pt = x.page_table.copy()
    pt[0, ::5] = -1
    pt[1, 7] = 10**8
    x = dataclasses.replace(x, page_table=pt)
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what=f"large table nq{n_q}")


def test_masking():
    """Page -1 masking, page ids past the pool, selected ids past the logical
    range, and an instance whose every page is masked."""
    say("case: masking")
    x = gen.make(None, seed=5, n_inst=4, n_q=3, pool_cells=2048, n_sel=300, sel="uniform",
                 chunk=128)
    pt = x.page_table.copy()
    sel = x.sel.copy()
    pt[0, ::3] = -1
    pt[1, 5:40] = -1
    pt[1, 50] = x.n_phys_pages + 3
    pt[2, :] = -1
    sel[3, ::7] = 2048 + 11       # past the logical range
    sel[3, 1] = -5
    x = dataclasses.replace(x, page_table=pt, sel=sel)
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what="masking")
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.all(g[2] == -1) and g[3, 0] == -1 and g[3, 1] == -1


def test_ragged_batch_and_unsorted():
    """Per-instance counts below max_sel (read on the device), unsorted
    selections and duplicate entries."""
    say("case: ragged batch")
    x = gen.make(None, seed=9, n_inst=6, n_q=4, pool_cells=4096, n_sel=700, sel="uniform",
                 chunk=256)
    rng = np.random.default_rng(3)
    sel = x.sel.copy()
    sel[1] = sel[1, rng.permutation(700)]
    sel[2, 100:200] = sel[2, 0:100]  # duplicates
    x = dataclasses.replace(x, sel=sel, n_sel=np.array([700, 511, 700, 1, 0, 257], np.int32))
    out, lse, g, _ = run_batch(x)
    check(x, out, lse, g, what="ragged")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_configs(cfg):
    """The batched workloads at full size, in the launch configuration the
    bench times (interleaved scale pairs); every instance against the oracle,
    every gather index bit-exact.  The heavy-tailed K scales of the batched
    decode workload put |lse| between about 800 and 2,300, where float32
    itself misses an absolute 1e-4: its lse keeps the relative bound."""
    say(f"case: config {cfg} full size, oracle on every instance")
    x = gen.make(cfg)
    out, lse, g, _ = run_batch(x, interleave=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    check(x, out, lse, g, what=f"cfg{cfg} ({x.n_inst} instances)", strict_lse=cfg != 2)


@pytest.mark.parametrize("cfg,n_q,n_inst", [(1, 4, None), (1, 1, 8), (2, 4, None)])
def test_batch_entry_equals_two_passes(cfg, n_q, n_inst):
    """sda_decode_attn_batch equals sda_chunk_batch followed by
    sda_merge_batch at the chunk size the fused call uses, bit for bit (the
    partials in the workspace included, where the call runs the merge pass),
    and the two passes at the caller's chunk size up to rounding."""
    import torch
    from decode_attention_sparse_amd import api
    say(f"case: batch entry vs the two passes, config {cfg}, n_q={n_q}, n_inst={n_inst}")
    x = gen.make(cfg, **({} if n_inst is None else {"n_inst": n_inst})).with_n_q(n_q)
    n_inst, _, nh, D = x.q.shape
    max_sel = int(x.sel.shape[1])
    fc = api.fused_chunk_cells(n_inst, max_sel, x.chunk)
    say(f"  fused chunk {fc} (caller's {x.chunk})")
    out1, lse1, _, ws1 = run_batch(x, gather=False)
    pool, dev = api.to_device(x)

    def two_pass(chunk):
        ws2 = api.workspace(n_inst, n_q, nh, max_sel, x.chunk)
        out2 = torch.empty((n_inst, n_q, nh, D), device="cuda")
        lse2 = torch.empty((n_inst, n_q, nh), device="cuda")
        api.chunk_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], max_sel, dev["q"],
                        x.softmax_scale, chunk, ws2)
        api.merge_batch(dev["n_sel"], max_sel, chunk, ws2, out2, lse2)
        torch.cuda.synchronize()
        return out2.cpu().numpy(), lse2.cpu().numpy(), ws2

    out2, lse2, ws2 = two_pass(fc)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
    if not api.fused_single_launch(n_inst, n_q, nh, max_sel, x.chunk):  # else no partials
        for a1, a2 in zip(api.partials(ws1, n_inst, n_q, nh, max_sel, fc),
                          api.partials(ws2, n_inst, n_q, nh, max_sel, fc)):
            assert torch.equal(a1, a2)
    if fc != x.chunk:
        out3, lse3, _ = two_pass(x.chunk)
        assert_close(out1, out3, OUT_ATOL, OUT_RTOL, "fused vs caller's chunk out")
        assert_close(lse1, lse3, LSE_ATOL, LSE_RTOL, "fused vs caller's chunk lse")


def test_workspace_sentinel():
    """Bytes past the contracted workspace size stay untouched."""
    import torch
    from decode_attention_sparse_amd import api
    say("case: workspace sentinel")
    x = gen.make(1).with_n_q(3)
    pool, dev = api.to_device(x)
    nb = api.workspace_bytes(1, 3, 12, 2051, 256)
    ws = torch.full((nb + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 3, 12, 256), device="cuda")
    lse = torch.empty((1, 3, 12), device="cuda")
    api.decode_attn_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], 2051, dev["q"],
                          x.softmax_scale, 256, out, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(ws[nb:] == 0xA5).item()


def test_graph_replay_changing_counts():
    """The batch call captured in a HIP graph and replayed with new device
    counts and query values; every replay equals the eager call bit for bit."""
    import torch
    from decode_attention_sparse_amd import api
    say("case: graph replay")
    x = gen.make(None, seed=11, n_inst=8, n_q=4, pool_cells=8192, n_sel=1500, sel="uniform",
                 chunk=256)
    pool, dev = api.to_device(x)
    out = torch.empty(x.q.shape, device="cuda")
    lse = torch.empty(x.q.shape[:3], device="cuda")
    ws = api.workspace(8, 4, 12, 1500, 256)
    args = lambda: (pool, dev["page_table"], dev["sel"], dev["n_sel"], 1500, dev["q"],
                    x.softmax_scale, 256, out, lse)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.decode_attn_batch(*args(), ws=ws)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.decode_attn_batch(*args(), ws=ws)
    rng = np.random.default_rng(0)
    for rep in range(4):
        counts = rng.integers(0, 1501, size=8).astype(np.int32)
        counts[rep % 8] = 0
        dev["n_sel"].copy_(torch.from_numpy(counts))
        dev["q"].copy_(torch.from_numpy(rng.standard_normal(x.q.shape, dtype=np.float32)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_lse = out.clone(), lse.clone()
        api.decode_attn_batch(*args(), ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(g_out, out) and torch.equal(g_lse, lse), f"replay {rep}"
        y = dataclasses.replace(x, n_sel=counts, q=dev["q"].cpu().numpy())
        check(y, out.cpu().numpy(), lse.cpu().numpy(), what=f"replay {rep}")
