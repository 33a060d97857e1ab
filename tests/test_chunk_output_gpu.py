"""GPU parity of the fused calls that run as one chunk-kernel launch writing
the head outputs: every instance has one multi-tile chunk at the call's chunk
size, or two with 17 to 48 query rows (one workgroup per instance, two
gather pipelines, the two partials merged in LDS).  Each launch shape is
checked bit for bit against sda_chunk_batch + sda_merge_batch at that chunk
size, against the oracle on sampled instances, and for the workspace being
left alone."""
import dataclasses

import numpy as np
import pytest

from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import check, say, two_pass

pytestmark = pytest.mark.gpu

# name: (make overrides, expected fused chunk, expected chunks per instance)
CASES = {
    "pair_24_rows": (dict(n_inst=100, n_q=2, pool_cells=1024, n_sel=500, chunk=256), 256, 2),
    "pair_36_rows": (dict(n_inst=180, n_q=3, pool_cells=1024, n_sel=700, chunk=256), 384, 2),
    "pair_48_rows": (dict(n_inst=200, n_q=4, pool_cells=2048, n_sel=1000, chunk=256), 512, 2),
    "single_small_grid_12_rows": (dict(n_inst=200, n_q=1, pool_cells=1024, n_sel=250, chunk=256),
                                  256, 1),
    "single_small_grid_24_rows": (dict(n_inst=200, n_q=2, pool_cells=1024, n_sel=250, chunk=256),
                                  256, 1),
    "single_36_rows": (dict(n_inst=600, n_q=3, pool_cells=1024, n_sel=600, chunk=256), 768, 1),
    "single_64_rows": (dict(n_inst=520, n_q=4, n_qheads=16, pool_cells=1024, n_sel=600,
                            chunk=256), 768, 1),
}


def ragged_counts(seed, n_inst, max_sel, fc):
    """Counts in [0, max_sel] with the edge cases first: empty, one cell, tile
    and chunk boundaries, the maximum."""
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, max_sel + 1, size=n_inst).astype(np.int32)
    edges = [0, 1, 63, 64, 65, fc - 1, fc, fc + 1, max_sel]
    edges = [e for e in edges if 0 <= e <= max_sel]
    counts[: len(edges)] = edges
    return counts, len(edges)


@pytest.mark.parametrize("name", sorted(CASES))
def test_output_from_chunk_pass(name):
    import torch
    from decode_attention_sparse_amd import api
    kw, want_fc, want_nch = CASES[name]
    seed = 500 + sorted(CASES).index(name)
    say(f"case: chunk kernel writes the outputs, {name} {kw} seed={seed}")
    x = gen.make(None, seed=seed, sel="uniform", **kw)
    n_inst, n_q, nh, D = x.q.shape
    max_sel = int(x.sel.shape[1])
    fc = api.fused_chunk_cells(n_inst, max_sel, x.chunk)
    assert (fc, -(-max_sel // fc)) == (want_fc, want_nch)
    assert api.fused_single_launch(n_inst, n_q, nh, max_sel, x.chunk)
    counts, n_edges = ragged_counts(seed, n_inst, max_sel, fc)
    x = dataclasses.replace(x, n_sel=counts)

    pool, dev = api.to_device(x)
    nb = api.workspace_bytes(n_inst, n_q, nh, max_sel, x.chunk)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full((n_inst, n_q, nh, D), float("nan"), device="cuda")
    lse = torch.full((n_inst, n_q, nh), float("nan"), device="cuda")
    g = torch.full(x.sel.shape, -7, dtype=torch.int32, device="cuda")
    api.decode_attn_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], max_sel, dev["q"],
                          x.softmax_scale, x.chunk, out, lse, gather_out=g, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(ws == 0x5A).item(), "the workspace was written"
    out, lse, g = out.cpu().numpy(), lse.cpu().numpy(), g.cpu().numpy()

    o2, l2, g2, _ = two_pass(x, fc)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2), "differs from the two passes"
    assert np.array_equal(g, g2)
    ids = sorted(set(range(n_edges)) | {n_inst // 2, n_inst - 1})
    check(x, out, lse, g, inst_ids=ids, what=name)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))  # count 0


@pytest.mark.parametrize("n_inst,n_q,n_sel", [(64, 2, 3000), (100, 1, 500)])
def test_merge_pass_calls_write_the_workspace(n_inst, n_q, n_sel):
    """The converse of the rule: calls with more chunks, or two chunks of at
    most 16 rows, run the merge pass and leave their partials in the
    workspace."""
    import torch
    from decode_attention_sparse_amd import api
    say(f"case: a fused call with the merge pass writes the workspace, {n_inst} x {n_sel}, n_q={n_q}")
    x = gen.make(None, seed=520, n_inst=n_inst, n_q=n_q, pool_cells=4096, n_sel=n_sel,
                 sel="uniform", chunk=256)
    nh, D = x.q.shape[2:]
    assert not api.fused_single_launch(n_inst, n_q, nh, n_sel, 256)
    pool, dev = api.to_device(x)
    nb = api.workspace_bytes(n_inst, n_q, nh, n_sel, 256)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.empty((n_inst, n_q, nh, D), device="cuda")
    lse = torch.empty((n_inst, n_q, nh), device="cuda")
    api.decode_attn_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], n_sel, dev["q"],
                          x.softmax_scale, 256, out, lse, ws=ws)
    torch.cuda.synchronize()
    assert not torch.all(ws == 0x5A).item()
    check(x, out.cpu().numpy(), lse.cpu().numpy(), inst_ids=[0, n_inst - 1],
          what="merge pass call")


def test_graph_replay_two_pipelines():
    """The two-pipeline launch captured in a HIP graph and replayed with new
    device counts and queries; every replay equals the eager call bit for
    bit and matches the oracle on sampled instances."""
    import torch
    from decode_attention_sparse_amd import api
    say("case: graph replay of the two-pipeline launch")
    x = gen.make(None, seed=530, n_inst=200, n_q=4, pool_cells=2048, n_sel=1200, sel="uniform",
                 chunk=256)
    fc = api.fused_chunk_cells(200, 1200, 256)
    assert -(-1200 // fc) == 2 and api.fused_single_launch(200, 4, 12, 1200, 256)
    pool, dev = api.to_device(x)
    out = torch.empty(x.q.shape, device="cuda")
    lse = torch.empty(x.q.shape[:3], device="cuda")
    ws = api.workspace(200, 4, 12, 1200, 256)
    args = lambda: (pool, dev["page_table"], dev["sel"], dev["n_sel"], 1200, dev["q"],
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
    rng = np.random.default_rng(531)
    for rep in range(3):
        counts = rng.integers(0, 1201, size=200).astype(np.int32)
        counts[rep] = 0
        counts[rep + 3] = fc
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
        check(y, out.cpu().numpy(), lse.cpu().numpy(), inst_ids=[rep, rep + 3, 199],
              what=f"replay {rep}")


@pytest.mark.parametrize("kw,nch", [
    (dict(n_inst=180, n_q=3, pool_cells=1024, n_sel=700, chunk=256), 2),  # two pipelines, 36 rows
    (dict(n_inst=180, n_q=2, pool_cells=1024, n_sel=700, chunk=256), 2),  # two pipelines, 24 rows
    (dict(n_inst=200, n_q=2, pool_cells=1024, n_sel=250, chunk=256), 1),  # one chunk, small grid
])
def test_output_from_chunk_pass_masked(kw, nch):
    """Masked pages (-1), page ids past the pool, selected ids past the
    logical range and an instance with every page masked, in single-launch
    calls: against the oracle, the two passes bit for bit, gather indices
    exact."""
    from decode_attention_sparse_amd import api
    say(f"case: single launch with masking, {kw}")
    x = gen.make(None, seed=540 + nch, sel="uniform", **kw)
    n_inst, n_q, nh, _ = x.q.shape
    max_sel = int(x.sel.shape[1])
    assert api.fused_single_launch(n_inst, n_q, nh, max_sel, x.chunk)
    assert -(-max_sel // api.fused_chunk_cells(n_inst, max_sel, x.chunk)) == nch
    pt, sel = x.page_table.copy(), x.sel.copy()
    pt[0, ::7] = -1
    pt[1, 3] = x.n_phys_pages + 5
    pt[2, :] = -1                      # every cell of instance 2 masked
    sel[3, ::11] = x.n_logical_pages * 16 + 3  # past the logical range
    sel[4, 1] = -9
    x = dataclasses.replace(x, page_table=pt, sel=sel)
    from tests.gpu_util import run_batch
    out, lse, g, _ = run_batch(x)
    o2, l2, g2, _ = two_pass(x, api.fused_chunk_cells(n_inst, max_sel, x.chunk))
    assert np.array_equal(out, o2) and np.array_equal(lse, l2) and np.array_equal(g, g2)
    check(x, out, lse, g, inst_ids=[0, 1, 2, 3, 4, n_inst - 1], what="masked single launch")
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.all(g[2] == -1) and g[3, 0] == -1 and g[4, 1] == -1
