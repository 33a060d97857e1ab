"""Seeded sweep of decode geometries through sda_decode_attn_batch: instance
counts, query counts, head counts (up to 64 rows), pool sizes, list lengths,
chunk sizes, ragged device counts and masked pages drawn at random, so that
every launch form the library chooses between (one-tile chunks, pipelined
chunks with one or several chunks per workgroup, the V accumulation split
over two waves, the single launch with one or two pipelines, the three merge
forms) meets the others' edge cases.  Each geometry: sampled instances
against the oracle, gather indices exact, and the outputs equal to the two
passes at the call's chunk size bit for bit."""
import dataclasses

import numpy as np
import pytest

from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import check, run_batch, say, two_pass

pytestmark = pytest.mark.gpu

N_CASES = 40


def draw(k):
    rng = np.random.default_rng(9100 + k)
    n_q = int(rng.integers(1, 5))
    nh = int(rng.integers(1, 64 // n_q + 1))
    nh = min(nh, 16)
    pool_cells = int(rng.choice([256, 512, 1024, 2048]))
    n_inst = int(rng.choice([1, 2, 3, 7, 20, 64, 150, 257, 300]))
    if n_inst * pool_cells > 300 * 1024:  # keep the host pools small
        pool_cells = 1024 if n_inst <= 300 else 512
    max_sel = int(rng.integers(1, pool_cells + 1))
    chunk = int(rng.choice([64, 128, 256, 512, 1024]))
    return rng, dict(n_inst=n_inst, n_q=n_q, n_qheads=nh, pool_cells=pool_cells, n_sel=max_sel,
                     chunk=chunk)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_geometry(k):
    from decode_attention_sparse_amd import api
    rng, kw = draw(k)
    x = gen.make(None, seed=9200 + k, sel="uniform", **kw)
    n_inst, n_q, nh, _ = x.q.shape
    max_sel = int(x.sel.shape[1])
    fc = api.fused_chunk_cells(n_inst, max_sel, x.chunk)
    single = api.fused_single_launch(n_inst, n_q, nh, max_sel, x.chunk)
    say(f"case {k}: {kw} fused chunk {fc}, single launch {single}")
    counts = rng.integers(0, max_sel + 1, size=n_inst).astype(np.int32)
    counts[0] = max_sel
    pt, sel = x.page_table.copy(), x.sel.copy()
    if rng.random() < 0.5:  # masked pages and ids past the pool
        pt[rng.integers(0, n_inst, size=3), rng.integers(0, pt.shape[1], size=3)] = -1
        pt[rng.integers(0, n_inst), rng.integers(0, pt.shape[1])] = x.n_phys_pages + 1
    if rng.random() < 0.3 and max_sel > 1:  # ids past the logical range
        sel[rng.integers(0, n_inst), rng.integers(0, max_sel)] = x.n_logical_pages * 16 + 7
    x = dataclasses.replace(x, page_table=pt, sel=sel, n_sel=counts)
    out, lse, g, _ = run_batch(x)
    o2, l2, g2, _ = two_pass(x, fc)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2), "differs from the two passes"
    assert np.array_equal(g, g2)
    ids = sorted({0, n_inst // 2, n_inst - 1, int(rng.integers(0, n_inst))})
    check(x, out, lse, g, inst_ids=ids, what=f"case {k}")
