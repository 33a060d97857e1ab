"""The entry point that allocates nothing (sda_decode_attn_batch_noalloc,
through the C ABI): its chunk partials live in the library's own device
array instead of a caller's workspace.  Same kernels and chunk size as
sda_decode_attn_batch, so outputs and gather indices must be identical bit
for bit, and match the oracle within the tolerance; three calls in a row,
each smaller than the one before (the array keeps the previous call's
partials), the last one a single launch that needs no partials."""
import numpy as np
import pytest

from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import check, run_batch, say

pytestmark = pytest.mark.gpu

CASES = [
    # 40 x 3,000 cells, 48 rows: 12 chunks of 256 per instance, pipelined
    # chunk pass + merge (23.8 MB of partials)
    ("pipelined + merge", dict(n_inst=40, n_q=4, pool_cells=8192, n_sel=3000, chunk=256, seed=71),
     False),
    # 8 x 1,000 cells, 24 rows: one-tile chunks + merge
    ("one-tile chunks + merge", dict(n_inst=8, n_q=2, pool_cells=4096, n_sel=1000, chunk=256,
                                     seed=72), False),
    # 260 x 1,000 cells, 24 rows, chunk 512: two chunks merged in place, one launch
    ("single launch", dict(n_inst=260, n_q=2, pool_cells=1024, n_sel=1000, chunk=512, seed=73),
     True),
]


def run_noalloc(x):
    import torch
    from decode_attention_sparse_amd import api
    pool, dev = api.to_device(x)
    n_inst, nq, nh, D = x.q.shape
    out = torch.full((n_inst, nq, nh, D), float("nan"), device="cuda")
    lse = torch.full((n_inst, nq, nh), float("nan"), device="cuda")
    g = torch.full(x.sel.shape, -7, dtype=torch.int32, device="cuda")
    api.decode_attn_batch_noalloc(pool, dev["page_table"], dev["sel"], dev["n_sel"],
                                  int(x.sel.shape[1]), dev["q"], x.softmax_scale, x.chunk, out, lse,
                                  gather_out=g)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), g.cpu().numpy()


def test_noalloc_equals_batch_entry():
    from decode_attention_sparse_amd import api
    for name, kw, single in CASES:
        x = gen.make(None, sel="uniform", **kw)
        n_inst, nq, nh, _ = x.q.shape
        max_sel = int(x.sel.shape[1])
        fc = api.fused_chunk_cells(n_inst, max_sel, x.chunk)
        need = 0 if single else api.workspace_bytes(n_inst, nq, nh, max_sel, fc)
        assert api.fused_single_launch(n_inst, nq, nh, max_sel, x.chunk) == single
        assert need <= api.SCRATCH_BYTES
        say(f"case: no-alloc entry point, {name}: {n_inst} x {max_sel} cells, {nq * nh} rows, "
            f"chunk {fc}, partials {need} B")
        o2, l2, g2 = run_noalloc(x)
        o1, l1, g1, _ = run_batch(x)
        assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
        assert np.array_equal(g1, g2)
        check(x, o2, l2, g2, inst_ids=[0, n_inst // 2, n_inst - 1], what=name)
