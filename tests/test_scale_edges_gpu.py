"""GPU parity at the edges of the binary16 scale range: cells whose K or V
scale is zero, the smallest subnormal (2^-24) or the smallest normal
(2^-14) among cells with ordinary scales, through the decode entry point
(fused call and the two passes) and prompt attention, against the oracle.

A zero K scale gives the cell a score of exactly 0 (it is not masked); a
zero V scale makes the cell add nothing to the output but its weight to the
denominator.  The oracle reads the stored binary16 values as they are, so
these cases need no reading of the pages beyond the dequantisation itself
(code times the cell's scale)."""
import dataclasses

import numpy as np
import pytest

from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import check, run_batch, run_prompt, say, two_pass
from tests.test_prompt_gpu import check as check_prompt

pytestmark = pytest.mark.gpu

ZERO, MIN_SUB, MIN_NORMAL = 0x0000, 0x0001, 0x0400


def edge_scales(x, seed):
    """Replace a tenth of the K scales and a tenth of the V scales with zero,
    and a twentieth of each with the smallest subnormal and with the
    smallest normal binary16 value (independently for K and V)."""
    rng = np.random.default_rng(seed)

    def edit(bits):
        b = bits.copy()
        u = rng.random(b.shape)
        b[u < 0.10] = ZERO
        b[(u >= 0.10) & (u < 0.15)] = MIN_SUB
        b[(u >= 0.15) & (u < 0.20)] = MIN_NORMAL
        return b

    return dataclasses.replace(x, k_scales=edit(x.k_scales), v_scales=edit(x.v_scales))


@pytest.mark.parametrize("n_q", [1, 4])
def test_decode_zero_and_tiny_scales(n_q):
    say(f"case: zero / subnormal / smallest normal scales, 2,051 cells, n_q={n_q}")
    x = edge_scales(gen.make(1).with_n_q(n_q), 70 + n_q)
    assert (x.k_scales == ZERO).any() and (x.v_scales == MIN_SUB).any()
    out, lse, g, _ = run_batch(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    check(x, out, lse, g, what=f"edge scales nq{n_q}")
    o2, l2, g2, _ = two_pass(x, 256)
    check(x, o2, l2, g2, what=f"edge scales nq{n_q}, two passes at chunk 256")


def test_decode_all_v_scales_zero():
    """Every V scale zero: the output is exactly 0 wherever a cell is
    visible, and the lse is that of the scores alone."""
    say("case: every V scale zero, 600 cells, n_q=1")
    x = gen.make(0)
    x = dataclasses.replace(x, v_scales=np.zeros_like(x.v_scales))
    out, lse, g, _ = run_batch(x)
    assert np.all(out == 0.0)
    check(x, out, lse, g, what="V scales zero")


def test_prompt_zero_and_tiny_scales():
    say("case: prompt attention, zero / subnormal / smallest normal scales")
    x = gen.make_prompt(None, seed=77, n_inst=2, n_q=40, n_qheads=12, pool_cells=1024)
    x = edge_scales(x, 78)
    out, lse = run_prompt(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    check_prompt(x, out, lse, "prompt edge scales", t_ids=[0, 13, 27, 39])
