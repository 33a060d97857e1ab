"""GPU parity at the edges of the binary16 scale range: cells whose K or V
scale is zero, the smallest subnormal (2^-24) or the smallest normal
(2^-14) among cells with ordinary scales, through the decode entry point
(fused call and the two passes) and prompt attention, against the oracle;
and V scales spread ever wider from cell to cell, against the error a
plain float32 computation makes on the same pools.

A zero K scale gives the cell a score of exactly 0 (it is not masked); a
zero V scale makes the cell add nothing to the output but its weight to the
denominator.  The oracle reads the stored binary16 values as they are, so
these cases need no reading of the pages beyond the dequantisation itself
(code times the cell's scale)."""
import dataclasses

import numpy as np
import pytest

import oracle
from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import (F32_FACTOR, OUT_ATOL, OUT_RTOL, check, dequant, f32_attend,
                            f32_online, run_batch, run_prompt, say, two_pass)
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


@pytest.mark.parametrize("octaves", [0, 4, 8, 12, 16, 20])
def test_v_scale_spread_envelope(octaves):
    """V scales spread over 2^+-octaves from cell to cell (clipped to the
    binary16 range), K as drawn (scores of order one: attention spread over
    many cells).  The P.V weights sit on a grid set by each tile's largest
    V scale, so the cells with small scales in a tile carry fewer bits; the
    output must stay within a few times a float32 computation's error at
    every spread, and within the elementwise tolerance up to 2^+-12 (at
    2^+-16 and beyond float32 itself comes near or past it)."""
    rng = np.random.default_rng(500 + octaves)
    x = gen.make(1).with_n_q(4)
    v = x.v_scales.view(np.float16).astype(np.float64)
    v = np.clip(v * np.exp2(rng.uniform(-octaves, octaves, v.shape)), 2.0**-24, 65504.0)
    x = dataclasses.replace(x, v_scales=v.astype(np.float16).view(np.uint16))
    out, lse, g, _ = run_batch(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ro, rl = oracle.attend(x)
    phys = oracle.gather(x)[0]
    fo, fl = f32_attend(x.q[0].reshape(-1, 256), dequant(x.k_codes, x.k_scales, phys),
                        dequant(x.v_codes, x.v_scales, phys), x.softmax_scale)
    go, ref = out[0].reshape(-1, 256), ro[0].reshape(-1, 256)
    e_g, e_f = np.abs(go - ref), np.abs(fo - ref)
    tol = OUT_ATOL + OUT_RTOL * np.abs(ref)
    say(f"  spread 2^+-{octaves}: max|out| {np.abs(ref).max():.2e}; max|dout| GPU {e_g.max():.2e} "
        f"float32 {e_f.max():.2e}; worst error / tolerance GPU {(e_g / tol).max():.3f} "
        f"float32 {(e_f / tol).max():.3f}")
    assert e_g.max() <= F32_FACTOR * e_f.max() + 1e-7
    assert np.abs(lse[0].reshape(-1) - rl[0].reshape(-1)).max() <= 1e-5
    if octaves <= 12:
        check(x, out, lse, g, what=f"V scales over 2^+-{octaves}")
    # the same through chunks of 2,048 cells (32 tiles accumulated in one
    # partial) against a float32 online softmax in the same tile order
    o2, l2, _, _ = two_pass(x, 2048)
    oo, _ = f32_online(x.q[0].reshape(-1, 256), dequant(x.k_codes, x.k_scales, phys),
                       dequant(x.v_codes, x.v_scales, phys), x.softmax_scale)
    e_2, e_o = np.abs(o2[0].reshape(-1, 256) - ref).max(), np.abs(oo - ref).max()
    say(f"  chunks of 2,048: max|dout| GPU {e_2:.2e} float32 online softmax {e_o:.2e}")
    assert e_2 <= F32_FACTOR * e_o + 1e-7


@pytest.mark.parametrize("octaves", [4, 8, 12])
def test_k_scale_spread_envelope(octaves):
    """K scales spread over 2^+-octaves from cell to cell: scores from order
    one to the thousands, so attention peaks on few cells and the
    log-sum-exp grows.  The query digits are exact to 2^-24 of each wave's
    largest query value, so the scores carry float32-level error relative
    to the largest score; outputs and log-sum-exps must stay within a few
    times a float32 computation's error."""
    rng = np.random.default_rng(600 + octaves)
    x = gen.make(1).with_n_q(4)
    k = x.k_scales.view(np.float16).astype(np.float64)
    k = np.clip(k * np.exp2(rng.uniform(-octaves, octaves, k.shape)), 2.0**-24, 65504.0)
    x = dataclasses.replace(x, k_scales=k.astype(np.float16).view(np.uint16))
    out, lse, g, _ = run_batch(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ro, rl = oracle.attend(x)
    phys = oracle.gather(x)[0]
    fo, fl = f32_attend(x.q[0].reshape(-1, 256), dequant(x.k_codes, x.k_scales, phys),
                        dequant(x.v_codes, x.v_scales, phys), x.softmax_scale)
    go, ref = out[0].reshape(-1, 256), ro[0].reshape(-1, 256)
    gl, rlf = lse[0].reshape(-1), rl[0].reshape(-1)
    e_o, f_o = np.abs(go - ref).max(), np.abs(fo - ref).max()
    e_l, f_l = np.abs(gl - rlf).max(), np.abs(fl - rlf).max()
    say(f"  K spread 2^+-{octaves}: max|lse| {np.abs(rlf).max():.1f}; max|dout| GPU {e_o:.2e} "
        f"float32 {f_o:.2e}; max|dlse| GPU {e_l:.2e} float32 {f_l:.2e}")
    assert e_o <= F32_FACTOR * f_o + 1e-7
    assert e_l <= F32_FACTOR * f_l + 1e-6
    check(x, out, lse, g, what=f"K scales over 2^+-{octaves}", strict_lse=False)


@pytest.mark.parametrize("octaves", [0, 8, 12, 16])
def test_prompt_v_scale_spread_envelope(octaves):
    """Prompt attention with V scales spread over 2^+-octaves (32 tiles per
    row): within a few times the error of a float32 online softmax taken in
    the same tile order, on the sampled positions."""
    rng = np.random.default_rng(700 + octaves)
    x = gen.make_prompt(None, seed=71, n_inst=1, n_q=64, n_qheads=12, pool_cells=2048)
    v = x.v_scales.view(np.float16).astype(np.float64)
    v = np.clip(v * np.exp2(rng.uniform(-octaves, octaves, v.shape)), 2.0**-24, 65504.0)
    x = dataclasses.replace(x, v_scales=v.astype(np.float16).view(np.uint16))
    out, lse = run_prompt(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    t_ids = [0, 21, 42, 63]
    ro, rl = oracle.prompt_attend(x, 0, t_ids)
    cells = x.page_table.shape[1] * 16
    c = np.arange(cells)
    phys_all = x.page_table[0][c >> 4] * 16 + (c & 15)
    nh = x.q.shape[2]
    t = np.repeat(np.asarray(t_ids), nh)
    vis = c[None, :] <= (int(x.pos0[0]) + t)[:, None]
    fo, _ = f32_online(x.q[0][t_ids].reshape(-1, 256), dequant(x.k_codes, x.k_scales, phys_all),
                       dequant(x.v_codes, x.v_scales, phys_all), x.softmax_scale, vis)
    go, ref = out[0][t_ids].reshape(-1, 256), ro.reshape(-1, 256)
    e_o, f_o = np.abs(go - ref).max(), np.abs(fo - ref).max()
    say(f"  prompt V spread 2^+-{octaves}: max|out| {np.abs(ref).max():.2e}; max|dout| GPU "
        f"{e_o:.2e} float32 online softmax {f_o:.2e}")
    assert e_o <= F32_FACTOR * f_o + 1e-7
    assert np.abs(lse[0][t_ids].reshape(-1) - rl.reshape(-1)).max() <= 1e-5
