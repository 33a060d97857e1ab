"""GPU parity of prompt (many-query) attention over the INT8 pools: the HIP
path (sda_prompt_attn_batch through the C ABI) against the CPU oracle's
prompt_attend (the decode definition over each position's causal prefix).

Tolerances as for decode (elementwise |gpu - oracle| <= atol + rtol*|oracle|):
out 1e-3 / 1e-3, lse 1e-4 / 1e-4; zero output and -inf lse for rows that
see no unmasked cell.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import (LSE_ATOL, LSE_RTOL, OUT_ATOL, OUT_RTOL, assert_close, run_prompt,
                            say)

pytestmark = pytest.mark.gpu


def check(x, out, lse, what, t_ids=None):
    e1 = e2 = 0.0
    for i in range(x.n_inst):
        ro, rl = oracle.prompt_attend(x, i, t_ids)
        sl = slice(None) if t_ids is None else np.asarray(t_ids)
        e1 = max(e1, assert_close(out[i][sl], ro, OUT_ATOL, OUT_RTOL, f"{what} inst {i} out"))
        e2 = max(e2, assert_close(lse[i][sl], rl, LSE_ATOL, LSE_RTOL, f"{what} inst {i} lse"))
    say(f"  {what}: max|dout| {e1:.2e} max|dlse| {e2:.2e}")


def masked(x, pages):
    pt = x.page_table.copy()
    for lp, val in pages:
        pt[:, lp] = val
    return dataclasses.replace(x, page_table=pt)


CASES = {
    # name: (make_prompt overrides, page-table edits)
    "tail_37q_12h": (dict(n_q=37, pool_cells=1024, seed=1), []),          # 444 rows: 7 groups, ragged
    "mid_64q_12h": (dict(n_q=64, pool_cells=4096, pos0=1000, seed=2), []),
    "first_positions_1h": (dict(n_q=70, n_qheads=1, pool_cells=512, pos0=0, seed=3), []),
    "rows_65_5h": (dict(n_q=13, n_qheads=5, pool_cells=512, seed=4), []),
    "rows_48_16h": (dict(n_q=3, n_qheads=16, pool_cells=512, seed=5), []),
    "rows_14_2h": (dict(n_q=7, n_qheads=2, pool_cells=256, seed=6), []),
    "one_row": (dict(n_q=1, n_qheads=1, pool_cells=256, pos0=100, seed=7), []),
    "masked_and_past_table": (dict(n_q=20, pool_cells=512, pos0=500, seed=8),
                              [(3, -1), (7, 99_999), (31, -1)]),
    "negative_pos0": (dict(n_q=10, pool_cells=256, pos0=-3, seed=9), []),
    "all_masked": (dict(n_q=6, pool_cells=128, seed=10), [(k, -1) for k in range(8)]),
    "three_instances": (dict(n_inst=3, n_q=9, pool_cells=1024, pos0=[100, 0, 700], seed=11), []),
    # 300 workgroups of 96 rows: more than one per CU
    "many_instances": (dict(n_inst=300, n_q=6, pool_cells=256,
                            pos0=list(range(-5, 295)), seed=14), []),
}


# Page tables of more than 2,048 pages (not staged whole in LDS): the
# launch takes the producer-wave form, 64-row workgroups while they fit one
# to a CU, 48-row ones beyond; checked on sampled positions and instances.
LARGE_TABLE = {
    "large_table_64row_groups": dict(n_inst=1, n_q=9, pool_cells=40960, pos0=[40000], seed=17),
    "large_table_48row_groups": dict(n_inst=130, n_q=8, pool_cells=32784,
                                     pos0=list(range(32700, 32830)), seed=18),
}


@pytest.mark.parametrize("name", sorted(LARGE_TABLE))
def test_prompt_large_page_table(name):
    kw = dict(LARGE_TABLE[name])
    say(f"case: prompt {name} {kw}")
    seed = kw.pop("seed")
    pos0 = kw.pop("pos0")
    x = gen.make_prompt(None, seed=seed, pos0=pos0, **kw)
    out, lse = run_prompt(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ids = [0, x.n_inst - 1]
    t_ids = [0, x.q.shape[1] - 1]
    xs = dataclasses.replace(x, q=x.q[ids], pos0=x.pos0[ids], page_table=x.page_table[ids])
    check(xs, out[ids], lse[ids], name, t_ids)


@pytest.mark.parametrize("name", sorted(CASES))
def test_prompt_cases(name):
    kw, edits = CASES[name]
    kw = dict(kw)
    say(f"case: prompt {name} {kw} edits={edits}")
    seed = kw.pop("seed")
    pos0 = kw.pop("pos0", None)
    x = masked(gen.make_prompt(None, seed=seed, pos0=pos0, **kw), edits)
    out, lse = run_prompt(x)
    check(x, out, lse, name)
    if name == "all_masked":
        assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_prompt_wide_scale_range():
    """K and V scales spread over 2^16 per cell (see the decode test)."""
    say("case: prompt, scales over 2^16")
    x = gen.make_prompt(None, seed=15, n_q=50, pool_cells=2048)
    rng = np.random.default_rng(16)
    def spread(bits):
        v = bits.view(np.float16).astype(np.float32)
        return (v * np.exp2(rng.uniform(-8, 8, v.shape)).astype(np.float32)).astype(
            np.float16).view(np.uint16)
    x = dataclasses.replace(x, k_scales=spread(x.k_scales), v_scales=spread(x.v_scales))
    out, lse = run_prompt(x)
    check(x, out, lse, "prompt wide scales")


def test_prompt_interleaved_scales():
    say("case: prompt, interleaved (K, V) scale pairs")
    x = gen.make_prompt(None, seed=12, n_q=21, pool_cells=1024)
    o1, l1 = run_prompt(x)
    o2, l2 = run_prompt(x, interleave=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    check(x, o2, l2, "interleaved")


def test_prompt_full_size_sampled():
    """The 32K-cell / 2,048-query workload in the launch configuration the
    bench times; the oracle checks sampled positions (12 rows each)."""
    x = gen.make_prompt("prompt_int8_32k_2048q")
    t_ids = [0, 1, 63, 64, 777, 1500, 2046, 2047]
    say(f"case: prompt full size 32K cells x 2,048 queries, oracle on positions {t_ids}")
    out, lse = run_prompt(x)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    check(x, out, lse, "prompt 32K x 2048", t_ids)


def test_prompt_deterministic_and_graph_replay():
    """Two eager calls agree bit for bit, and a captured call replays with a
    new pos0 (read on the device) to the eager result of that pos0."""
    import torch
    from decode_attention_sparse_amd import api
    say("case: prompt determinism and graph replay with changing pos0")
    x = gen.make_prompt(None, seed=13, n_q=40, pool_cells=2048)
    pool, dev = api.to_device(x)
    outs = []
    for _ in range(2):
        out = torch.empty(x.q.shape, device="cuda")
        lse = torch.empty(x.q.shape[:3], device="cuda")
        api.prompt_attn_batch(pool, dev["page_table"], dev["pos0"], dev["q"], x.softmax_scale,
                              out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    pos0 = dev["pos0"]
    out = torch.empty(x.q.shape, device="cuda")
    lse = torch.empty(x.q.shape[:3], device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.prompt_attn_batch(pool, dev["page_table"], pos0, dev["q"], x.softmax_scale, out,
                                  lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for k, p0 in enumerate([2008, 500, 0, 1999]):
        pos0.fill_(p0)
        g.replay()
        torch.cuda.synchronize()
        y = dataclasses.replace(x, pos0=np.array([p0], np.int32))
        ref_o = torch.empty_like(out)
        ref_l = torch.empty_like(lse)
        api.prompt_attn_batch(pool, dev["page_table"], pos0, dev["q"], x.softmax_scale, ref_o,
                              ref_l)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {k}"
        check(y, out.cpu().numpy(), lse.cpu().numpy(), f"replay {k} pos0={p0}",
              t_ids=[0, 17, 39])


@pytest.mark.parametrize("k", range(20))
def test_prompt_random_geometry(k):
    """Seeded sweep: instance, query and head counts, pool sizes, start
    positions (some negative, some running past the page table) and masked
    pages at random; sampled positions of every instance against the
    oracle."""
    rng = np.random.default_rng(9300 + k)
    n_inst = int(rng.choice([1, 2, 3, 5]))
    nh = int(rng.integers(1, 17))
    n_q = int(rng.integers(1, 301))
    pool_cells = int(rng.choice([256, 512, 1024, 2048]))
    pos0 = rng.integers(-20, pool_cells + 20, size=n_inst).astype(np.int32)
    say(f"case {k}: prompt n_inst={n_inst} n_q={n_q} n_qheads={nh} pool={pool_cells} "
        f"pos0={pos0.tolist()}")
    x = gen.make_prompt(None, seed=9400 + k, pos0=pos0, n_inst=n_inst, n_q=n_q, n_qheads=nh,
                        pool_cells=pool_cells)
    if rng.random() < 0.5:
        pt = x.page_table.copy()
        pt[rng.integers(0, n_inst, size=2), rng.integers(0, pt.shape[1], size=2)] = -1
        x = dataclasses.replace(x, page_table=pt)
    out, lse = run_prompt(x)
    t_ids = sorted({0, n_q - 1, n_q // 2, int(rng.integers(0, n_q)), int(rng.integers(0, n_q))})
    check(x, out, lse, f"case {k}", t_ids=t_ids)
    assert np.isfinite(out).all()
