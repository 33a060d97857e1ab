"""GPU parity of the INT8 KV append (sda_kv_append_batch through the C ABI)
against the CPU oracle's kv_append: the whole pools after the call (codes and
scales of every cell, written or not) must be identical bit for bit, since
every code is an integer decision both sides take in float32."""
import dataclasses

import numpy as np
import pytest

import oracle
from decode_attention_sparse_amd import inputs as gen
from tests.gpu_util import (F32_FACTOR, LSE_ATOL, LSE_RTOL, OUT_ATOL, OUT_RTOL, assert_close,
                            dequant, f32_attend, run_prompt, say)

pytestmark = pytest.mark.gpu


def random_pools(seed, n_inst, cells, scale_stride=1):
    rng = np.random.default_rng(seed)
    total = n_inst * cells
    kc = rng.integers(-127, 128, size=(total, 256), dtype=np.int8)
    vc = rng.integers(-127, 128, size=(total, 256), dtype=np.int8)
    scales = rng.integers(0, 0x7c00, size=(2, total * scale_stride)).astype(np.uint16)
    return kc, scales[0].copy(), vc, scales[1].copy()


def run_append(pools, x, scale_stride=1):
    """Upload pools and rows, append on the GPU, return the four arrays."""
    import torch
    from decode_attention_sparse_amd import api
    kc, ks, vc, vs = pools
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if scale_stride == 2:
        # one [cells][2] array of (K, V) pairs; the oracle's K and V scale
        # arrays hold them at the even indices (cell * 2)
        pairs = t(np.stack([ks[0::2], vs[0::2]], axis=1).view(np.int16))
        pool = api.Pool(t(kc), None, t(vc), None, scales=pairs)
    else:
        pool = api.Pool(t(kc), t(ks.view(np.int16)), t(vc), t(vs.view(np.int16)))
    api.kv_append_batch(pool, t(x.page_table), t(x.pos0), t(x.k_new), t(x.v_new))
    torch.cuda.synchronize()
    if scale_stride == 2:
        pr = pool.scales.cpu().numpy().view(np.uint16)
        ks2, vs2 = ks.copy(), vs.copy()
        ks2[0::2], vs2[0::2] = pr[:, 0], pr[:, 1]
        return pool.k_codes.cpu().numpy(), ks2, pool.v_codes.cpu().numpy(), vs2
    return (pool.k_codes.cpu().numpy(), pool.k_scales.cpu().numpy().view(np.uint16),
            pool.v_codes.cpu().numpy(), pool.v_scales.cpu().numpy().view(np.uint16))


def oracle_append(pools, x, scale_stride=1):
    cur = tuple(np.array(a, copy=True) for a in pools)
    for i in range(x.n_inst):
        cur = oracle.kv_append(cur, x.page_table[i], x.page_table.shape[1], int(x.pos0[i]),
                               x.k_new[i], x.v_new[i], scale_stride=scale_stride)
    return cur


def check_equal(got, ref, what):
    names = ("k codes", "k scales", "v codes", "v scales")
    for g, r, nm in zip(got, ref, names):
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what}: {nm} differ at {len(bad)} places, first {bad[:3].tolist()}")
    say(f"  {what}: pools identical")


def special_rows(x):
    """Zero, tiny (subnormal binary16 scale), huge (saturated scale) rows and
    rows of exact ties (x / scale = k + 1/2) as the first new rows (as many
    as there are)."""
    k, v = x.k_new.copy(), x.v_new.copy()
    D = k.shape[-1]
    s = np.float32(2.0 ** -3)  # the tie rows' amax is exactly 127 s
    ties = (np.arange(D) % 120 - 60 + 0.5).astype(np.float32) * s
    ties[0] = 127 * s
    rows = [(np.zeros(D), np.zeros(D)),
            (np.linspace(-1e-5, 1e-5, D), np.full(D, 3e-6)),       # scale 7.9e-8: subnormal
            (np.linspace(-1e9, 1e9, D), np.full(D, -5e7)),         # saturated, clamped
            (ties, -ties)]
    for t, (rk, rv) in enumerate(rows[: x.n_new]):
        k[0, t], v[0, t] = rk, rv
    return dataclasses.replace(x, k_new=k, v_new=v)


CASES = {
    # name: (make_append overrides, pos0, page-table edits, scale_stride)
    "tail_37_rows": (dict(n_inst=1, n_new=37, pool_cells=1024, seed=1), None, [], 1),
    "three_instances": (dict(n_inst=3, n_new=100, pool_cells=1024, seed=2), [0, 500, 924], [], 1),
    "masked_and_past_table": (dict(n_inst=2, n_new=60, pool_cells=512, seed=3), [470, 10],
                              [(1, -1), (30, 99_999)], 1),
    "negative_pos0": (dict(n_inst=1, n_new=20, pool_cells=256, seed=4), [-7], [], 1),
    "interleaved_scales": (dict(n_inst=2, n_new=45, pool_cells=512, seed=5), [3, 200], [], 2),
    "one_row": (dict(n_inst=1, n_new=1, pool_cells=256, seed=6), [255], [], 1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_cases(name):
    kw, pos0, edits, stride = CASES[name]
    kw = dict(kw)
    seed = kw.pop("seed")
    say(f"case: kv append {name} {kw} pos0={pos0} edits={edits} stride={stride}")
    x = special_rows(gen.make_append(None, seed=seed, pos0=pos0, **kw))
    pt = x.page_table.copy()
    for lp, val in edits:
        pt[:, lp] = val
    x = dataclasses.replace(x, page_table=pt)
    pools = random_pools(seed + 100, x.n_inst, x.pool_cells, stride)
    check_equal(run_append(pools, x, stride), oracle_append(pools, x, stride), name)


def test_append_full_size_sampled():
    """The bench workload (64 instances x 2,048 rows into 32K-cell pools); the
    oracle recomputes sampled instances on their own pool slices."""
    x = gen.make_append("kv_append_64inst_2048rows")
    say("case: kv append 64 x 2,048 rows, oracle on instances [0, 17, 63]")
    cells = x.pool_cells
    pools = tuple(np.zeros(s, dt) for s, dt in (((64 * cells, 256), np.int8), (64 * cells, np.uint16),
                                                ((64 * cells, 256), np.int8), (64 * cells, np.uint16)))
    got = run_append(pools, x)
    for i in (0, 17, 63):
        sl = slice(i * cells, (i + 1) * cells)
        sub = (pools[0][sl], pools[1][sl], pools[2][sl], pools[3][sl])
        pt = x.page_table[i] - i * (cells // 16)  # the instance's pages, counted from its slice
        ref = oracle.kv_append(sub, pt, pt.size, int(x.pos0[i]), x.k_new[i], x.v_new[i])
        check_equal(tuple(g[sl] for g in got), ref, f"instance {i}")


def test_append_then_prompt_attention():
    """A prompt chunk's K and V appended into the pool, then attended to by
    the chunk's queries: GPU append + GPU prompt attention against the
    oracle's append + prompt attention.  The appended rows spread over 2^+-2
    (scores of order 10); with rows over 2^+-8 the scores reach the
    thousands, where a plain float32 attention already misses 1e-3."""
    say("case: append a 300-row prompt chunk, then prompt attention over the pool")
    base = gen.make_prompt(None, seed=21, n_q=300, pool_cells=2048)
    app = gen.make_append(None, seed=22, n_inst=1, n_new=300, pool_cells=2048,
                          pos0=int(base.pos0[0]), spread=2.0)
    app = dataclasses.replace(app, page_table=base.page_table)
    pools = (base.k_codes, base.k_scales, base.v_codes, base.v_scales)
    gpu_pools = run_append(pools, app)
    ref_pools = oracle_append(pools, app)
    check_equal(gpu_pools, ref_pools, "appended pools")
    x = dataclasses.replace(base, k_codes=gpu_pools[0], k_scales=gpu_pools[1],
                            v_codes=gpu_pools[2], v_scales=gpu_pools[3])
    out, lse = run_prompt(x)
    ro, rl = oracle.prompt_attend(x, 0)
    e1 = assert_close(out[0], ro, OUT_ATOL, OUT_RTOL, "append+prompt out")
    e2 = assert_close(lse[0], rl, LSE_ATOL, LSE_RTOL, "append+prompt lse")
    say(f"  append + prompt: max|dout| {e1:.2e} max|dlse| {e2:.2e}")


def test_append_wide_v_diffuse_attention():
    """V rows at the append workload's full range (N(0, 1) x 2^U(-8, 8): V
    scales over 2^16) and K rows N(0, 1), so scores are of order 1 and
    attention spreads over hundreds of cells: a weight's rounding then adds
    up over many cells.  GPU append, then GPU decode over a selection holding
    every appended cell, and GPU prompt attention over the pool; each against
    the oracle's append + attention, and no further from it than a few times
    a plain float32 attention on the same pools."""
    n_new, cells, n_sel = 300, 2048, 1024
    pos0 = cells - n_new
    say("case: V rows over 2^+-8 and K rows N(0,1) appended at 1748..2047 of a 2,048-cell pool")
    x = gen.make(None, seed=31, n_inst=1, n_q=4, pool_cells=cells, n_sel=n_sel, sel="uniform",
                 chunk=256)
    app = gen.make_append(None, seed=32, n_inst=1, n_new=n_new, pool_cells=cells, pos0=pos0,
                          spread=8.0, k_spread=0.0)
    app = dataclasses.replace(app, page_table=x.page_table)
    pools = (x.k_codes, x.k_scales, x.v_codes, x.v_scales)
    gp = run_append(pools, app)
    check_equal(gp, oracle_append(pools, app), "appended pools")
    rng = np.random.default_rng(33)
    others = rng.choice(pos0, n_sel - n_new, replace=False)
    sel = np.empty((1, n_sel), np.int32)
    sel[0] = np.sort(np.concatenate([others, np.arange(pos0, cells)]))
    x = dataclasses.replace(x, sel=sel, k_codes=gp[0], k_scales=gp[1], v_codes=gp[2],
                            v_scales=gp[3])

    def compare(got_o, got_l, ref_o, ref_l, f32_o, f32_l, what):
        assert np.isfinite(got_o).all() and np.isfinite(got_l).all(), what
        assert_close(got_o, ref_o, OUT_ATOL, OUT_RTOL, f"{what} out")
        assert_close(got_l, ref_l, LSE_ATOL, LSE_RTOL, f"{what} lse")
        e_o, f_o = np.abs(got_o - ref_o).max(), np.abs(f32_o - ref_o).max()
        e_l, f_l = np.abs(got_l - ref_l).max(), np.abs(f32_l - ref_l).max()
        say(f"  {what}: max|out| {np.abs(ref_o).max():.1f}; max|dout| GPU {e_o:.2e} float32 "
            f"{f_o:.2e}; max|dlse| GPU {e_l:.2e} float32 {f_l:.2e}")
        assert e_o <= F32_FACTOR * f_o, f"{what}: out error {e_o:.3e} vs float32 {f_o:.3e}"
        assert e_l <= F32_FACTOR * f_l + 1e-6, f"{what}: lse error {e_l:.3e} vs float32 {f_l:.3e}"

    # decode over the selection
    from tests.gpu_util import run_batch
    out, lse, g, _ = run_batch(x)
    ro, rl = oracle.attend(x)
    phys = oracle.gather(x)[0]
    qr = x.q[0].reshape(-1, 256)
    fo, fl = f32_attend(qr, dequant(gp[0], gp[1], phys), dequant(gp[2], gp[3], phys),
                        x.softmax_scale)
    compare(out[0].reshape(-1, 256), lse[0].reshape(-1), ro[0].reshape(-1, 256),
            rl[0].reshape(-1), fo, fl, "append + decode")

    # prompt attention of the appended chunk's positions over the pool
    xp = gen.make_prompt(None, seed=34, n_q=n_new, pool_cells=cells)
    xp = dataclasses.replace(xp, page_table=x.page_table, k_codes=gp[0], k_scales=gp[1],
                             v_codes=gp[2], v_scales=gp[3])
    assert int(xp.pos0[0]) == pos0
    po, pl = run_prompt(xp)
    pro, prl = oracle.prompt_attend(xp, 0)
    c = np.arange(cells)
    phys_all = x.page_table[0][c >> 4] * 16 + (c & 15)
    t = np.repeat(np.arange(n_new), xp.q.shape[2])
    vis = c[None, :] <= (pos0 + t)[:, None]
    fo, fl = f32_attend(xp.q[0].reshape(-1, 256), dequant(gp[0], gp[1], phys_all),
                        dequant(gp[2], gp[3], phys_all), xp.softmax_scale, vis)
    compare(po[0].reshape(-1, 256), pl[0].reshape(-1), pro.reshape(-1, 256), prl.reshape(-1),
            fo, fl, "append + prompt")


@pytest.mark.parametrize("k", range(15))
def test_append_random_geometry(k):
    """Seeded sweep: instance and row counts, pool sizes, start positions
    (some negative, some past the table), masked pages and both scale
    layouts; the whole pools against the oracle, bit for bit."""
    rng = np.random.default_rng(9500 + k)
    n_inst = int(rng.choice([1, 2, 3, 7]))
    pool_cells = int(rng.choice([256, 512, 1024]))
    n_new = int(rng.integers(1, 400))
    pos0 = rng.integers(-30, pool_cells, size=n_inst).astype(np.int32)
    stride = int(rng.choice([1, 2]))
    say(f"case {k}: append n_inst={n_inst} n_new={n_new} pool={pool_cells} pos0={pos0.tolist()} "
        f"stride={stride}")
    x = special_rows(gen.make_append(None, seed=9600 + k, pos0=pos0, n_inst=n_inst, n_new=n_new,
                                     pool_cells=pool_cells))
    if rng.random() < 0.5:
        pt = x.page_table.copy()
        pt[rng.integers(0, n_inst), rng.integers(0, pt.shape[1])] = -1
        pt[rng.integers(0, n_inst), rng.integers(0, pt.shape[1])] = 10**7
        x = dataclasses.replace(x, page_table=pt)
    pools = random_pools(9700 + k, x.n_inst, x.pool_cells, stride)
    check_equal(run_append(pools, x, stride), oracle_append(pools, x, stride), f"case {k}")
