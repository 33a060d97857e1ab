"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes an oracle module-like object `O` (functions gather, attend,
chunk_partials, merge, half_to_double) and raises AssertionError when the
oracle disagrees with:
  - a library routine (numpy's binary16 decode; scipy's softmax and
    logsumexp applied to a dense matrix built by numpy reshapes of the pool);
  - a closed form (one cell, two cells, identical keys, zero query, a
    hand-computed example stored under tests/golden/, the merge of two
    partials with known values);
  - an invariant that the exact result has (selection order, chunk size,
    a uniform score shift realised through the inputs, relabelling of
    physical pages, masking equals deletion, doubling V scales doubles the
    output, duplicate entries);
  - brute force: every one- and two-cell subset (and random larger ones) of
    a 32-cell pool, recomputed with scalar Python arithmetic.
test_oracle.py runs every pin against the oracle, and also against mutated
copies of the oracle source to show that plausible mistakes are caught.
"""
from __future__ import annotations

import dataclasses
import math
import os
import types

import numpy as np
import scipy.special

from decode_attention_sparse_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def tiny(seed, **kw):
    spec = dict(n_inst=1, n_q=1, n_qheads=3, head_dim=8, pool_cells=64, n_sel=10,
                sel="uniform", heavy=False, chunk=4)
    spec.update(kw)
    return gen.make(None, seed=seed, **spec)


def textbook(x, i):
    """softmax(S) V over the selected rows of a dense dequantised matrix.

    The logical view of the pool is built with numpy: the physical pool is
    reshaped into pages, the page table indexes pages, and the result is
    flattened back to cells; a selected id then indexes that flattened view."""
    D = x.q.shape[-1]
    n_pages_phys = x.k_codes.shape[0] // 16
    Kp = (x.k_codes.astype(np.float64) * f16(x.k_scales)[:, None]).reshape(n_pages_phys, 16, D)
    Vp = (x.v_codes.astype(np.float64) * f16(x.v_scales)[:, None]).reshape(n_pages_phys, 16, D)
    pt = np.asarray(x.page_table[i], np.int64)
    page_ok = (pt >= 0) & (pt < n_pages_phys)
    safe = np.where(page_ok, pt, 0)
    Klog = Kp[safe].reshape(-1, D)
    Vlog = Vp[safe].reshape(-1, D)
    ok_log = np.repeat(page_ok, 16)
    s = np.asarray(x.sel[i, : x.n_sel[i]], np.int64)
    in_range = (s >= 0) & (s < Klog.shape[0])
    s_in = s[in_range]
    keep = ok_log[s_in]
    Ks, Vs = Klog[s_in][keep], Vlog[s_in][keep]
    Q = np.asarray(x.q[i], np.float64).reshape(-1, D)
    R = Q.shape[0]
    if Ks.shape[0] == 0:
        return np.zeros((R, D)), np.full((R,), -np.inf)
    S = float(x.softmax_scale) * (Q @ Ks.T)
    P = scipy.special.softmax(S, axis=1)
    return P @ Vs, scipy.special.logsumexp(S, axis=1)


def _close(a, b, rtol, atol=0.0, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):  # inf - inf where both are the same infinity
        bad = ~same_inf & ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    assert not bad.any(), f"{what}: max |diff| {np.nanmax(np.abs(np.where(same_inf, 0, a - b)))}"


def _attend_flat(O, x, ids=None):
    out, lse = O.attend(x, ids)
    k = out.shape[0]
    D = out.shape[-1]
    return out.reshape(k, -1, D), lse.reshape(k, -1)


# ---------------------------------------------------------------- library pins
def pin_half_decode(O):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = O.half_to_double(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_textbook(O):
    cases = [
        tiny(1),
        tiny(2, n_q=2, n_sel=40, pool_cells=128),
        tiny(3, n_inst=3, n_q=2, n_qheads=2, head_dim=16, pool_cells=96, n_sel=64),
        tiny(4, head_dim=256, n_qheads=12, pool_cells=256, n_sel=33),
        tiny(5, n_sel=20, pool_cells=64, heavy=True),
    ]
    # masked pages and out-of-range entries
    x = tiny(6, n_sel=30, pool_cells=128)
    pt = x.page_table.copy()
    pt[0, 1] = -1
    pt[0, 5] = 10_000
    sel = x.sel.copy()
    sel[0, 0] = -3
    sel[0, 1] = 128 + 5
    cases.append(dataclasses.replace(x, page_table=pt, sel=sel))
    for x in cases:
        out, lse = _attend_flat(O, x)
        for i in range(x.q.shape[0]):
            ro, rl = textbook(x, i)
            _close(out[i], ro, 1e-12, 1e-14, "textbook out")
            _close(lse[i], rl, 1e-12, 1e-14, "textbook lse")


def pin_gather_exhaustive(O):
    """Every logical cell of a 4,096-cell pool (one chunk of 256 pages) against
    the numpy page view of physical cell ids, with masked pages."""
    x = gen.make(0, n_sel=4096)  # all cells, permuted table
    pt = x.page_table.copy()
    pt[0, [0, 7, 255]] = -1
    x = dataclasses.replace(x, page_table=pt)
    got = O.gather(x)[0]
    phys_ids = np.arange(x.k_codes.shape[0], dtype=np.int64).reshape(-1, 16)
    ok = pt[0] >= 0
    view = np.where(ok[:, None], phys_ids[np.where(ok, pt[0], 0)], -1).reshape(-1)
    assert np.array_equal(got, view[x.sel[0]])


# ---------------------------------------------------------------- closed forms
def pin_one_cell(O):
    x = tiny(11, n_sel=1, n_qheads=4)
    out, lse = _attend_flat(O, x)
    c = int(x.sel[0, 0])
    ph = int(x.page_table[0, c // 16]) * 16 + c % 16
    v_hat = x.v_codes[ph].astype(np.float64) * f16(x.v_scales[ph])
    for r in range(out.shape[1]):
        assert np.array_equal(out[0, r], v_hat)  # weight exactly 1
    # lse equals the score; the score itself is pinned by pin_textbook
    ro, rl = textbook(x, 0)
    _close(lse[0], rl, 1e-13, 0, "one-cell lse")


def pin_two_cells(O):
    x = tiny(12, n_sel=2, n_qheads=2, heavy=True)
    out, lse = _attend_flat(O, x)
    D = x.q.shape[-1]
    phs = [int(x.page_table[0, c // 16]) * 16 + c % 16 for c in x.sel[0]]
    vh = [x.v_codes[p].astype(np.float64) * f16(x.v_scales[p]) for p in phs]
    kh = [x.k_codes[p].astype(np.float64) * f16(x.k_scales[p]) for p in phs]
    for r in range(out.shape[1]):
        q = x.q[0].reshape(-1, D)[r].astype(np.float64)
        s1, s2 = (x.softmax_scale * float(q @ k) for k in kh)
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        _close(out[0, r], w1 * vh[0] + w2 * vh[1], 1e-12, 1e-15, "two-cell out")
        _close(lse[0, r], np.logaddexp(s1, s2), 1e-13, 0, "two-cell lse")


def pin_zero_query(O):
    """q = 0: every score is 0, weights are uniform, lse = ln n."""
    x = tiny(13, n_sel=37, pool_cells=128, n_qheads=2)
    x = dataclasses.replace(x, q=np.zeros_like(x.q))
    out, lse = _attend_flat(O, x)
    phs = [int(x.page_table[0, c // 16]) * 16 + c % 16 for c in x.sel[0]]
    mean = np.mean([x.v_codes[p].astype(np.float64) * f16(x.v_scales[p]) for p in phs], axis=0)
    for r in range(out.shape[1]):
        assert lse[0, r] == math.log(37)
        _close(out[0, r], mean, 1e-13, 1e-16, "zero-q out")


def pin_identical_keys(O):
    """All selected cells share one key row and scale: uniform weights,
    lse = s + ln n with s the common score."""
    x = tiny(14, n_sel=9, pool_cells=64, n_qheads=3)
    kc = x.k_codes.copy()
    kc[:] = kc[5]
    ks = x.k_scales.copy()
    ks[:] = ks[5]
    y = dataclasses.replace(x, k_codes=kc, k_scales=ks)
    out, lse = _attend_flat(O, y)
    D = x.q.shape[-1]
    k_hat = kc[5].astype(np.float64) * f16(ks[5])
    phs = [int(x.page_table[0, c // 16]) * 16 + c % 16 for c in x.sel[0]]
    mean = np.mean([x.v_codes[p].astype(np.float64) * f16(x.v_scales[p]) for p in phs], axis=0)
    for r in range(out.shape[1]):
        s = x.softmax_scale * float(x.q[0].reshape(-1, D)[r].astype(np.float64) @ k_hat)
        _close(lse[0, r], s + math.log(9), 1e-13, 1e-15, "identical-keys lse")
        _close(out[0, r], mean, 1e-13, 1e-16, "identical-keys out")


def load_worked_example():
    """tests/golden/worked_example.txt: a hand-computed instance (see the file)."""
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split("=", 1)
            vals[key.strip()] = [float(t) for t in rest.split()]
    return vals


def pin_worked_example(O):
    g = load_worked_example()
    D = 4
    # pool: one physical page (16 cells); page table maps logical page 0 to it
    kc = np.zeros((16, D), np.int8)
    vc = np.zeros((16, D), np.int8)
    kc[2, 0], kc[7, 0], kc[9, 0] = 8, 0, -8
    vc[2] = [1, 2, 3, 4]
    vc[7] = [10, 0, -10, 0]
    vc[9] = [-4, 4, -4, 4]
    one = np.full(16, np.float16(1.0)).view(np.uint16)
    half = np.full(16, np.float16(0.5)).view(np.uint16)
    q = np.zeros((1, 1, 1, D), np.float32)
    q[..., 0] = 2.0  # scores: (1/16) * 1 * 2 * {8, 0, -8} = {1, 0, -1}
    x = types.SimpleNamespace(k_codes=kc, v_codes=vc, k_scales=one, v_scales=half,
                              page_table=np.zeros((1, 1), np.int32),
                              sel=np.array([[2, 7, 9]], np.int32), n_sel=np.array([3], np.int32),
                              q=q, softmax_scale=1.0 / 16.0)
    out, lse = _attend_flat(O, x)
    _close(out[0, 0], np.array(g["out"]), 1e-15, 1e-15, "worked out")
    _close(lse[0], np.array(g["lse"]), 1e-15, 0, "worked lse")


def pin_merge_closed_form(O):
    """Two partials: (acc a, m 0, l 1) and (acc b, m ln 3, l 1), plus an empty
    one.  M = ln 3, L = 1/3 + 1 = 4/3, out = (a + 3b)/4, lse = ln 4."""
    a = np.array([4.0, -8.0, 0.5])
    b = np.array([0.0, 8.0, 2.5])
    acc = np.zeros((1, 3, 1, 3))
    acc[0, 0, 0], acc[0, 1, 0] = a, b
    m = np.array([[[0.0], [math.log(3.0)], [-np.inf]]])
    l = np.array([[[1.0], [1.0], [0.0]]])
    out, lse = O.merge(acc, m, l)
    _close(out[0, 0], (a + 3 * b) / 4, 1e-15, 1e-15, "merge out")
    _close(lse[0, 0], math.log(4.0), 1e-15, 0, "merge lse")
    out, lse = O.merge(np.zeros((1, 2, 1, 3)), np.full((1, 2, 1), -np.inf), np.zeros((1, 2, 1)))
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- invariants
def pin_empty_and_masked(O):
    x = tiny(21, n_sel=12)
    y = dataclasses.replace(x, n_sel=np.zeros(1, np.int32))
    out, lse = _attend_flat(O, y)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    pt = np.full_like(x.page_table, -1)
    out, lse = _attend_flat(O, dataclasses.replace(x, page_table=pt))
    assert np.all(out == 0) and np.all(lse == -np.inf)


def pin_permutation(O):
    x = tiny(22, n_sel=50, pool_cells=256, n_q=2)
    rng = np.random.default_rng(5)
    y = dataclasses.replace(x, sel=x.sel[:, rng.permutation(50)].copy())
    a, b = _attend_flat(O, x), _attend_flat(O, y)
    _close(b[0], a[0], 1e-12, 1e-15, "perm out")
    _close(b[1], a[1], 1e-13, 0, "perm lse")


def pin_chunking(O):
    x = tiny(23, n_sel=67, pool_cells=256, n_q=2, heavy=True)
    ref = _attend_flat(O, x)
    for C in (1, 3, 64, 66, 67, 256):
        acc, m, l = O.chunk_partials(x, C)
        out, lse = O.merge(acc, m, l)
        _close(out, ref[0], 1e-12, 1e-15, f"chunk {C} out")
        _close(lse, ref[1], 1e-13, 0, f"chunk {C} lse")
    # a partial over one chunk is the dense un-normalised result
    acc, m, l = O.chunk_partials(x, 1000)
    _close(acc[:, 0] / l[:, 0, :, None], ref[0], 1e-12, 1e-15, "single chunk")
    _close(m[:, 0] + np.log(l[:, 0]), ref[1], 1e-13, 0, "single chunk lse")


def pin_score_shift(O):
    """Scores shifted by a constant through the inputs: every cell has the same
    K scale and code 127 in dimension 0; adding delta to q[..., 0] shifts all
    scores by softmax_scale * k_scale * 127 * delta.  Output unchanged, lse
    shifted by that amount."""
    x = tiny(24, n_sel=25, pool_cells=128, n_qheads=2, head_dim=8)
    kc = x.k_codes.copy()
    kc[:, 0] = 127
    ks = np.full_like(x.k_scales, np.float16(0.25).view(np.uint16))
    x = dataclasses.replace(x, k_codes=kc, k_scales=ks)
    delta = 3.0
    q2 = x.q.copy()
    q2[..., 0] += np.float32(delta)
    shift = (1.0 / 16.0) * 0.25 * 127 * (float(q2[0, 0, 0, 0]) - float(x.q[0, 0, 0, 0]))
    y = dataclasses.replace(x, q=q2)
    a, b = _attend_flat(O, x), _attend_flat(O, y)
    _close(b[0], a[0], 1e-12, 1e-15, "shift out")
    for r in range(a[1].shape[1]):
        s_r = (1.0 / 16.0) * 0.25 * 127 * (float(q2[0].reshape(-1, 8)[r, 0])
                                            - float(x.q[0].reshape(-1, 8)[r, 0]))
        _close(b[1][0, r], a[1][0, r] + s_r, 1e-13, 0, "shift lse")
    assert shift != 0


def pin_relabel_pages(O):
    """Moving physical pages and rewriting the table leaves results unchanged."""
    x = tiny(25, n_sel=40, pool_cells=256, n_q=2)
    n_pages = x.k_codes.shape[0] // 16
    perm = np.random.default_rng(7).permutation(n_pages)  # new page p holds old page perm[p]
    inv = np.argsort(perm)
    def mv(a, w):
        return np.ascontiguousarray(a.reshape(n_pages, 16, *a.shape[1:])[perm].reshape(a.shape))
    y = dataclasses.replace(x, k_codes=mv(x.k_codes, 1), v_codes=mv(x.v_codes, 1),
                            k_scales=mv(x.k_scales, 0), v_scales=mv(x.v_scales, 0),
                            page_table=inv[x.page_table].astype(np.int32))
    a, b = _attend_flat(O, x), _attend_flat(O, y)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_mask_equals_delete(O):
    x = tiny(26, n_sel=60, pool_cells=256)
    lp = x.sel[0] // 16
    victim = int(lp[10])
    pt = x.page_table.copy()
    pt[0, victim] = -1
    masked = dataclasses.replace(x, page_table=pt)
    keep = x.sel[0][lp != victim]
    deleted = dataclasses.replace(x, sel=keep[None].copy(),
                                  n_sel=np.array([keep.size], np.int32))
    a, b = _attend_flat(O, masked), _attend_flat(O, deleted)
    _close(a[0], b[0], 1e-13, 1e-16, "mask=delete out")
    _close(a[1], b[1], 1e-14, 0, "mask=delete lse")


def pin_double_v_scales(O):
    x = tiny(27, n_sel=30, pool_cells=128, n_q=2)
    vs2 = (f16(x.v_scales) * 2).astype(np.float16).view(np.uint16)
    y = dataclasses.replace(x, v_scales=vs2)
    a, b = _attend_flat(O, x), _attend_flat(O, y)
    assert np.array_equal(b[0], 2 * a[0]) and np.array_equal(b[1], a[1])


def pin_duplicates(O):
    """An entry listed twice counts twice: [c, c] gives lse = s + ln 2 and the
    same output as [c]."""
    x = tiny(28, n_sel=1)
    y = dataclasses.replace(x, sel=np.repeat(x.sel, 2, axis=1), n_sel=np.array([2], np.int32))
    a, b = _attend_flat(O, x), _attend_flat(O, y)
    _close(b[0], a[0], 1e-15, 0, "dup out")
    _close(b[1], a[1] + math.log(2), 1e-14, 0, "dup lse")


def _brute(x, subset, page_table):
    """Attention over the logical cells in `subset` with plain Python scalar
    arithmetic (math.fsum, math.exp): no numpy contraction, no oracle code."""
    D = x.q.shape[-1]
    Q = x.q[0].reshape(-1, D)
    kc, vc = x.k_codes, x.v_codes
    ks, vs = f16(x.k_scales), f16(x.v_scales)
    cells = []
    for c in subset:
        pp = int(page_table[c // 16])
        if 0 <= pp < kc.shape[0] // 16:
            cells.append(pp * 16 + c % 16)
    outs, lses = [], []
    for r in range(Q.shape[0]):
        q = [float(v) for v in Q[r]]
        if not cells:
            outs.append([0.0] * D)
            lses.append(-math.inf)
            continue
        s = [float(x.softmax_scale) * float(ks[ph]) * math.fsum(q[d] * int(kc[ph, d]) for d in range(D))
             for ph in cells]
        m = max(s)
        w = [math.exp(v - m) for v in s]
        L = math.fsum(w)
        outs.append([math.fsum(w[j] * float(vs[ph]) * int(vc[ph, d]) for j, ph in enumerate(cells)) / L
                     for d in range(D)])
        lses.append(m + math.log(L))
    return np.array(outs), np.array(lses)


def pin_brute_force_subsets(O):
    """Every subset of one or two cells of a 32-cell pool (two pages, one of
    them masked in a second table), and 150 random subsets of 3..8 cells,
    each against _brute.  All subsets run as instances of one oracle call."""
    import itertools
    x = tiny(29, pool_cells=32, n_sel=1, n_q=2, n_qheads=2, head_dim=8)
    rng = np.random.default_rng(2929)
    subsets = [list(c) for k in (1, 2) for c in itertools.combinations(range(32), k)]
    subsets += [sorted(rng.choice(32, size=int(k), replace=False).tolist())
                for k in rng.integers(3, 9, size=150)]
    for masked in (False, True):
        pt = x.page_table[0].copy()
        if masked:
            pt[1] = -1
        n = len(subsets)
        sel = np.zeros((n, 8), np.int32)
        for i, sub in enumerate(subsets):
            sel[i, : len(sub)] = sub
        y = dataclasses.replace(
            x, page_table=np.repeat(pt[None], n, 0), sel=sel,
            n_sel=np.array([len(sb) for sb in subsets], np.int32),
            q=np.ascontiguousarray(np.repeat(x.q, n, 0)))
        out, lse = _attend_flat(O, y)
        for i, sub in enumerate(subsets):
            ro, rl = _brute(x, sub, pt)
            _close(out[i], ro, 1e-12, 1e-14, f"brute out {sub} masked={masked}")
            _close(lse[i], rl, 1e-12, 1e-14, f"brute lse {sub} masked={masked}")


# ------------------------------------------------------------ prompt attention
def tiny_prompt(seed, pos0=None, **kw):
    spec = dict(n_inst=1, n_q=6, n_qheads=3, head_dim=8, pool_cells=64)
    spec.update(kw)
    return gen.make_prompt(None, seed=seed, pos0=pos0, **spec)


def textbook_prompt(x, i):
    """Causal softmax attention over the dense dequantised logical view built
    with numpy (as in textbook()): row (t, h) sees the logical cells
    c <= pos0 + t that lie on unmasked pages; scipy's softmax and logsumexp."""
    D = x.q.shape[-1]
    n_pages_phys = x.k_codes.shape[0] // 16
    Kp = (x.k_codes.astype(np.float64) * f16(x.k_scales)[:, None]).reshape(n_pages_phys, 16, D)
    Vp = (x.v_codes.astype(np.float64) * f16(x.v_scales)[:, None]).reshape(n_pages_phys, 16, D)
    pt = np.asarray(x.page_table[i], np.int64)
    page_ok = (pt >= 0) & (pt < n_pages_phys)
    safe = np.where(page_ok, pt, 0)
    Klog = Kp[safe].reshape(-1, D)
    Vlog = Vp[safe].reshape(-1, D)
    ok_log = np.repeat(page_ok, 16)
    n_q, nh = x.q.shape[1], x.q.shape[2]
    Q = np.asarray(x.q[i], np.float64).reshape(-1, D)
    pos = int(x.pos0[i]) + np.repeat(np.arange(n_q), nh)
    visible = (np.arange(Klog.shape[0])[None, :] <= pos[:, None]) & ok_log[None, :]
    S = np.where(visible, float(x.softmax_scale) * (Q @ Klog.T), -np.inf)
    out = np.zeros((Q.shape[0], D))
    lse = np.full((Q.shape[0],), -np.inf)
    live = visible.any(axis=1)
    if live.any():
        out[live] = scipy.special.softmax(S[live], axis=1) @ Vlog
        lse[live] = scipy.special.logsumexp(S[live], axis=1)
    return out.reshape(n_q, nh, D), lse.reshape(n_q, nh)


def pin_prompt_textbook(O):
    cases = [
        tiny_prompt(31),                                               # last 6 cells of the pool
        tiny_prompt(32, pos0=0, n_q=5),                                # the first positions
        tiny_prompt(33, pos0=-2, n_q=4),                               # two positions see nothing
        tiny_prompt(34, pos0=60, n_q=8),                               # positions past the table
        tiny_prompt(35, n_q=20, n_qheads=12, head_dim=256, pool_cells=256),
        tiny_prompt(36, n_inst=2, pos0=[10, 40], n_q=7, n_qheads=5),   # instances apart
    ]
    x = tiny_prompt(37, n_q=30, pool_cells=128, pos0=70)
    pt = x.page_table.copy()
    pt[0, 2] = -1      # cells 32..47 masked
    pt[0, 4] = 9_999   # cells 64..79 out of the pool
    cases.append(dataclasses.replace(x, page_table=pt))
    for x in cases:
        for i in range(x.n_inst):
            out, lse = O.prompt_attend(x, i)
            ro, rl = textbook_prompt(x, i)
            _close(out, ro, 1e-12, 1e-14, "prompt textbook out")
            _close(lse, rl, 1e-12, 1e-14, "prompt textbook lse")


def pin_prompt_first_cell(O):
    """Position 0 sees cell 0 alone: out = its dequantised V row, lse = its
    score (scalar Python arithmetic)."""
    x = tiny_prompt(38, pos0=0, n_q=1)
    out, lse = O.prompt_attend(x, 0)
    ph = int(x.page_table[0, 0]) * 16
    ks, vs = float(f16(x.k_scales[ph])), float(f16(x.v_scales[ph]))
    for h in range(x.n_qheads):
        dot = sum(float(a) * float(b) for a, b in zip(x.q[0, 0, h], x.k_codes[ph]))
        s0 = float(x.softmax_scale) * ks * dot
        _close(lse[0, h], s0, 1e-13, 1e-15, "first cell lse")
        _close(out[0, h], [vs * float(v) for v in x.v_codes[ph]], 1e-15, 0.0, "first cell out")


def pin_prompt_is_decode_of_prefix(O):
    """Row (t, h) equals the decode result for the explicit selection 0..p."""
    x = tiny_prompt(39, n_q=9, n_qheads=4, pool_cells=96, pos0=50)
    out, lse = O.prompt_attend(x, 0)
    for t in range(x.n_q):
        p = int(x.pos0[0]) + t
        d = dataclasses.replace(x, sel=np.arange(p + 1, dtype=np.int32)[None, :],
                                n_sel=np.array([p + 1], np.int32),
                                q=np.ascontiguousarray(x.q[:, t:t + 1]))
        ro, rl = O.attend(d)
        assert np.array_equal(out[t], ro[0, 0]) and np.array_equal(lse[t], rl[0, 0]), t


def pin_prompt_causal(O):
    """Changing the K/V rows of cells after a position leaves every row at or
    before it bit for bit unchanged and changes the rows after it."""
    x = tiny_prompt(40, n_q=12, pool_cells=64, pos0=50)
    out, lse = O.prompt_attend(x, 0)
    cut = 55  # change logical cells 56..63
    phys = (x.page_table[0][np.arange(cut + 1, 64) // 16] * 16 + np.arange(cut + 1, 64) % 16)
    kc, vc = x.k_codes.copy(), x.v_codes.copy()
    kc[phys] = -kc[phys]
    vc[phys] = 127 - np.abs(vc[phys])
    y = dataclasses.replace(x, k_codes=kc, v_codes=vc)
    out2, lse2 = O.prompt_attend(y, 0)
    t_cut = cut - int(x.pos0[0])
    assert np.array_equal(out[: t_cut + 1], out2[: t_cut + 1])
    assert np.array_equal(lse[: t_cut + 1], lse2[: t_cut + 1])
    assert all(not np.array_equal(out[t], out2[t]) for t in range(t_cut + 1, x.n_q))


# ------------------------------------------------------------ KV append (INT8 quantisation)
def pin_half_encode(O):
    """binary16 rounding against numpy's float32 -> float16 conversion
    (round to nearest even): log-uniform magnitudes over the whole range,
    every tie between neighbouring binary16 values, subnormals, overflow."""
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-30, 17, 20000)).astype(np.float32)
    x = np.concatenate([mag, -mag])
    h = np.arange(0, 0x7c00, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    ties = (h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2  # exact in float32
    special = np.array([0.0, -0.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14, 65504, 65519.99,
                        65520, 1e30, -1e30, np.inf, -np.inf], np.float32)
    x = np.concatenate([x, ties.astype(np.float32), special])
    got = O.float_to_half(x)
    with np.errstate(over="ignore"):  # values past the binary16 range become inf, on purpose
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def _append_case(seed, n_new=40, D=256, cells=256, pos0=100, scale_stride=1, rows=None):
    rng = np.random.default_rng(seed)
    kc = rng.integers(-127, 128, size=(cells, D), dtype=np.int8)
    vc = rng.integers(-127, 128, size=(cells, D), dtype=np.int8)
    ks = rng.integers(0, 0x7c00, size=cells * scale_stride).astype(np.uint16)
    vs = rng.integers(0, 0x7c00, size=cells * scale_stride).astype(np.uint16)
    pt = rng.permutation(cells // 16).astype(np.int32)
    k_new = (rng.standard_normal((n_new, D)) * np.exp2(rng.uniform(-8, 8, (n_new, 1)))).astype(np.float32)
    v_new = (rng.standard_normal((n_new, D)) * np.exp2(rng.uniform(-8, 8, (n_new, 1)))).astype(np.float32)
    if rows is not None:
        for t, (k, v) in rows.items():
            k_new[t], v_new[t] = k, v
    return (kc, ks, vc, vs), pt, pos0, k_new, v_new


def _written(pt, pos0, n_new, n_phys_pages):
    """physical cell of every new row (-1: not written), from the page view."""
    out = []
    for t in range(n_new):
        c = pos0 + t
        lp = c // 16
        ok = 0 <= c and lp < pt.size and 0 <= pt[lp] < n_phys_pages
        out.append(int(pt[lp]) * 16 + c % 16 if ok else -1)
    return out


def pin_append_quantiser(O):
    """Per written row: the scale is the binary16 of amax/127 (float32), every
    code reconstructs its value within half a scale step, the largest |code|
    is 127; zero rows give scale 0 and zero codes; tiny rows a zero scale;
    huge rows a saturated scale and clamped codes."""
    D = 256
    rows = {0: (np.zeros(D, np.float32), np.zeros(D, np.float32)),
            1: (np.full(D, 1e-9, np.float32), np.linspace(-1e-7, 1e-7, D).astype(np.float32)),
            2: (np.linspace(-1e8, 1e8, D).astype(np.float32), np.full(D, 3e7, np.float32))}
    pool, pt, pos0, kn, vn = _append_case(11, rows=rows)
    kc, ks, vc, vs = O.kv_append(pool, pt, pt.size, pos0, kn, vn)
    for t, ph in enumerate(_written(pt, pos0, kn.shape[0], kc.shape[0] // 16)):
        assert ph >= 0
        for x, codes, s16 in ((kn[t], kc[ph], ks[ph]), (vn[t], vc[ph], vs[ph])):
            amax = np.float32(np.max(np.abs(x)))
            s32 = min(amax / np.float32(127), np.float32(65504))
            assert s16 == np.float32(s32).astype(np.float16).view(np.uint16), (t, s16)
            s = float(np.uint16(s16).view(np.float16))
            if s == 0:
                assert not codes.any()
                continue
            q = codes.astype(np.float64)
            clipped = np.abs(x.astype(np.float64) / s) > 127.5
            err = np.abs(x.astype(np.float64) - q * s)
            assert np.all(err[~clipped] <= s / 2 * (1 + 1e-6)), (t, err.max() / s)
            assert np.all(np.abs(q[clipped]) == 127)
            assert np.max(np.abs(q)) == 127, t
    assert ks[_written(pt, pos0, 3, kc.shape[0] // 16)[2]] == 0x7bff  # saturated


def pin_append_exact_rows(O):
    """Rows that are integer multiples k * s of a binary16 step s with
    max |k| = 127 come back as exactly k and s."""
    rng = np.random.default_rng(12)
    D, n = 256, 24
    rows = {}
    for t in range(n):
        while True:
            s = np.float16(np.exp2(rng.uniform(-12, 6))).astype(np.float32)
            if np.float32(np.float32(127) * s / np.float32(127)).astype(np.float16) == s:
                break
        k = rng.integers(-127, 128, D)
        k[rng.integers(D)] = 127 * rng.choice([-1, 1])
        rows[t] = ((k * s).astype(np.float32), (-k * s).astype(np.float32))
    pool, pt, pos0, kn, vn = _append_case(13, n_new=n, rows=rows)
    kc, ks, vc, vs = O.kv_append(pool, pt, pt.size, pos0, kn, vn)
    for t, ph in enumerate(_written(pt, pos0, n, kc.shape[0] // 16)):
        s = kn[t][np.argmax(np.abs(kn[t]))] / 127
        assert np.array_equal(kc[ph].astype(np.float32) * abs(s), kn[t]), t
        assert np.array_equal(vc[ph], -kc[ph])
        assert ks[ph] == vs[ph] == np.float32(abs(s)).astype(np.float16).view(np.uint16)


def pin_append_placement(O):
    """Rows land on the page view's physical cells and nowhere else: cells of
    masked pages, rows past the table and rows before position 0 are not
    written; with interleaved (K, V) scale pairs (stride 2) the scales go to
    the pair of their cell."""
    for pos0, n_new, stride in ((100, 40, 1), (-5, 20, 1), (230, 40, 1), (37, 90, 2)):
        pool, pt, _, kn, vn = _append_case(14 + pos0 % 7, n_new=n_new, pos0=pos0,
                                           scale_stride=stride)
        pt = pt.copy()
        pt[3] = -1
        pt[9] = 10_000
        kc, ks, vc, vs = O.kv_append(pool, pt, pt.size, pos0, kn, vn, scale_stride=stride)
        dest = _written(pt, pos0, n_new, kc.shape[0] // 16)
        written = sorted(p for p in dest if p >= 0)
        changed = np.flatnonzero((kc != pool[0]).any(axis=1) | (vc != pool[2]).any(axis=1))
        assert set(changed) <= set(written)
        keep = np.setdiff1d(np.arange(kc.shape[0]), written)
        assert np.array_equal(kc[keep], pool[0][keep]) and np.array_equal(vc[keep], pool[2][keep])
        sk = np.setdiff1d(np.arange(ks.size), [p * stride for p in written])
        assert np.array_equal(ks[sk], pool[1][sk]) and np.array_equal(vs[sk], pool[3][sk])
        for t, ph in enumerate(dest):
            if ph < 0:
                continue
            amax = np.max(np.abs(kn[t]))
            assert ks[ph * stride] == np.float32(amax / np.float32(127)).astype(np.float16).view(np.uint16)
            assert abs(int(kc[ph][np.argmax(np.abs(kn[t]))])) == 127  # this row, not another


def pin_append_then_attend(O):
    """A row appended and then attended to alone: out is its dequantised V
    row, within half a scale step of the appended values; lse is the score
    of the dequantised K row, within the error those steps allow."""
    D = 256
    pool, pt, pos0, kn, vn = _append_case(15, n_new=1, D=D, pos0=77)
    kc, ks, vc, vs = O.kv_append(pool, pt, pt.size, pos0, kn, vn)
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 1, 3, D)).astype(np.float32)
    x = gen.Inputs(k_codes=kc, v_codes=vc, k_scales=ks, v_scales=vs,
                   page_table=pt[None, :], sel=np.array([[pos0]], np.int32),
                   n_sel=np.array([1], np.int32), q=q, softmax_scale=1 / 16, chunk=64,
                   workload="append_then_attend", seed=0)
    out, lse = O.attend(x)
    sv = float(np.uint16(vs[_written(pt, pos0, 1, kc.shape[0] // 16)[0]]).view(np.float16))
    sk = float(np.uint16(ks[_written(pt, pos0, 1, kc.shape[0] // 16)[0]]).view(np.float16))
    for h in range(3):
        assert np.all(np.abs(out[0, 0, h] - vn[0]) <= sv / 2 * (1 + 1e-6))
        exact = float(q[0, 0, h].astype(np.float64) @ kn[0].astype(np.float64)) / 16
        bound = np.sum(np.abs(q[0, 0, h].astype(np.float64))) * sk / 2 / 16
        assert abs(lse[0, 0, h] - exact) <= bound * (1 + 1e-6) + 1e-12


# ----------------------------------------------------------------------------
# QSA block scorer and top-k selection.  Readings (the pages give only the
# scorer's arguments and tests): score = sum over indexer heads of the dot
# product of the row's indexer query with the block's pooled key, -inf for a
# dead block or one whose first cell the row cannot see; selection = the k
# blocks with the highest maximum-over-rows score, equal scores by increasing
# block index, expanded to their cells below the largest row extent.

def qsa_case(pooled, q, dead, n_visible, R, k):
    return gen.QsaInputs(pooled=np.asarray(pooled, np.float32), dead=np.asarray(dead, np.uint8),
                         q_idx=np.asarray(q, np.float32),
                         n_visible=np.asarray(n_visible, np.int32), block_cells=R, k_blocks=k,
                         workload="pin", seed=0)


def pin_qsa_hand_example(O):
    """Two rows, two heads of two dims, four 16-cell blocks, worked out by
    hand: row 0 sees 40 cells (blocks 0-2), row 1 all 64; block 2 is dead.
    Row 0: b0 = (1+2) + 0 = 3, b1 = 3 + 2 = 5.  Row 1: b0 = 2 + 1 = 3,
    b1 = 0 + 0 = 0, b3 = 4 + 2 = 6.  Combined: b0 3, b1 5, b3 6."""
    pooled = [[[1, 2], [0, -1]], [[3, 0], [1, 1]], [[5, 5], [5, 5]], [[-1, 4], [2, 0]]]
    q = [[[1, 1], [2, 0]], [[0, 1], [1, -1]]]
    x = qsa_case([pooled], [q], [[0, 0, 1, 0]], [[40, 64]], 16, 2)
    ninf = -np.inf
    want = np.array([[[3, 5, ninf, ninf], [3, 0, ninf, 6]]])
    assert np.array_equal(O.qsa_scores(x), want)
    s = O.qsa_scores(x)
    for k, blocks in ((2, [1, 3]), (3, [0, 1, 3]), (4, [0, 1, 3]), (1, [3]), (0, [])):
        sel, n = O.qsa_select(s, x.n_visible, 16, k)
        cells = [c for b in blocks for c in range(16 * b, 16 * b + 16)]
        assert n[0] == len(cells) and list(sel[0, :n[0]]) == cells, (k, sel[0, :n[0]])
    # row 1 sees 52 cells: block 3 contributes cells 48..51 only
    sel, n = O.qsa_select(s, np.array([[40, 52]]), 16, 2)
    assert list(sel[0, :n[0]]) == list(range(16, 32)) + [48, 49, 50, 51]


def pin_qsa_unit_queries(O):
    """A query that is a unit vector on (head h, dim d) scores each live
    block with that component of its pooled key."""
    rng = np.random.default_rng(61)
    B, H, D = 9, 3, 8
    pooled = rng.standard_normal((1, B, H, D)).astype(np.float32)
    for h, d in ((0, 0), (2, 7), (1, 3)):
        q = np.zeros((1, 1, H, D), np.float32)
        q[0, 0, h, d] = 1
        x = qsa_case(pooled, q, np.zeros((1, B)), [[B * 32]], 32, 3)
        assert np.array_equal(O.qsa_scores(x)[0, 0], pooled[0, :, h, d].astype(np.float64))


def pin_qsa_linearity(O):
    """Scores are linear in the query: s(q1) + s(q2) = s(q1 + q2) and
    s(-2 q) = -2 s(q), exactly for small-integer inputs."""
    rng = np.random.default_rng(62)
    B, H, D = 12, 2, 16
    pooled = rng.integers(-8, 9, (1, B, H, D)).astype(np.float32)
    q1 = rng.integers(-8, 9, (1, 1, H, D)).astype(np.float32)
    q2 = rng.integers(-8, 9, (1, 1, H, D)).astype(np.float32)
    mk = lambda q: O.qsa_scores(qsa_case(pooled, q, np.zeros((1, B)), [[B * 16]], 16, 1))
    assert np.array_equal(mk(q1) + mk(q2), mk(q1 + q2))
    assert np.array_equal(mk(-2 * q1), -2 * mk(q1))


def pin_qsa_heads_add(O):
    """The score is the sum of the per-head scores (each head scored as a
    one-head scorer on its slice), and permuting the heads of both the query
    and the keys changes nothing."""
    rng = np.random.default_rng(63)
    B, H, D = 10, 4, 8
    pooled = rng.integers(-5, 6, (1, B, H, D)).astype(np.float32)
    q = rng.integers(-5, 6, (1, 2, H, D)).astype(np.float32)
    vis = [[B * 16, B * 16]]
    full = O.qsa_scores(qsa_case(pooled, q, np.zeros((1, B)), vis, 16, 1))
    parts = sum(O.qsa_scores(qsa_case(pooled[:, :, h:h + 1], q[:, :, h:h + 1], np.zeros((1, B)),
                                      vis, 16, 1)) for h in range(H))
    assert np.array_equal(full, parts)
    perm = [2, 0, 3, 1]
    permuted = O.qsa_scores(qsa_case(pooled[:, :, perm], q[:, :, perm], np.zeros((1, B)), vis, 16, 1))
    assert np.array_equal(full, permuted)


def pin_qsa_masks(O):
    """A dead block scores -inf for every row; block b is visible to a row
    exactly when b * R < n_visible (boundaries R b and R b + 1)."""
    rng = np.random.default_rng(64)
    B, H, D, R = 6, 1, 4, 16
    pooled = rng.standard_normal((1, B, H, D)).astype(np.float32)
    q = rng.standard_normal((1, 3, H, D)).astype(np.float32)
    dead = np.zeros((1, B))
    dead[0, 4] = 1
    x = qsa_case(pooled, q, dead, [[3 * R, 3 * R + 1, 0]], R, 2)
    s = O.qsa_scores(x)
    assert np.all(np.isneginf(s[0, :, 4]))
    assert np.all(np.isfinite(s[0, 0, :3])) and np.all(np.isneginf(s[0, 0, 3:]))
    assert np.all(np.isfinite(s[0, 1, :4])) and np.all(np.isneginf(s[0, 1, 4:]))
    assert np.all(np.isneginf(s[0, 2]))


def _numpy_select(scores, n_visible, R, k):
    """Top-k with numpy: lexsort by (-combined score, block index)."""
    n_inst, _, B = scores.shape
    out = []
    for i in range(n_inst):
        c = scores[i].max(axis=0)
        order = np.lexsort((np.arange(B), -c))
        blocks = sorted(int(b) for b in order[:k] if c[b] > -np.inf)
        ext = min(int(np.max(n_visible[i])), B * R)
        out.append([cell for b in blocks for cell in range(b * R, min(b * R + R, ext))])
    return out


def pin_qsa_select_numpy(O):
    """Selection against numpy's lexsort on random scores with injected
    ties, -inf entries, partial last blocks and several k."""
    rng = np.random.default_rng(65)
    for trial in range(12):
        n_inst, n_rows, B, R = 3, int(rng.integers(1, 5)), int(rng.integers(1, 40)), 16
        sc = rng.integers(-6, 7, (n_inst, n_rows, B)).astype(np.float64)  # many ties
        sc[rng.random(sc.shape) < 0.2] = -np.inf
        vis = rng.integers(0, B * R + 30, (n_inst, n_rows))
        for k in (0, 1, 3, B // 2, B, B + 2):
            sel, n = O.qsa_select(sc, vis, R, k)
            want = _numpy_select(sc, vis, R, k)
            for i in range(n_inst):
                assert list(sel[i, :n[i]]) == want[i], (trial, k, i)


def pin_qsa_select_brute(O):
    """Brute force on tiny inputs: among all block subsets of size
    min(k, live blocks), exactly one ranks every member above every
    non-member (higher score, or equal score and lower index); the oracle's
    selection is that subset."""
    import itertools
    rng = np.random.default_rng(66)
    for trial in range(40):
        B, R = int(rng.integers(1, 8)), 16
        sc = rng.integers(-3, 4, (1, 2, B)).astype(np.float64)
        sc[rng.random(sc.shape) < 0.3] = -np.inf
        c = sc[0].max(axis=0)
        live = [b for b in range(B) if c[b] > -np.inf]
        k = int(rng.integers(0, B + 2))
        kk = min(k, len(live))
        above = lambda s, u: c[s] > c[u] or (c[s] == c[u] and s < u)
        good = [set(S) for S in itertools.combinations(live, kk)
                if all(above(s, u) for s in S for u in live if u not in S)]
        assert len(good) == 1
        sel, n = O.qsa_select(sc, np.array([[B * R, B * R]]), R, k)
        got = sorted({int(v) // R for v in sel[0, :n[0]]})
        assert got == sorted(good[0]), (trial, got, good)


def pin_qsa_select_special(O):
    """All scores equal: the lowest k blocks.  No live block: nothing.  k at
    least the live count: every live block.  Extent 0: no cells."""
    B, R = 10, 32
    sel, n = O.qsa_select(np.zeros((1, 3, B)), np.array([[B * R] * 3]), R, 4)
    assert list(sel[0, :n[0]]) == list(range(4 * R))
    sel, n = O.qsa_select(np.full((2, 1, B), -np.inf), np.array([[B * R], [B * R]]), R, 4)
    assert list(n) == [0, 0]
    sc = np.full((1, 1, B), -np.inf)
    sc[0, 0, [7, 2, 5]] = [1.0, -3.0, 0.5]
    sel, n = O.qsa_select(sc, np.array([[B * R]]), R, 9)
    assert list(sel[0, :n[0]]) == [c for b in (2, 5, 7) for c in range(b * R, b * R + R)]
    sel, n = O.qsa_select(sc, np.array([[0]]), R, 9)
    assert n[0] == 0


ALL_PINS = [pin_half_decode, pin_textbook, pin_gather_exhaustive, pin_one_cell, pin_two_cells,
            pin_zero_query, pin_identical_keys, pin_worked_example, pin_merge_closed_form,
            pin_empty_and_masked, pin_permutation, pin_chunking, pin_score_shift,
            pin_relabel_pages, pin_mask_equals_delete, pin_double_v_scales, pin_duplicates,
            pin_brute_force_subsets, pin_prompt_textbook, pin_prompt_first_cell,
            pin_prompt_is_decode_of_prefix, pin_prompt_causal, pin_half_encode,
            pin_append_quantiser, pin_append_exact_rows, pin_append_placement,
            pin_append_then_attend, pin_qsa_hand_example, pin_qsa_unit_queries,
            pin_qsa_linearity, pin_qsa_heads_add, pin_qsa_masks, pin_qsa_select_numpy,
            pin_qsa_select_brute, pin_qsa_select_special]
