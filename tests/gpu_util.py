"""Helpers shared by the GPU tests: run the HIP path through the C ABI on
generated inputs and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances: elementwise |gpu - oracle| <= atol + rtol * |oracle|.
OUT_ATOL, OUT_RTOL = 1e-3, 1e-3
LSE_ATOL, LSE_RTOL = 1e-4, 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def assert_close(got, ref, atol, rtol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_ninf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both are -inf
        diff = np.where(both_ninf, 0.0, np.abs(got - ref))
    tol = atol + rtol * np.where(both_ninf, 0.0, np.abs(ref))
    bad = ~(diff <= tol)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, diff - tol, -np.inf)), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
                             f"{idx}: got {got[idx]!r} ref {ref[idx]!r}; max|diff| {diff.max():.3e}")
    return float(diff.max()) if diff.size else 0.0


def run_batch(x, chunk=None, n_q=None, gather=True, device="cuda", interleave=False):
    """Upload inputs and run sda_decode_attn_batch; returns numpy out, lse,
    gather indices and the device workspace.  interleave: store the K and V
    scales as (K, V) pairs per cell (scale_stride 2)."""
    import torch
    from decode_attention_sparse_amd import api
    if n_q is not None:
        x = x.with_n_q(n_q)
    chunk = chunk or x.chunk
    pool, dev = api.to_device(x, device, interleave_scales=interleave)
    n_inst, nq, nh, D = x.q.shape
    out = torch.full((n_inst, nq, nh, D), float("nan"), device=device)
    lse = torch.full((n_inst, nq, nh), float("nan"), device=device)
    g = torch.full(x.sel.shape, -7, dtype=torch.int32, device=device) if gather else None
    max_sel = int(x.sel.shape[1])
    ws = api.decode_attn_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], max_sel,
                               dev["q"], x.softmax_scale, chunk, out, lse, gather_out=g)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(), None if g is None else g.cpu().numpy(), ws)


def check(x, out, lse, g=None, inst_ids=None, what="", strict_out=True, strict_lse=True):
    """The outputs (and gather indices) of a decode call against the oracle,
    on all instances or the sampled inst_ids (and finite on all of them).  Beyond the elementwise
    atol + rtol |ref| bound, strict_out / strict_lse assert the absolute
    bounds alone (max |dout| <= 1e-3, max |dlse| <= 1e-4), which float32
    meets wherever |lse| stays below about 100 (scores far larger, as in the
    heavy-tailed batched workload, leave float32 itself short of 1e-4)."""
    import oracle
    # every row of every instance, sampled or not: a finite output (a kernel
    # that gives up on a bounded wait writes NaN rows and still returns OK;
    # lse is -inf only for rows with no visible cell)
    assert np.isfinite(out).all(), f"{what}: non-finite outputs"
    assert not (np.isnan(lse).any() or np.isposinf(lse).any()), f"{what}: NaN or +inf lse"
    ro, rl = oracle.attend(x, inst_ids)
    sl = slice(None) if inst_ids is None else np.asarray(inst_ids)
    e1 = assert_close(out[sl], ro, OUT_ATOL, OUT_RTOL, f"{what} out")
    e2 = assert_close(lse[sl], rl, LSE_ATOL, LSE_RTOL, f"{what} lse")
    if g is not None:
        rg = oracle.gather(x)
        valid = np.arange(x.sel.shape[1])[None, :] < x.n_sel[:, None]
        assert np.array_equal(g[valid], rg[valid]), f"{what}: gather indices differ"
    say(f"  {what}: max|dout| {e1:.2e} ({e1 / OUT_ATOL:.1%} of {OUT_ATOL:g}), max|dlse| {e2:.2e} "
        f"({e2 / LSE_ATOL:.1%} of {LSE_ATOL:g})")
    if strict_out:
        assert e1 <= OUT_ATOL, f"{what}: max|dout| {e1:.3e} above {OUT_ATOL}"
    if strict_lse:
        assert e2 <= LSE_ATOL, f"{what}: max|dlse| {e2:.3e} above {LSE_ATOL}"
    return e1, e2


def two_pass(x, chunk, gather=True):
    """sda_chunk_batch then sda_merge_batch at the given chunk size."""
    import torch
    from decode_attention_sparse_amd import api
    n_inst, n_q, nh, D = x.q.shape
    max_sel = int(x.sel.shape[1])
    pool, dev = api.to_device(x)
    ws = api.workspace(n_inst, n_q, nh, max_sel, chunk)
    out = torch.full((n_inst, n_q, nh, D), float("nan"), device="cuda")
    lse = torch.full((n_inst, n_q, nh), float("nan"), device="cuda")
    g = torch.full(x.sel.shape, -7, dtype=torch.int32, device="cuda") if gather else None
    api.chunk_batch(pool, dev["page_table"], dev["sel"], dev["n_sel"], max_sel, dev["q"],
                    x.softmax_scale, chunk, ws, gather_out=g)
    api.merge_batch(dev["n_sel"], max_sel, chunk, ws, out, lse)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(), None if g is None else g.cpu().numpy(), ws)


def run_prompt(x, device="cuda", interleave=False):
    """Upload prompt inputs and run sda_prompt_attn_batch; returns numpy out
    [n_inst][n_q][n_qheads][D] and lse [n_inst][n_q][n_qheads]."""
    import torch
    from decode_attention_sparse_amd import api
    pool, dev = api.to_device(x, device, interleave_scales=interleave)
    out = torch.full(x.q.shape, float("nan"), device=device)
    lse = torch.full(x.q.shape[:3], float("nan"), device=device)
    api.prompt_attn_batch(pool, dev["page_table"], dev["pos0"], dev["q"], x.softmax_scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def f32_attend(q, k_hat, v_hat, scale, visible=None):
    """Plain float32 softmax attention (numpy float32 products and sums) over
    dequantised rows: the error level a float32 computation reaches."""
    s = (q @ k_hat.T) * np.float32(scale)
    if visible is not None:
        s = np.where(visible, s, np.float32(-np.inf))
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True, dtype=np.float32)
    return (p @ v_hat) / l, (m + np.log(l))[:, 0]


def dequant(codes, scales, phys):
    """float32 rows code * scale of the physical cells phys (-1: a zero row)."""
    ok = phys >= 0
    rows = np.where(ok[:, None], codes[np.where(ok, phys, 0)].astype(np.float32), np.float32(0))
    return rows * scales[np.where(ok, phys, 0)].view(np.float16).astype(np.float32)[:, None]


# GPU error may exceed a float32 computation's by at most this factor
F32_FACTOR = 4.0


def f32_online(q, k_hat, v_hat, scale, visible=None, tile=64):
    """float32 attention in the order a tiled kernel takes: per tile of
    cells the scores, its maximum and probabilities (numpy float32), the
    running maximum, denominator and accumulator rescaled and accumulated
    tile after tile: the error level of a plain float32 online softmax."""
    R, N = q.shape[0], k_hat.shape[0]
    m = np.full(R, -np.inf, np.float32)
    l = np.zeros(R, np.float32)
    acc = np.zeros((R, v_hat.shape[1]), np.float32)
    for t0 in range(0, N, tile):
        s = (q @ k_hat[t0:t0 + tile].T) * np.float32(scale)
        if visible is not None:
            s = np.where(visible[:, t0:t0 + tile], s, np.float32(-np.inf))
        m_new = np.maximum(m, s.max(axis=1))
        ref = np.where(np.isneginf(m_new), np.float32(0), m_new)
        corr = np.where(np.isneginf(m), np.float32(0), np.exp(m - ref)).astype(np.float32)
        p = np.exp(s - ref[:, None]).astype(np.float32)
        l = l * corr + p.sum(axis=1, dtype=np.float32)
        acc = acc * corr[:, None] + p @ v_hat[t0:t0 + tile]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        return acc / l[:, None], m + np.log(l)
