"""Seeded synthetic inputs for selected-cell INT8 decode attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no gather, no dot product, no softmax).  Both the CPU
oracle (through the tests and the bench's CPU leg) and the HIP path consume
exactly the arrays produced here.

Workload shapes follow the kernel benchmark on the Strata PR #2220 page
("Kernel (chunk kernel + merge, synthetic INT8 pools, permuted page table,
200 calls)"): INT8 K/V pools behind a permuted page table, 12 query heads per
KV head with head_dim 256 (the PR's description of one lane holding 8 dims of
each of the 12 heads across a 32-lane warp), 1-4 query positions (MTP verify
positions), 600 or 2,051 selected cells.

Layout produced (all numpy, C-contiguous):

  k_codes, v_codes  int8   [n_inst * pool_cells, head_dim]  one global pool;
                           instance i physically owns pages
                           [i*pages, (i+1)*pages)
  k_scales, v_scales uint16 [n_inst * pool_cells]  IEEE binary16 bit patterns,
                           one scale per physical cell
  page_table        int32  [n_inst, pages]  global physical page id per
                           logical page (a random permutation of the
                           instance's own pages); -1 would mask a page
  sel               int32  [n_inst, n_sel]  selected logical cell ids
  n_sel             int32  [n_inst]
  q                 float32 [n_inst, n_q, n_qheads, head_dim]

Random streams: numpy Generator(PCG64); the config seed is 20261200 + cfg
unless given; instance i draws from SeedSequence(seed).spawn(n_inst)[i] in a
fixed order (page permutation, selection, K codes, V codes, K scales,
V scales, heavy-tail offsets, q), so any instance can be regenerated alone.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

PAGE_SIZE = 16
HEAD_DIM = 256
N_QHEADS = 12
SOFTMAX_SCALE = 1.0 / 16.0
SCALE_LO, SCALE_HI = 0.002, 0.02

# The five workloads.  "chunk" is the chunk size in selected cells; the batched
# decode workload leaves it open, so a value is chosen here (see DEFAULT_CHUNK_2).
DEFAULT_CHUNK_2 = 1024

CONFIGS = {
    0: dict(workload="tiny_single_step", n_inst=1, n_q=1, pool_cells=4096,
            n_sel=600, sel="uniform", heavy=False, chunk=256),
    1: dict(workload="pages_kernel_point_2051x1-4q", n_inst=1, n_q=4,
            pool_cells=32768, n_sel=2051, sel="uniform", heavy=False, chunk=256),
    2: dict(workload="batched_decode_256inst_2051x4q", n_inst=256, n_q=4,
            pool_cells=32768, n_sel=2051, sel="uniform", heavy=True,
            chunk=DEFAULT_CHUNK_2),
    3: dict(workload="long_context_runs_64inst_16384x2q", n_inst=64, n_q=2,
            pool_cells=131072, n_sel=16384, sel="runs", heavy=False, chunk=512,
            n_runs=64, run_len=256),
    4: dict(workload="dense_fallback_32inst_131072x4q", n_inst=32, n_q=4,
            pool_cells=131072, n_sel=131072, sel="all", heavy=False, chunk=1024),
}


@dataclasses.dataclass
class Inputs:
    k_codes: np.ndarray
    v_codes: np.ndarray
    k_scales: np.ndarray
    v_scales: np.ndarray
    page_table: np.ndarray
    sel: np.ndarray
    n_sel: np.ndarray
    q: np.ndarray
    softmax_scale: float
    chunk: int
    workload: str
    seed: int

    @property
    def n_inst(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def n_qheads(self) -> int:
        return int(self.q.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[3])

    @property
    def n_logical_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def n_phys_pages(self) -> int:
        return int(self.k_codes.shape[0] // PAGE_SIZE)

    def with_n_q(self, n_q: int) -> "Inputs":
        """View with the first n_q query positions (same pools and selection)."""
        return dataclasses.replace(self, q=np.ascontiguousarray(self.q[:, :n_q]))


def config_seed(cfg: int) -> int:
    return 20261200 + int(cfg)


def _draw_selection(rng, mode, pool_cells, n_sel, spec):
    if mode == "uniform":
        s = rng.choice(pool_cells, size=n_sel, replace=False)
        return np.sort(s).astype(np.int32)
    if mode == "all":
        return np.arange(pool_cells, dtype=np.int32)[:n_sel]
    if mode == "runs":
        # n_runs non-overlapping runs of run_len cells at random offsets: the
        # unselected cells are cut into n_runs+1 gaps at sorted uniform points
        # and run k starts after gap k.  Gaps may be empty (runs may touch).
        n_runs, run_len = spec["n_runs"], spec["run_len"]
        assert n_runs * run_len == n_sel
        free = pool_cells - n_sel
        cuts = np.sort(rng.integers(0, free, size=n_runs, endpoint=True))
        starts = cuts + run_len * np.arange(n_runs)
        s = (starts[:, None] + np.arange(run_len)[None, :]).reshape(-1)
        return s.astype(np.int32)
    raise ValueError(mode)


def _fill_instance(i, ss, spec, out, heavy):
    rng = np.random.Generator(np.random.PCG64(ss))
    pool_cells = spec["pool_cells"]
    pages = pool_cells // PAGE_SIZE
    D = out["k_codes"].shape[1]
    lo, hi = i * pool_cells, (i + 1) * pool_cells
    out["page_table"][i] = (rng.permutation(pages) + i * pages).astype(np.int32)
    out["sel"][i] = _draw_selection(rng, spec["sel"], pool_cells, spec["n_sel"], spec)
    out["k_codes"][lo:hi] = rng.integers(-127, 127, size=(pool_cells, D),
                                         dtype=np.int8, endpoint=True)
    out["v_codes"][lo:hi] = rng.integers(-127, 127, size=(pool_cells, D),
                                         dtype=np.int8, endpoint=True)
    ks = rng.uniform(SCALE_LO, SCALE_HI, size=pool_cells)
    vs = rng.uniform(SCALE_LO, SCALE_HI, size=pool_cells)
    if heavy:
        # Heavy-tailed K scales: a per-cell N(0, sigma=3) offset added to the
        # (positive) scale magnitude; the sign is kept positive by taking the
        # magnitude of the sum.
        ks = np.abs(ks + rng.normal(0.0, 3.0, size=pool_cells))
    out["k_scales"][lo:hi] = ks.astype(np.float16).view(np.uint16)
    out["v_scales"][lo:hi] = vs.astype(np.float16).view(np.uint16)
    out["q"][i] = rng.standard_normal(size=out["q"].shape[1:], dtype=np.float32)


def make(cfg: int | None = None, seed: int | None = None, *, threads: int | None = None,
         **overrides) -> Inputs:
    """Generate the inputs of workload `cfg` (0-4), optionally with overrides.

    Overrides accept any key of CONFIGS[cfg] plus n_qheads / head_dim, e.g.
    make(1, n_sel=65, pool_cells=1024) for an edge case with a given seed.
    With cfg=None the overrides must give the whole spec.
    """
    spec = dict(CONFIGS[cfg]) if cfg is not None else {}
    spec.update(overrides)
    spec.setdefault("n_qheads", N_QHEADS)
    spec.setdefault("head_dim", HEAD_DIM)
    spec.setdefault("heavy", False)
    spec.setdefault("chunk", 256)
    spec.setdefault("workload", "custom")
    if seed is None:
        seed = config_seed(cfg if cfg is not None else 99)
    n_inst, pool_cells = int(spec["n_inst"]), int(spec["pool_cells"])
    if pool_cells % PAGE_SIZE:
        raise ValueError("pool_cells must be a multiple of the page size")
    n_sel, D = int(spec["n_sel"]), int(spec["head_dim"])
    if n_sel > pool_cells:
        raise ValueError("n_sel > pool_cells")
    pages = pool_cells // PAGE_SIZE
    total = n_inst * pool_cells
    out = dict(
        k_codes=np.empty((total, D), np.int8),
        v_codes=np.empty((total, D), np.int8),
        k_scales=np.empty((total,), np.uint16),
        v_scales=np.empty((total,), np.uint16),
        page_table=np.empty((n_inst, pages), np.int32),
        sel=np.empty((n_inst, n_sel), np.int32),
        q=np.empty((n_inst, int(spec["n_q"]), int(spec["n_qheads"]), D), np.float32),
    )
    children = np.random.SeedSequence(seed).spawn(n_inst)
    heavy = bool(spec["heavy"])
    if n_inst == 1:
        _fill_instance(0, children[0], spec, out, heavy)
    else:
        nt = threads or min(16, os.cpu_count() or 1)
        with _cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda i: _fill_instance(i, children[i], spec, out, heavy),
                        range(n_inst)))
    return Inputs(n_sel=np.full((n_inst,), n_sel, np.int32),
                  softmax_scale=SOFTMAX_SCALE, chunk=int(spec["chunk"]),
                  workload=str(spec["workload"]), seed=int(seed), **out)


# Prompt (many-query) attention over the same pools: the workload of the
# prompt attention parity test on the Strata PR #2220 page (an INT8 context
# of 32K cells and 2,048 queries per prompt chunk).  The chunk's own cells are
# the last n_q cells of the context, so query t sits at position
# pos0 + t with pos0 = pool_cells - n_q and sees cells 0..pos0 + t.
PROMPT_CONFIGS = {
    "prompt_int8_32k_2048q": dict(n_inst=1, n_q=2048, pool_cells=32768),
}


@dataclasses.dataclass
class PromptInputs(Inputs):
    pos0: np.ndarray = None  # int32 [n_inst]: position of query 0


def make_prompt(name: str | None = None, seed: int | None = None, pos0=None,
                **overrides) -> PromptInputs:
    """Pools, permuted page tables and queries drawn exactly as make() draws
    them (no selection list); pos0 defaults to pool_cells - n_q."""
    spec = dict(PROMPT_CONFIGS[name]) if name is not None else {"n_inst": 1}
    spec.update(overrides)
    spec.update(sel="all", n_sel=0, chunk=64)
    spec.setdefault("workload", name or "custom_prompt")
    x = make(None, seed=20261300 if seed is None else seed, **spec)
    n_inst = x.n_inst
    if pos0 is None:
        pos0 = np.full((n_inst,), int(spec["pool_cells"]) - x.n_q, np.int32)
    pos0 = np.broadcast_to(np.asarray(pos0, np.int32), (n_inst,)).copy()
    fields = {f.name: getattr(x, f.name) for f in dataclasses.fields(x)}  # no copies
    return PromptInputs(**fields, pos0=pos0)


# KV append (new K/V rows quantised into the pools).  The pages give no
# append workload; this one appends a prompt chunk of 2,048 rows to each of
# 64 (sequence, KV head) instances whose pools hold 32K cells, the new rows
# at the end of each context (pos0 = pool_cells - n_new).
APPEND_CONFIGS = {
    "kv_append_64inst_2048rows": dict(n_inst=64, n_new=2048, pool_cells=32768),
}


@dataclasses.dataclass
class AppendInputs:
    page_table: np.ndarray  # int32 [n_inst][pages]: a permutation of the instance's own pages
    pos0: np.ndarray        # int32 [n_inst]: logical cell of new row 0
    k_new: np.ndarray       # float32 [n_inst][n_new][head_dim]
    v_new: np.ndarray
    pool_cells: int         # cells per instance (pool = n_inst * pool_cells cells)
    workload: str
    seed: int

    @property
    def n_inst(self) -> int:
        return int(self.k_new.shape[0])

    @property
    def n_new(self) -> int:
        return int(self.k_new.shape[1])


def make_append(name: str | None = None, seed: int | None = None, pos0=None, spread: float = 8.0,
                k_spread: float | None = None, **overrides) -> AppendInputs:
    """Page tables drawn as make() draws them, new rows N(0, 1) scaled per row
    by 2^U(-spread, spread) (rows of very different magnitudes); k_spread,
    when given, replaces spread for the K rows (k_spread 0: K rows N(0, 1),
    so scores stay of order 1 and attention spreads over many cells)."""
    spec = dict(APPEND_CONFIGS[name]) if name is not None else {"n_inst": 1}
    spec.update(overrides)
    n_inst, n_new, cells = int(spec["n_inst"]), int(spec["n_new"]), int(spec["pool_cells"])
    D = int(spec.get("head_dim", HEAD_DIM))
    pages = cells // PAGE_SIZE
    seed = 20261400 if seed is None else seed
    children = np.random.SeedSequence(seed).spawn(n_inst)
    pt = np.empty((n_inst, pages), np.int32)
    k_new = np.empty((n_inst, n_new, D), np.float32)
    v_new = np.empty((n_inst, n_new, D), np.float32)
    def fill(i):
        rng = np.random.Generator(np.random.PCG64(children[i]))
        pt[i] = rng.permutation(pages) + i * pages
        for a, sp in ((k_new, spread if k_spread is None else k_spread), (v_new, spread)):
            a[i] = rng.standard_normal((n_new, D), dtype=np.float32)
            a[i] *= np.exp2(rng.uniform(-sp, sp, (n_new, 1))).astype(np.float32)

    with _cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n_inst)))
    if pos0 is None:
        pos0 = cells - n_new
    pos0 = np.broadcast_to(np.asarray(pos0, np.int32), (n_inst,)).copy()
    return AppendInputs(page_table=pt, pos0=pos0, k_new=k_new, v_new=v_new, pool_cells=cells,
                        workload=str(spec.get("workload", name or "custom_append")), seed=seed)


# QSA block scoring and selection (the step that produces the selected cell
# list).  The pages give the scorer's arguments (pooled block keys, dead
# flags, indexer queries, per-row extents) but not its geometry; the
# workload takes config 3's shape: 64 instances (16 sequences x 4 KV heads)
# with 131,072-cell contexts cut into 512 blocks of 256 cells, 2 query
# positions, and the top 64 blocks (16,384 cells, config 3's selection
# size), with 4 indexer heads of 128 dims (one 2 KB pooled key per block).
QSA_CONFIGS = {
    "qsa_select_64inst_128k_2q": dict(n_inst=64, n_rows=2, n_heads=4, idx_dim=128,
                                      block_cells=256, max_blocks=512, k_blocks=64,
                                      context=131072 - 100, dead_frac=0.02),
}


@dataclasses.dataclass
class QsaInputs:
    pooled: np.ndarray     # float32 [n_inst][max_blocks][n_heads][idx_dim]
    dead: np.ndarray       # uint8 [n_inst][max_blocks], 1 = dead block
    q_idx: np.ndarray      # float32 [n_inst][n_rows][n_heads][idx_dim]
    n_visible: np.ndarray  # int32 [n_inst][n_rows]: cells visible to each query row
    block_cells: int
    k_blocks: int
    workload: str
    seed: int

    @property
    def n_inst(self) -> int:
        return int(self.pooled.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.pooled.shape[1])

    @property
    def n_rows(self) -> int:
        return int(self.q_idx.shape[1])


def make_qsa(name: str | None = None, seed: int | None = None, context=None,
             **overrides) -> QsaInputs:
    """Pooled keys and indexer queries N(0, 1) (queries scaled by
    1/sqrt(n_heads * idx_dim)), a fraction dead_frac of the blocks dead at
    random; query row r of an instance sees context - n_rows + 1 + r cells
    (consecutive verify positions at the end of its context).  context may be
    a number or one per instance."""
    spec = dict(QSA_CONFIGS[name]) if name is not None else {}
    spec.update(overrides)
    n_inst, n_rows = int(spec["n_inst"]), int(spec["n_rows"])
    H, D = int(spec["n_heads"]), int(spec["idx_dim"])
    R, B = int(spec["block_cells"]), int(spec["max_blocks"])
    seed = 20261500 if seed is None else seed
    if context is None:
        context = spec.get("context", B * R)
    ctx = np.broadcast_to(np.asarray(context, np.int64), (n_inst,))
    children = np.random.SeedSequence(seed).spawn(n_inst)
    pooled = np.empty((n_inst, B, H, D), np.float32)
    q = np.empty((n_inst, n_rows, H, D), np.float32)
    dead = np.zeros((n_inst, B), np.uint8)
    frac = float(spec.get("dead_frac", 0.0))

    def fill(i):
        rng = np.random.Generator(np.random.PCG64(children[i]))
        pooled[i] = rng.standard_normal((B, H, D), dtype=np.float32)
        q[i] = rng.standard_normal((n_rows, H, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(H * D))
        if frac > 0:
            dead[i] = (rng.random(B) < frac).astype(np.uint8)

    with _cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n_inst)))
    vis = (ctx[:, None] - n_rows + 1 + np.arange(n_rows)[None, :]).clip(0, 2**31 - 1).astype(np.int32)
    return QsaInputs(pooled=pooled, dead=dead, q_idx=q, n_visible=vis, block_cells=R,
                     k_blocks=int(spec["k_blocks"]),
                     workload=str(spec.get("workload", name or "custom_qsa")), seed=int(seed))
