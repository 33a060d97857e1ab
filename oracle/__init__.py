"""CPU oracle (fp64, plain C) for selected-cell INT8 decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and
by bench.py's CPU-baseline leg, never by the product path.  The C source
(oracle.c) states the definitions it follows and the readings taken where the
Strata pages are silent.

Inputs are passed as any object carrying the arrays described in
decode_attention_sparse_amd/inputs.py (k_codes, v_codes, k_scales, v_scales,
page_table, sel, n_sel, q, softmax_scale); nothing here imports that package.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")


def build(force: bool = True, extra_flags: tuple = ()) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           *extra_flags, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = C.CDLL(_LIB)
    lib.oracle_threads.restype = C.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_half_to_double.restype = C.c_double
    lib.oracle_half_to_double.argtypes = [C.c_uint16]
    lib.oracle_gather.restype = None
    lib.oracle_gather.argtypes = [C.c_int64, _i32p, C.c_int64, _i32p, _i32p, C.c_int64,
                                  C.c_int64, C.c_int64, _i64p]
    pool = [_i8p, _u16p, _i8p, _u16p, C.c_int64, C.c_int64, _i32p, C.c_int64, C.c_int64,
            _i32p, C.c_int64, _i32p, _f32p, C.c_int64, C.c_double]
    lib.oracle_attend.restype = None
    lib.oracle_attend.argtypes = pool + [C.c_void_p, C.c_int64, _f64p, _f64p]
    lib.oracle_chunk_partials.restype = None
    lib.oracle_chunk_partials.argtypes = pool + [C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                                 _f64p, _f64p, _f64p]
    lib.oracle_float_to_half.restype = C.c_uint16
    lib.oracle_float_to_half.argtypes = [C.c_float]
    lib.oracle_kv_append.restype = None
    lib.oracle_kv_append.argtypes = [_i8p, _u16p, _i8p, _u16p, C.c_int64, C.c_int64, C.c_int64,
                                     _i32p, C.c_int64, C.c_int64, _f32p, _f32p, C.c_int64]
    lib.oracle_prompt_attend.restype = None
    lib.oracle_prompt_attend.argtypes = [_i8p, _u16p, _i8p, _u16p, C.c_int64, C.c_int64, _i32p,
                                         C.c_int64, C.c_int64, _f32p, C.c_int64, C.c_int64,
                                         C.c_double, _i64p, C.c_int64, _f64p, _f64p]
    lib.oracle_qsa_scores.restype = None
    lib.oracle_qsa_scores.argtypes = [C.c_int64] * 6 + [_f32p, _u8p, _f32p, _i32p, _f64p]
    lib.oracle_qsa_select.restype = None
    lib.oracle_qsa_select.argtypes = [C.c_int64] * 4 + [_f64p, _i32p, C.c_int64, _i32p,
                                                         C.c_int64, _i32p]
    lib.oracle_merge.restype = None
    lib.oracle_merge.argtypes = [C.c_int64, C.c_int64, C.c_int64, _f64p, _f64p, _f64p, _f64p,
                                 _f64p]
    _lib = lib
    return lib


def threads() -> int:
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def half_to_double(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, np.uint16).reshape(-1)
    return np.array([lib.oracle_half_to_double(int(x)) for x in b], np.float64)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def gather(x) -> np.ndarray:
    """Physical cell per list entry (int64, -1 = masked), [n_inst][sel_stride].
    Entries at or past n_sel[i] are -2 (not written)."""
    lib = _load()
    sel = _c(x.sel, np.int32)
    pt = _c(x.page_table, np.int32)
    n_inst, stride = sel.shape
    out = np.full((n_inst, stride), -2, np.int64)
    n_phys_pages = x.k_codes.shape[0] // 16
    lib.oracle_gather(n_inst, sel, stride, _c(x.n_sel, np.int32), pt, pt.shape[1],
                      pt.shape[1], n_phys_pages, out)
    return out


def _pool_args(x):
    q = _c(x.q, np.float32)
    n_inst = q.shape[0]
    D = q.shape[-1]
    n_rows = int(np.prod(q.shape[1:-1]))
    sel = _c(x.sel, np.int32)
    pt = _c(x.page_table, np.int32)
    kc = _c(x.k_codes, np.int8)
    args = [kc, _c(x.k_scales, np.uint16), _c(x.v_codes, np.int8), _c(x.v_scales, np.uint16),
            kc.shape[0] // 16, D, pt, pt.shape[1], pt.shape[1], sel, sel.shape[1],
            _c(x.n_sel, np.int32), q.reshape(n_inst, n_rows, D), n_rows,
            float(x.softmax_scale)]
    return args, n_inst, n_rows, D


def _ids(inst_ids, n_inst):
    if inst_ids is None:
        return None, n_inst
    ids = np.ascontiguousarray(inst_ids, np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= n_inst):
        raise ValueError("instance id out of range")
    return ids, ids.size


def attend(x, inst_ids=None):
    """Dense result: out float64 [k][n_q][n_qheads][D], lse [k][n_q][n_qheads]
    for the listed instances (all when inst_ids is None)."""
    lib = _load()
    args, n_inst, n_rows, D = _pool_args(x)
    ids, k = _ids(inst_ids, n_inst)
    out = np.zeros((k, n_rows, D), np.float64)
    lse = np.zeros((k, n_rows), np.float64)
    lib.oracle_attend(*args, None if ids is None else ids.ctypes.data, k, out, lse)
    shp = (k,) + tuple(x.q.shape[1:-1])
    return out.reshape(shp + (D,)), lse.reshape(shp)


def chunk_partials(x, chunk: int, n_chunks: int | None = None, inst_ids=None):
    """Per-chunk partials: acc [k][n_chunks][n_rows][D], m and l [k][n_chunks][n_rows]."""
    lib = _load()
    args, n_inst, n_rows, D = _pool_args(x)
    ids, k = _ids(inst_ids, n_inst)
    if n_chunks is None:
        n_chunks = max(1, -(-int(np.max(x.n_sel)) // chunk))
    acc = np.zeros((k, n_chunks, n_rows, D), np.float64)
    m = np.zeros((k, n_chunks, n_rows), np.float64)
    l = np.zeros((k, n_chunks, n_rows), np.float64)
    lib.oracle_chunk_partials(*args, chunk, n_chunks, None if ids is None else ids.ctypes.data,
                              k, acc, m, l)
    return acc, m, l


def float_to_half(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of float32 values, round to nearest even."""
    lib = _load()
    a = np.asarray(x, np.float32).reshape(-1)
    return np.array([lib.oracle_float_to_half(float(v)) for v in a], np.uint16)


def kv_append(pool, page_table, n_logical_pages, pos0, k_new, v_new, scale_stride=1):
    """The KV append of one instance on copies of the pool arrays.  pool =
    (k_codes int8 [cells][D], k_scales uint16, v_codes, v_scales), the scales
    as flat arrays indexed by cell * scale_stride; page_table int32 row;
    k_new, v_new float32 [n_new][D].  Returns the four updated copies."""
    lib = _load()
    kc, ks, vc, vs = (np.array(a, copy=True) for a in pool)
    for a, dt in ((kc, np.int8), (ks, np.uint16), (vc, np.int8), (vs, np.uint16)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("pool arrays: int8 codes and uint16 scales, C-contiguous")
    kn, vn = _c(k_new, np.float32), _c(v_new, np.float32)
    D = kc.shape[1]
    lib.oracle_kv_append(kc, ks.reshape(-1), vc, vs.reshape(-1), int(scale_stride),
                         kc.shape[0] // 16, D, _c(page_table, np.int32), int(n_logical_pages),
                         int(pos0), kn, vn, kn.shape[0])
    return kc, ks, vc, vs


def prompt_attend(x, inst: int = 0, t_ids=None):
    """Prompt attention of instance `inst`: query position t sits at position
    x.pos0[inst] + t and attends to logical cells 0..that position.  Returns
    out float64 [k][n_qheads][D] and lse [k][n_qheads] for the positions t in
    t_ids (all n_q when None)."""
    lib = _load()
    q = _c(x.q[inst], np.float32)
    n_q, n_qheads, D = q.shape
    t = np.arange(n_q, dtype=np.int64) if t_ids is None else _c(t_ids, np.int64).reshape(-1)
    if t.size and (t.min() < 0 or t.max() >= n_q):
        raise ValueError("position index out of range")
    pt = _c(x.page_table[inst], np.int32)
    kc = _c(x.k_codes, np.int8)
    out = np.zeros((t.size, n_qheads, D), np.float64)
    lse = np.zeros((t.size, n_qheads), np.float64)
    lib.oracle_prompt_attend(kc, _c(x.k_scales, np.uint16), _c(x.v_codes, np.int8),
                             _c(x.v_scales, np.uint16), kc.shape[0] // 16, D, pt, pt.shape[0],
                             int(x.pos0[inst]), q, n_q, n_qheads, float(x.softmax_scale), t,
                             t.size, out, lse)
    return out, lse


def merge(acc, m, l):
    """Merge partials laid out [k][n_chunks][n_rows][...] into out [k][n_rows][D], lse [k][n_rows]."""
    lib = _load()
    k, nc, R, D = acc.shape
    a = _c(np.transpose(acc, (0, 2, 1, 3)), np.float64)
    mm = _c(np.transpose(m, (0, 2, 1)), np.float64)
    ll = _c(np.transpose(l, (0, 2, 1)), np.float64)
    out = np.zeros((k * R, D), np.float64)
    lse = np.zeros((k * R,), np.float64)
    lib.oracle_merge(k * R, nc, D, a, mm, ll, out, lse)
    return out.reshape(k, R, D), lse.reshape(k, R)


def qsa_scores(x) -> np.ndarray:
    """Block scores float64 [n_inst][n_rows][max_blocks] of QSA inputs x
    (pooled [n_inst][max_blocks][n_heads][idx_dim], dead [n_inst][max_blocks],
    q_idx [n_inst][n_rows][n_heads][idx_dim], n_visible [n_inst][n_rows],
    block_cells)."""
    lib = _load()
    pooled = _c(x.pooled, np.float32)
    n_inst, max_blocks, n_heads, idx_dim = pooled.shape
    q = _c(x.q_idx, np.float32)
    n_rows = q.shape[1]
    out = np.empty((n_inst, n_rows, max_blocks), np.float64)
    lib.oracle_qsa_scores(n_inst, n_rows, n_heads, idx_dim, max_blocks, int(x.block_cells),
                          pooled, _c(x.dead, np.uint8), q, _c(x.n_visible, np.int32), out)
    return out


def qsa_select(scores, n_visible, block_cells: int, k_blocks: int):
    """Top-k selection from scores [n_inst][n_rows][max_blocks]: returns
    (sel int32 [n_inst][k_blocks * block_cells], n_sel int32 [n_inst]);
    entries past n_sel[i] are -1."""
    lib = _load()
    sc = _c(scores, np.float64)
    n_inst, n_rows, max_blocks = sc.shape
    stride = max(int(k_blocks) * int(block_cells), 1)
    sel = np.full((n_inst, stride), -1, np.int32)
    n_sel = np.zeros((n_inst,), np.int32)
    lib.oracle_qsa_select(n_inst, n_rows, max_blocks, int(block_cells), sc,
                          _c(n_visible, np.int32), int(k_blocks), sel, stride, n_sel)
    if np.any(n_sel > stride):
        raise ValueError("more selected cells than k_blocks * block_cells")
    return sel, n_sel
