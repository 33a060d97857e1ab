"""Thin Python binding of libsda.so (include/sda.h), argument marshalling only.

PyTorch provides device memory and the stream; every step of the attention
runs in the library's HIP kernels.  If libsda.so is missing the calls raise;
there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsda.so")

SDA_OK, SDA_ERR_INVALID_ARG, SDA_ERR_UNSUPPORTED, SDA_ERR_WORKSPACE, SDA_ERR_LAUNCH = 0, -1, -2, -3, -4
SDA_ERR_SCRATCH = -5
SCRATCH_BYTES = 32 << 20  # the device array behind sda_decode_attn_batch_noalloc, per GPU
PAGE_SIZE, HEAD_DIM, MAX_ROWS, CHUNK_ALIGN, MAX_CHUNKS = 16, 256, 64, 64, 65535
PROMPT_MAX_ROWS = 65535 * 48
QSA_MAX_ROWS, QSA_HD_ALIGN, QSA_MAX_HD, QSA_MAX_BLOCKS, QSA_MAX_K = 8, 64, 1024, 16384, 4096

EXPORTED = ("sda_workspace_bytes", "sda_decode_attn_step", "sda_decode_attn_batch",
            "sda_decode_attn_batch_noalloc",
            "sda_chunk_batch", "sda_merge_batch", "sda_prompt_attn_batch", "sda_fused_chunk_cells",
            "sda_fused_single_launch", "sda_kv_append_batch", "sda_qsa_block_scores",
            "sda_qsa_select", "sda_status_string")


class SdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {library().sda_status_string(status).decode()}")


class _Pool(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("k_scales", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_scales", C.c_void_p), ("n_phys_pages", C.c_int64), ("page_size", C.c_int32),
                ("head_dim", C.c_int32), ("scale_stride", C.c_int32), ("reserved", C.c_int32)]


_lib = None


def library() -> C.CDLL:
    """Load libsda.so (built by decode_attention_sparse_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m decode_attention_sparse_amd.build`")
        lib = C.CDLL(LIB_PATH)
        i32, i64, vp, f32, sz = C.c_int32, C.c_int64, C.c_void_p, C.c_float, C.c_size_t
        lib.sda_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, C.POINTER(sz)]
        lib.sda_workspace_bytes.restype = C.c_int
        lib.sda_decode_attn_step.argtypes = [C.POINTER(_Pool), vp, i32, vp, i32, vp, i32, i32, f32,
                                             i32, vp, vp, vp, vp, sz, vp]
        lib.sda_decode_attn_step.restype = C.c_int
        lib.sda_decode_attn_batch.argtypes = [C.POINTER(_Pool), i32, vp, i64, i32, vp, i64, vp, i32,
                                              vp, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp]
        lib.sda_decode_attn_batch.restype = C.c_int
        lib.sda_decode_attn_batch_noalloc.argtypes = [C.POINTER(_Pool), i32, vp, i64, i32, vp, i64,
                                                      vp, i32, vp, i32, i32, f32, i32, vp, vp, vp,
                                                      vp]
        lib.sda_decode_attn_batch_noalloc.restype = C.c_int
        lib.sda_chunk_batch.argtypes = [C.POINTER(_Pool), i32, vp, i64, i32, vp, i64, vp, i32, vp,
                                        i32, i32, f32, i32, vp, vp, sz, vp]
        lib.sda_chunk_batch.restype = C.c_int
        lib.sda_merge_batch.argtypes = [i32, i32, i32, vp, i32, i32, vp, sz, vp, vp, vp]
        lib.sda_merge_batch.restype = C.c_int
        lib.sda_prompt_attn_batch.argtypes = [C.POINTER(_Pool), i32, vp, i64, i32, vp, vp, i32, i32,
                                              f32, vp, vp, vp]
        lib.sda_prompt_attn_batch.restype = C.c_int
        # sda_pool_mut has sda_pool's layout (writable pointers)
        lib.sda_kv_append_batch.argtypes = [C.POINTER(_Pool), i32, vp, i64, i32, vp, vp, vp, i32, vp]
        lib.sda_kv_append_batch.restype = C.c_int
        lib.sda_fused_chunk_cells.argtypes = [i32, i32, i32, C.POINTER(i32)]
        lib.sda_fused_chunk_cells.restype = C.c_int
        lib.sda_fused_single_launch.argtypes = [i32, i32, i32, i32, i32, C.POINTER(i32)]
        lib.sda_fused_single_launch.restype = C.c_int
        lib.sda_qsa_block_scores.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        lib.sda_qsa_block_scores.restype = C.c_int
        lib.sda_qsa_select.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, i64, vp, vp]
        lib.sda_qsa_select.restype = C.c_int
        lib.sda_status_string.argtypes = [C.c_int]
        lib.sda_status_string.restype = C.c_char_p
        _lib = lib
    return _lib


@dataclasses.dataclass
class Pool:
    """Device tensors of the INT8 pools: codes int8 [cells][256]; scales as
    binary16 bit patterns (int16/uint16/float16 tensors), either two arrays
    [cells] or one array [cells][2] of interleaved (K, V) pairs (pass it as
    `scales`, leaving k_scales / v_scales None)."""
    k_codes: torch.Tensor
    k_scales: torch.Tensor | None
    v_codes: torch.Tensor
    v_scales: torch.Tensor | None
    scales: torch.Tensor | None = None

    @property
    def n_phys_pages(self) -> int:
        return self.k_codes.shape[0] // PAGE_SIZE

    def c_struct(self) -> _Pool:
        hd = int(self.k_codes.shape[1]) if self.k_codes.dim() == 2 else 0
        if self.scales is not None:
            if self.scales.dim() != 2 or self.scales.shape[1] != 2:
                raise ValueError("interleaved scales must have shape [cells][2]")
            base = _ptr(self.scales)
            es = self.scales.element_size()
            return _Pool(_ptr(self.k_codes), base, _ptr(self.v_codes), base + es,
                         self.n_phys_pages, PAGE_SIZE, hd, 2, 0)
        return _Pool(_ptr(self.k_codes), _ptr(self.k_scales), _ptr(self.v_codes),
                     _ptr(self.v_scales), self.n_phys_pages, PAGE_SIZE, hd, 1, 0)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsda must be contiguous")
    return t.data_ptr() or None


_HALF = (torch.int16, torch.uint16, torch.float16)


def _check(t, name, dtypes, shape=None, optional=False):
    """Raise ValueError unless t is a contiguous tensor of one of dtypes with
    the given shape (None entries: any size).  The library trusts sizes it
    cannot see, so a tensor smaller than the arguments say would be read or
    written out of bounds on the device.  (Devices: _on.)"""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, "
                         f"not {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(a) != int(s)
                                         for a, s in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                             f"{tuple('*' if s is None else s for s in shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on(**tensors):
    """Raise ValueError unless every given tensor (None: absent) is on one GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, not {t.device}")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
        dev = t.device


def _check_pool(pool):
    """The pool's shapes and dtypes; returns its tensors by name (for _on)."""
    _check(pool.k_codes, "pool.k_codes", torch.int8, (None, HEAD_DIM))
    cells = int(pool.k_codes.shape[0])
    if cells % PAGE_SIZE:
        raise ValueError(f"pool cells ({cells}) must be a multiple of {PAGE_SIZE}")
    _check(pool.v_codes, "pool.v_codes", torch.int8, (cells, HEAD_DIM))
    if pool.scales is not None:
        if pool.k_scales is not None or pool.v_scales is not None:
            raise ValueError("give either interleaved scales or k_scales and v_scales")
        _check(pool.scales, "pool.scales", _HALF, (cells, 2))
    else:
        _check(pool.k_scales, "pool.k_scales", _HALF, (cells,))
        _check(pool.v_scales, "pool.v_scales", _HALF, (cells,))
    return {"pool.k_codes": pool.k_codes, "pool.v_codes": pool.v_codes,
            "pool.k_scales": pool.k_scales, "pool.v_scales": pool.v_scales,
            "pool.scales": pool.scales}


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def workspace_bytes(n_inst: int, n_q: int, n_qheads: int, max_sel: int, chunk_cells: int,
                    head_dim: int = HEAD_DIM) -> int:
    out = C.c_size_t(0)
    st = library().sda_workspace_bytes(n_inst, n_q, n_qheads, head_dim, max_sel, chunk_cells,
                                       C.byref(out))
    if st != SDA_OK:
        raise SdaError(st, "sda_workspace_bytes")
    return int(out.value)


def fused_chunk_cells(n_inst: int, max_sel: int, chunk_cells: int) -> int:
    """Chunk size sda_decode_attn_step/_batch use for this geometry."""
    out = C.c_int32(0)
    st = library().sda_fused_chunk_cells(n_inst, max_sel, chunk_cells, C.byref(out))
    if st != SDA_OK:
        raise SdaError(st, "sda_fused_chunk_cells")
    return int(out.value)


def fused_single_launch(n_inst: int, n_q: int, n_qheads: int, max_sel: int,
                        chunk_cells: int) -> bool:
    """Whether sda_decode_attn_step/_batch run this geometry as one chunk-kernel
    launch that writes the outputs (the workspace is then left untouched)."""
    out = C.c_int32(0)
    st = library().sda_fused_single_launch(n_inst, n_q, n_qheads, max_sel, chunk_cells,
                                           C.byref(out))
    if st != SDA_OK:
        raise SdaError(st, "sda_fused_single_launch")
    return bool(out.value)


def workspace(n_inst, n_q, n_qheads, max_sel, chunk_cells, device="cuda") -> torch.Tensor:
    """A device buffer of the required size (torch allocates it)."""
    nb = workspace_bytes(n_inst, n_q, n_qheads, max_sel, chunk_cells)
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def partials(ws: torch.Tensor, n_inst, n_q, n_qheads, max_sel, chunk_cells):
    """Views (acc, m, l) of the chunk partials inside a workspace, as the
    header lays them out."""
    R = n_q * n_qheads
    nch = -(-max_sel // chunk_cells)
    units = n_inst * nch * R
    al = lambda x: (x + 255) // 256 * 256
    f = ws.view(torch.float32) if ws.dtype != torch.float32 else ws
    m_off = al(units * HEAD_DIM * 4) // 4
    l_off = m_off + al(units * 4) // 4
    acc = f[: units * HEAD_DIM].view(n_inst, nch, R, HEAD_DIM)
    m = f[m_off: m_off + units].view(n_inst, nch, R)
    l = f[l_off: l_off + units].view(n_inst, nch, R)
    return acc, m, l


def decode_attn_step(pool: Pool, page_table, sel, q, softmax_scale: float, chunk_cells: int,
                     out, lse, gather_out=None, ws=None, stream=None, n_sel: int | None = None):
    """One sequence: q [n_q][n_qheads][256] fp32; out like q; lse [n_q][n_qheads].
    Chunks of fused_chunk_cells(1, n_sel, chunk_cells) cells, as the batch call."""
    _check(q, "q", torch.float32, (None, None, HEAD_DIM))
    n_q, n_qheads = int(q.shape[0]), int(q.shape[1])
    _check(sel, "sel", torch.int32, (None,))
    n = int(sel.numel()) if n_sel is None else int(n_sel)
    if not 0 <= n <= sel.numel():
        raise ValueError(f"n_sel {n} outside [0, {sel.numel()}]")
    _check(page_table, "page_table", torch.int32, (None,))
    _check(out, "out", torch.float32, tuple(q.shape))
    _check(lse, "lse", torch.float32, (n_q, n_qheads))
    _check(gather_out, "gather_out", torch.int32, (sel.numel(),), optional=True)
    _check(ws, "ws", torch.uint8, (None,), optional=True)
    _on(q=q, sel=sel, page_table=page_table, out=out, lse=lse, gather_out=gather_out, ws=ws,
        **_check_pool(pool))
    if ws is None:
        ws = workspace(1, n_q, n_qheads, n, chunk_cells, q.device)
    ps = pool.c_struct()
    st = library().sda_decode_attn_step(
        C.byref(ps), _ptr(page_table), int(page_table.numel()), _ptr(sel), n, _ptr(q), n_q,
        n_qheads, float(softmax_scale), int(chunk_cells), _ptr(out), _ptr(lse), _ptr(gather_out),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_decode_attn_step")
    return ws


def decode_attn_batch(pool: Pool, page_table, sel, n_sel, max_sel: int, q, softmax_scale: float,
                      chunk_cells: int, out, lse, gather_out=None, ws=None, stream=None,
                      n_logical_pages: int | None = None):
    """Many instances: page_table [n_inst][pt_stride], sel [n_inst][sel_stride],
    n_sel device int32 [n_inst], q [n_inst][n_q][n_qheads][256].  The call
    runs chunks of fused_chunk_cells(n_inst, max_sel, chunk_cells) cells; the
    workspace then holds those partials (partials(..., that chunk size)),
    unless fused_single_launch(...) says the call is one launch that leaves
    the workspace untouched."""
    n_inst, n_q, n_qheads = _check_decode(pool, page_table, sel, n_sel, max_sel, q, gather_out,
                                          ws, out=out, lse=lse)
    if ws is None:
        ws = workspace(n_inst, n_q, n_qheads, max_sel, chunk_cells, q.device)
    nlp = _n_logical(page_table, n_logical_pages)
    ps = pool.c_struct()
    st = library().sda_decode_attn_batch(
        C.byref(ps), n_inst, _ptr(page_table), int(page_table.shape[1]), nlp, _ptr(sel),
        int(sel.shape[1]), _ptr(n_sel), int(max_sel), _ptr(q), n_q, n_qheads,
        float(softmax_scale), int(chunk_cells), _ptr(out), _ptr(lse), _ptr(gather_out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_decode_attn_batch")
    return ws


def decode_attn_batch_noalloc(pool: Pool, page_table, sel, n_sel, max_sel: int, q,
                              softmax_scale: float, chunk_cells: int, out, lse, gather_out=None,
                              stream=None, n_logical_pages: int | None = None):
    """decode_attn_batch without a workspace: the chunk partials go to the
    library's own device array (SCRATCH_BYTES per GPU); the call allocates
    nothing.  Calls that overlap on one GPU share that array and race."""
    n_inst, n_q, n_qheads = _check_decode(pool, page_table, sel, n_sel, max_sel, q, gather_out,
                                          None, out=out, lse=lse)
    nlp = _n_logical(page_table, n_logical_pages)
    ps = pool.c_struct()
    st = library().sda_decode_attn_batch_noalloc(
        C.byref(ps), n_inst, _ptr(page_table), int(page_table.shape[1]), nlp, _ptr(sel),
        int(sel.shape[1]), _ptr(n_sel), int(max_sel), _ptr(q), n_q, n_qheads,
        float(softmax_scale), int(chunk_cells), _ptr(out), _ptr(lse), _ptr(gather_out),
        _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_decode_attn_batch_noalloc")


def _n_logical(page_table, n_logical_pages):
    """Logical pages per instance: the table's row length, or fewer."""
    nlp = int(page_table.shape[1]) if n_logical_pages is None else int(n_logical_pages)
    if not 0 <= nlp <= int(page_table.shape[1]):
        raise ValueError(f"n_logical_pages {nlp} outside [0, {int(page_table.shape[1])}]")
    return nlp


def _check_decode(pool, page_table, sel, n_sel, max_sel, q, gather_out, ws, out=None, lse=None):
    """Shapes, dtypes and devices of a batched decode call's tensors (out and
    lse when given); returns (n_inst, n_q, n_qheads)."""
    _check(q, "q", torch.float32, (None, None, None, HEAD_DIM))
    n_inst, n_q, n_qheads = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    _check(page_table, "page_table", torch.int32, (n_inst, None))
    _check(sel, "sel", torch.int32, (n_inst, None))
    if not 0 <= int(max_sel) <= int(sel.shape[1]):
        raise ValueError(f"max_sel {max_sel} outside [0, {int(sel.shape[1])}] (sel's row length)")
    _check(n_sel, "n_sel", torch.int32, (n_inst,))
    _check(gather_out, "gather_out", torch.int32, tuple(sel.shape), optional=True)
    _check(ws, "ws", torch.uint8, (None,), optional=True)
    if out is not None or lse is not None:
        _check(out, "out", torch.float32, tuple(q.shape))
        _check(lse, "lse", torch.float32, (n_inst, n_q, n_qheads))
    _on(q=q, page_table=page_table, sel=sel, n_sel=n_sel, gather_out=gather_out, ws=ws, out=out,
        lse=lse, **_check_pool(pool))
    return n_inst, n_q, n_qheads


def chunk_batch(pool: Pool, page_table, sel, n_sel, max_sel: int, q, softmax_scale: float,
                chunk_cells: int, ws, gather_out=None, stream=None):
    """Chunk pass only, at exactly chunk_cells: partials into ws (see partials())."""
    if ws is None:
        raise ValueError("ws is required")
    _check_decode(pool, page_table, sel, n_sel, max_sel, q, gather_out, ws)
    n_inst, n_q, n_qheads = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    ps = pool.c_struct()
    st = library().sda_chunk_batch(
        C.byref(ps), n_inst, _ptr(page_table), int(page_table.shape[1]), int(page_table.shape[1]),
        _ptr(sel), int(sel.shape[1]), _ptr(n_sel), int(max_sel), _ptr(q), n_q, n_qheads,
        float(softmax_scale), int(chunk_cells), _ptr(gather_out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_chunk_batch")


def merge_batch(n_sel, max_sel: int, chunk_cells: int, ws, out, lse, stream=None):
    """Merge pass only: partials in ws -> out [n_inst][n_q][n_qheads][256], lse."""
    _check(out, "out", torch.float32, (None, None, None, HEAD_DIM))
    n_inst, n_q, n_qheads = int(out.shape[0]), int(out.shape[1]), int(out.shape[2])
    _check(lse, "lse", torch.float32, (n_inst, n_q, n_qheads))
    _check(n_sel, "n_sel", torch.int32, (n_inst,))
    _check(ws, "ws", torch.uint8, (None,))
    _on(out=out, lse=lse, n_sel=n_sel, ws=ws)
    st = library().sda_merge_batch(n_inst, n_q, n_qheads, _ptr(n_sel), int(max_sel),
                                   int(chunk_cells), _ptr(ws), ws.numel() * ws.element_size(),
                                   _ptr(out), _ptr(lse), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_merge_batch")


def prompt_attn_batch(pool: Pool, page_table, pos0, q, softmax_scale: float, out, lse,
                      stream=None, n_logical_pages: int | None = None):
    """Prompt attention: page_table [n_inst][pt_stride], pos0 device int32
    [n_inst] (position of query 0), q [n_inst][n_q][n_qheads][256] fp32; query
    t of instance i attends causally to logical cells 0..pos0[i] + t.  out like
    q, lse [n_inst][n_q][n_qheads]."""
    _check(q, "q", torch.float32, (None, None, None, HEAD_DIM))
    n_inst, n_q, n_qheads = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    _check(page_table, "page_table", torch.int32, (n_inst, None))
    _check(pos0, "pos0", torch.int32, (n_inst,))
    _check(out, "out", torch.float32, tuple(q.shape))
    _check(lse, "lse", torch.float32, (n_inst, n_q, n_qheads))
    _on(q=q, page_table=page_table, pos0=pos0, out=out, lse=lse, **_check_pool(pool))
    nlp = _n_logical(page_table, n_logical_pages)
    ps = pool.c_struct()
    st = library().sda_prompt_attn_batch(
        C.byref(ps), n_inst, _ptr(page_table), int(page_table.shape[1]), nlp, _ptr(pos0), _ptr(q),
        n_q, n_qheads, float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_prompt_attn_batch")


def kv_append_batch(pool: Pool, page_table, pos0, k_new, v_new, stream=None,
                    n_logical_pages: int | None = None):
    """Quantise new rows k_new, v_new float32 [n_inst][n_new][256] into the
    pools at logical cells pos0[i] + t (pos0 device int32 [n_inst]) through
    page_table [n_inst][pt_stride]; writes the pool tensors in place."""
    _check(k_new, "k_new", torch.float32, (None, None, HEAD_DIM))
    n_inst, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    _check(v_new, "v_new", torch.float32, tuple(k_new.shape))
    _check(page_table, "page_table", torch.int32, (n_inst, None))
    _check(pos0, "pos0", torch.int32, (n_inst,))
    _on(k_new=k_new, v_new=v_new, page_table=page_table, pos0=pos0, **_check_pool(pool))
    nlp = _n_logical(page_table, n_logical_pages)
    ps = pool.c_struct()
    st = library().sda_kv_append_batch(C.byref(ps), n_inst, _ptr(page_table),
                                       int(page_table.shape[1]), nlp, _ptr(pos0), _ptr(k_new),
                                       _ptr(v_new), n_new, _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_kv_append_batch")


def qsa_block_scores(pooled, dead, q_idx, n_visible, block_cells: int, scores, stream=None):
    """Block scores: pooled float32 [n_inst][max_blocks][n_heads][idx_dim],
    dead uint8 [n_inst][max_blocks], q_idx float32 [n_inst][n_rows][n_heads]
    [idx_dim], n_visible int32 [n_inst][n_rows] (cells each row sees);
    scores float32 [n_inst][n_rows][max_blocks] is written."""
    _check(pooled, "pooled", torch.float32, (None, None, None, None))
    n_inst, max_blocks, n_heads, idx_dim = (int(v) for v in pooled.shape)
    _check(q_idx, "q_idx", torch.float32, (n_inst, None, n_heads, idx_dim))
    n_rows = int(q_idx.shape[1])
    _check(dead, "dead", torch.uint8, (n_inst, max_blocks))
    _check(n_visible, "n_visible", torch.int32, (n_inst, n_rows))
    _check(scores, "scores", torch.float32, (n_inst, n_rows, max_blocks))
    _on(pooled=pooled, dead=dead, q_idx=q_idx, n_visible=n_visible, scores=scores)
    st = library().sda_qsa_block_scores(n_inst, n_rows, n_heads, idx_dim, int(block_cells),
                                        max_blocks, _ptr(pooled), _ptr(dead), _ptr(q_idx),
                                        _ptr(n_visible), _ptr(scores), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_qsa_block_scores")


def qsa_select(scores, n_visible, block_cells: int, k_blocks: int, sel, n_sel, stream=None):
    """Top-k blocks of scores [n_inst][n_rows][max_blocks] expanded to sorted
    cells: sel int32 [n_inst][>= k_blocks * block_cells] and n_sel int32
    [n_inst] are written (the sel / n_sel arguments of decode_attn_batch)."""
    _check(scores, "scores", torch.float32, (None, None, None))
    n_inst, n_rows, max_blocks = (int(v) for v in scores.shape)
    _check(n_visible, "n_visible", torch.int32, (n_inst, n_rows))
    _check(sel, "sel", torch.int32, (n_inst, None))
    if int(sel.shape[1]) < int(k_blocks) * int(block_cells):
        raise ValueError("sel rows are shorter than k_blocks * block_cells")
    _check(n_sel, "n_sel", torch.int32, (n_inst,))
    _on(scores=scores, n_visible=n_visible, sel=sel, n_sel=n_sel)
    st = library().sda_qsa_select(n_inst, n_rows, int(block_cells), max_blocks, _ptr(scores),
                                  _ptr(n_visible), int(k_blocks), _ptr(sel), int(sel.shape[1]),
                                  _ptr(n_sel), _stream(stream))
    if st != SDA_OK:
        raise SdaError(st, "sda_qsa_select")


def to_device(x, device="cuda", interleave_scales=False):
    """Upload generated inputs (decode_attention_sparse_amd.inputs.Inputs):
    returns (Pool, dict of device tensors).  With interleave_scales the K and
    V scales are stored as one [cells][2] array of (K, V) pairs."""
    import numpy as np
    t = lambda a: torch.from_numpy(a).to(device)
    if interleave_scales:
        pairs = np.stack([x.k_scales.view("int16"), x.v_scales.view("int16")], axis=1)
        pool = Pool(t(x.k_codes), None, t(x.v_codes), None, scales=t(np.ascontiguousarray(pairs)))
    else:
        pool = Pool(t(x.k_codes), t(x.k_scales.view("int16")), t(x.v_codes),
                    t(x.v_scales.view("int16")))
    dev = dict(page_table=t(x.page_table), sel=t(x.sel), n_sel=t(x.n_sel), q=t(x.q))
    if getattr(x, "pos0", None) is not None:  # prompt inputs
        dev["pos0"] = t(x.pos0)
    return pool, dev
