"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/sda.h declares, sizes the workspace as documented, and
rejects bad arguments with the documented status before launching anything."""
import ctypes as C
import os
import re
import subprocess

import pytest

from decode_attention_sparse_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sda_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert set(api.EXPORTED) <= set(declared_functions())


def test_library_exports_every_declared_symbol():
    lib = api.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = set(re.findall(r"\bT (sda_\w+)", out))
    assert set(declared_functions()) <= syms


def test_header_compiles_as_c():
    src = '#include "sda.h"\nint main(void){ sda_pool p; (void)p; return SDA_OK; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-x", "c", "-", "-fsyntax-only"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define SDA_(\w+) (\d+)", text))
    assert {k: int(v) for k, v in defs.items()} == {
        "PAGE_SIZE": api.PAGE_SIZE, "HEAD_DIM": api.HEAD_DIM, "MAX_ROWS": api.MAX_ROWS,
        "CHUNK_ALIGN": api.CHUNK_ALIGN, "MAX_CHUNKS": api.MAX_CHUNKS,
        "PROMPT_MAX_ROWS": api.PROMPT_MAX_ROWS, "QSA_MAX_ROWS": api.QSA_MAX_ROWS,
        "QSA_HD_ALIGN": api.QSA_HD_ALIGN, "QSA_MAX_HD": api.QSA_MAX_HD,
        "QSA_MAX_BLOCKS": api.QSA_MAX_BLOCKS, "QSA_MAX_K": api.QSA_MAX_K}


def test_scratch_size_matches_binding():
    text = open(HEADER).read()
    m = re.search(r"#define SDA_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == api.SCRATCH_BYTES


def test_status_strings():
    lib = api.library()
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert lib.sda_status_string(st)
    assert b"SCRATCH" in lib.sda_status_string(api.SDA_ERR_SCRATCH)


def _al(x):
    return (x + 255) // 256 * 256


def fused_chunk(n_inst, max_sel, chunk):
    """The documented choice, restated: a grid of at most 256 (instance,
    chunk) pairs takes the smallest multiple of 64 keeping it within 256; one
    of more than 512 pairs takes k = min(pairs // 512, chunks per instance)
    times the chunk."""
    if n_inst <= 0 or max_sel <= 0:
        return chunk
    pairs = lambda c: n_inst * -(-max_sel // c)
    if pairs(chunk) <= 256:
        return next(c for c in range(64, chunk + 1, 64) if pairs(c) <= 256)
    if n_inst <= 256:
        m = min(512 // n_inst, -(-max_sel // chunk))
        return -(-(-(-max_sel // m)) // 64) * 64
    if pairs(chunk) > 512:
        return chunk * min(pairs(chunk) // 512, -(-max_sel // chunk))
    return chunk


@pytest.mark.parametrize("n_inst,max_sel,chunk,expect", [
    (1, 2051, 256, 64), (1, 600, 256, 64), (8, 2051, 256, 128), (8, 1500, 256, 64),
    (256, 2051, 1024, 1088), (64, 16384, 512, 2048), (32, 131072, 1024, 8192),
    (256, 2051, 256, 1088), (1, 16384, 512, 64), (1, 16385, 512, 128), (200, 512, 64, 256),
    (300, 2051, 1024, 1024), (1000, 2051, 256, 2304), (400, 600, 256, 512),
    (3, 1, 64, 64), (1, 0, 256, 256), (0, 100, 256, 256), (29, 2051, 256, 256),
    (28, 2051, 256, 256), (7, 2051, 1024, 64), (20, 2051, 1024, 192), (100, 2051, 512, 448)])
def test_fused_chunk_cells(n_inst, max_sel, chunk, expect):
    assert api.fused_chunk_cells(n_inst, max_sel, chunk) == expect == fused_chunk(n_inst, max_sel, chunk)


def test_fused_chunk_cells_sweep():
    for n_inst in (1, 2, 3, 5, 8, 13, 32, 100, 257):
        for max_sel in (1, 63, 64, 65, 600, 2051, 4096, 16384, 65536):
            for chunk in (64, 128, 192, 256, 512, 1024):
                assert api.fused_chunk_cells(n_inst, max_sel, chunk) == fused_chunk(n_inst, max_sel, chunk)
    # near the int32 limit the choice stays a valid positive multiple of 64
    for n_inst, max_sel in ((2, 2**31 - 1), (200, 2**31 - 1), (1, 2**31 - 1)):
        c = api.fused_chunk_cells(n_inst, max_sel, 64 * 2**20)
        assert 0 < c and c % 64 == 0
    out = C.c_int32(0)
    assert api.library().sda_fused_chunk_cells(1, 10, 100, C.byref(out)) == api.SDA_ERR_UNSUPPORTED
    assert api.library().sda_fused_chunk_cells(-1, 10, 64, C.byref(out)) == api.SDA_ERR_INVALID_ARG
    assert api.library().sda_fused_chunk_cells(1, 10, 64, None) == api.SDA_ERR_INVALID_ARG


def single_launch(n_inst, n_q, nh, max_sel, chunk):
    """The documented rule, restated: chunks of more than 64 cells, one per
    instance, or two with 17 to 48 query rows."""
    c = fused_chunk(n_inst, max_sel, chunk)
    nch = -(-max_sel // c)
    return c > 64 and (nch == 1 or (nch == 2 and 16 < n_q * nh <= 48))


@pytest.mark.parametrize("n_inst,n_q,nh,max_sel,chunk,expect", [
    (256, 4, 12, 2051, 1024, True),     # two 1,088-cell chunks, 48 rows
    (256, 1, 12, 2051, 1024, False),    # two chunks of 12 rows: chunk + merge
    (256, 4, 16, 2051, 1024, False),    # 64 rows
    (64, 2, 12, 16384, 512, False),     # eight chunks
    (1, 4, 12, 2051, 256, False),       # one-tile chunks
    (200, 2, 12, 250, 256, True),       # one 256-cell chunk
    (520, 4, 16, 600, 256, True),       # one 768-cell chunk, 64 rows
    (100, 1, 12, 500, 256, False),
    (3, 1, 12, 1, 64, False),           # one cell: one-tile chunk
    (5, 1, 12, 0, 256, False),          # nothing selected: the merge writes the empty rows
])
def test_fused_single_launch(n_inst, n_q, nh, max_sel, chunk, expect):
    got = api.fused_single_launch(n_inst, n_q, nh, max_sel, chunk)
    assert got == expect == single_launch(n_inst, n_q, nh, max_sel, chunk)


def test_fused_single_launch_sweep_and_status():
    for n_inst in (1, 7, 100, 200, 256, 300, 1000):
        for max_sel in (1, 64, 65, 500, 2051, 16384):
            for n_q, nh in ((1, 12), (2, 12), (3, 12), (4, 12), (1, 16), (4, 16)):
                for chunk in (64, 256, 1024):
                    assert (api.fused_single_launch(n_inst, n_q, nh, max_sel, chunk)
                            == single_launch(n_inst, n_q, nh, max_sel, chunk))
    out = C.c_int32(0)
    lib = api.library()
    assert lib.sda_fused_single_launch(1, 1, 12, 10, 100, C.byref(out)) == api.SDA_ERR_UNSUPPORTED
    assert lib.sda_fused_single_launch(1, 0, 12, 10, 64, C.byref(out)) == api.SDA_ERR_INVALID_ARG
    assert lib.sda_fused_single_launch(1, 5, 13, 10, 64, C.byref(out)) == api.SDA_ERR_UNSUPPORTED
    assert lib.sda_fused_single_launch(-1, 1, 12, 10, 64, C.byref(out)) == api.SDA_ERR_INVALID_ARG
    assert lib.sda_fused_single_launch(1, 1, 12, 10, 64, None) == api.SDA_ERR_INVALID_ARG


@pytest.mark.parametrize("n_inst,n_q,nh,max_sel,chunk", [
    (1, 1, 12, 600, 256), (1, 4, 12, 2051, 256), (256, 4, 12, 2051, 1024),
    (64, 2, 12, 16384, 512), (32, 4, 12, 131072, 1024), (3, 2, 5, 1, 64), (8, 4, 12, 2051, 256)])
def test_workspace_layout(n_inst, n_q, nh, max_sel, chunk):
    """The partials layout for the caller's chunk or the fused call's, whichever is larger."""
    R = n_q * nh
    def size(c):
        units = n_inst * -(-max_sel // c) * R
        return _al(units * 256 * 4) + 2 * _al(units * 4)
    expect = max(size(chunk), size(fused_chunk(n_inst, max_sel, chunk)))
    assert api.workspace_bytes(n_inst, n_q, nh, max_sel, chunk) == expect


def test_workspace_monotone_and_zero():
    assert api.workspace_bytes(1, 1, 12, 0, 256) == 0
    prev = 0
    for n in range(0, 3000, 97):
        cur = api.workspace_bytes(2, 3, 12, n, 256)
        assert cur >= prev
        prev = cur


@pytest.mark.parametrize("args,status", [
    ((1, 1, 12, 256, 100, 256), 0),
    ((1, 1, 12, 128, 100, 256), api.SDA_ERR_UNSUPPORTED),      # head_dim
    ((1, 5, 13, 256, 100, 256), api.SDA_ERR_UNSUPPORTED),      # rows > 64
    ((1, 1, 12, 256, 100, 100), api.SDA_ERR_UNSUPPORTED),      # chunk not multiple of 64
    ((1, 0, 12, 256, 100, 256), api.SDA_ERR_INVALID_ARG),      # n_q
    ((-1, 1, 12, 256, 100, 256), api.SDA_ERR_INVALID_ARG),
    ((1, 1, 12, 256, -5, 256), api.SDA_ERR_INVALID_ARG),
    ((1, 1, 12, 256, 100, 0), api.SDA_ERR_INVALID_ARG),
])
def test_workspace_status(args, status):
    out = C.c_size_t(0)
    assert api.library().sda_workspace_bytes(*args, C.byref(out)) == status


FAKE = 1 << 20  # an aligned, never-dereferenced address: every case below fails validation first


def _pool(**kw):
    d = dict(k_codes=FAKE, k_scales=FAKE, v_codes=FAKE, v_scales=FAKE, n_phys_pages=16,
             page_size=16, head_dim=256, scale_stride=1, reserved=0)
    d.update(kw)
    return api._Pool(**d)


def _step(pool, **kw):
    a = dict(page_table=FAKE, nlp=4, sel=FAKE, n_sel=10, q=FAKE, n_q=1, nh=12, scale=0.0625,
             chunk=256, out=FAKE, lse=FAKE, gather=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return api.library().sda_decode_attn_step(
        C.byref(pool) if pool is not None else None, a["page_table"], a["nlp"], a["sel"],
        a["n_sel"], a["q"], a["n_q"], a["nh"], a["scale"], a["chunk"], a["out"], a["lse"],
        a["gather"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("pool_kw,kw,status", [
    ({}, dict(n_sel=-1), api.SDA_ERR_INVALID_ARG),
    (dict(page_size=8), {}, api.SDA_ERR_UNSUPPORTED),
    (dict(head_dim=128), {}, api.SDA_ERR_UNSUPPORTED),
    (dict(k_codes=None), {}, api.SDA_ERR_INVALID_ARG),
    (dict(v_scales=None), {}, api.SDA_ERR_INVALID_ARG),
    (dict(k_codes=FAKE + 8), {}, api.SDA_ERR_INVALID_ARG),          # misaligned codes
    (dict(n_phys_pages=0), {}, api.SDA_ERR_INVALID_ARG),
    (dict(n_phys_pages=(1 << 27) + 1), {}, api.SDA_ERR_INVALID_ARG),
    (dict(scale_stride=0), {}, api.SDA_ERR_INVALID_ARG),
    (dict(scale_stride=65), {}, api.SDA_ERR_INVALID_ARG),
    (dict(reserved=1), {}, api.SDA_ERR_INVALID_ARG),
    ({}, dict(n_q=5, nh=13), api.SDA_ERR_UNSUPPORTED),
    ({}, dict(chunk=96), api.SDA_ERR_UNSUPPORTED),
    ({}, dict(q=None), api.SDA_ERR_INVALID_ARG),
    ({}, dict(q=FAKE + 4), api.SDA_ERR_INVALID_ARG),
    ({}, dict(out=None), api.SDA_ERR_INVALID_ARG),
    ({}, dict(out=FAKE + 4), api.SDA_ERR_INVALID_ARG),             # out rows are 16-byte stores
    ({}, dict(n_sel=65535 * 256 + 1), api.SDA_ERR_UNSUPPORTED),    # more than 65,535 chunks
    ({}, dict(lse=None), api.SDA_ERR_INVALID_ARG),
    ({}, dict(sel=None), api.SDA_ERR_INVALID_ARG),
    ({}, dict(page_table=None), api.SDA_ERR_INVALID_ARG),
    ({}, dict(scale=float("nan")), api.SDA_ERR_INVALID_ARG),
    ({}, dict(ws=None), api.SDA_ERR_WORKSPACE),
    ({}, dict(wsb=1024), api.SDA_ERR_WORKSPACE),
    ({}, dict(ws=FAKE + 64), api.SDA_ERR_WORKSPACE),
])
def test_step_rejects_before_launch(pool_kw, kw, status):
    assert _step(_pool(**pool_kw), **kw) == status


def test_null_pool():
    assert _step(None) == api.SDA_ERR_INVALID_ARG


def test_batch_rejects_before_launch():
    lib = api.library()
    p = _pool()
    def call(**kw):
        a = dict(n_inst=2, pt=FAKE, pts=4, nlp=4, sel=FAKE, sels=10, nsel=FAKE, max_sel=10,
                 q=FAKE, n_q=1, nh=12, scale=0.0625, chunk=256, out=FAKE, lse=FAKE, g=None,
                 ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.sda_decode_attn_batch(C.byref(p), a["n_inst"], a["pt"], a["pts"], a["nlp"],
                                         a["sel"], a["sels"], a["nsel"], a["max_sel"], a["q"],
                                         a["n_q"], a["nh"], a["scale"], a["chunk"], a["out"],
                                         a["lse"], a["g"], a["ws"], a["wsb"], None)
    assert call(nsel=None) == api.SDA_ERR_INVALID_ARG
    assert call(pts=3) == api.SDA_ERR_INVALID_ARG        # pt_stride < n_logical_pages
    assert call(sels=9) == api.SDA_ERR_INVALID_ARG       # sel_stride < max_sel
    assert call(max_sel=-1) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=-1) == api.SDA_ERR_INVALID_ARG
    assert call(wsb=100) == api.SDA_ERR_WORKSPACE
    assert call(n_inst=0) == api.SDA_OK                  # nothing to do, nothing launched


def test_prompt_rejects_before_launch():
    lib = api.library()
    p = _pool()
    def call(pool=p, **kw):
        a = dict(n_inst=2, pt=FAKE, pts=8, nlp=8, pos0=FAKE, q=FAKE, n_q=5, nh=12, scale=0.0625,
                 out=FAKE, lse=FAKE)
        a.update(kw)
        return lib.sda_prompt_attn_batch(C.byref(pool) if pool is not None else None,
                                         a["n_inst"], a["pt"], a["pts"], a["nlp"], a["pos0"],
                                         a["q"], a["n_q"], a["nh"], a["scale"], a["out"],
                                         a["lse"], None)
    assert call(pool=None) == api.SDA_ERR_INVALID_ARG
    assert call(pool=_pool(head_dim=128)) == api.SDA_ERR_UNSUPPORTED
    assert call(pool=_pool(scale_stride=0)) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=-1) == api.SDA_ERR_INVALID_ARG
    assert call(n_q=0) == api.SDA_ERR_INVALID_ARG
    assert call(nh=0) == api.SDA_ERR_INVALID_ARG
    assert call(n_q=65535, nh=65) == api.SDA_ERR_UNSUPPORTED      # more rows than the grid holds
    assert call(n_q=api.PROMPT_MAX_ROWS + 1, nh=1) == api.SDA_ERR_UNSUPPORTED
    assert call(nlp=0) == api.SDA_ERR_INVALID_ARG                 # a prompt has cells
    assert call(pts=7) == api.SDA_ERR_INVALID_ARG                 # pt_stride < n_logical_pages
    assert call(scale=float("inf")) == api.SDA_ERR_INVALID_ARG
    assert call(pt=None) == api.SDA_ERR_INVALID_ARG
    assert call(pos0=None) == api.SDA_ERR_INVALID_ARG
    assert call(q=FAKE + 4) == api.SDA_ERR_INVALID_ARG
    assert call(out=FAKE + 8) == api.SDA_ERR_INVALID_ARG
    assert call(lse=None) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=0) == api.SDA_OK                           # nothing to do, nothing launched


def test_append_rejects_before_launch():
    lib = api.library()
    def call(pool=None, **kw):
        pool = _pool() if pool is None else pool
        a = dict(n_inst=2, pt=FAKE, pts=8, nlp=8, pos0=FAKE, k=FAKE, v=FAKE, n_new=5)
        a.update(kw)
        return lib.sda_kv_append_batch(C.byref(pool), a["n_inst"], a["pt"], a["pts"], a["nlp"],
                                       a["pos0"], a["k"], a["v"], a["n_new"], None)
    assert lib.sda_kv_append_batch(None, 1, FAKE, 8, 8, FAKE, FAKE, FAKE, 1, None) == api.SDA_ERR_INVALID_ARG
    assert call(pool=_pool(head_dim=128)) == api.SDA_ERR_UNSUPPORTED
    assert call(pool=_pool(page_size=8)) == api.SDA_ERR_UNSUPPORTED
    assert call(pool=_pool(v_codes=None)) == api.SDA_ERR_INVALID_ARG
    assert call(pool=_pool(k_codes=FAKE + 8)) == api.SDA_ERR_INVALID_ARG
    assert call(pool=_pool(scale_stride=0)) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=-1) == api.SDA_ERR_INVALID_ARG
    assert call(n_new=-1) == api.SDA_ERR_INVALID_ARG
    assert call(nlp=-1) == api.SDA_ERR_INVALID_ARG
    assert call(pts=7) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=65536) == api.SDA_ERR_UNSUPPORTED
    assert call(pos0=None) == api.SDA_ERR_INVALID_ARG
    assert call(k=None) == api.SDA_ERR_INVALID_ARG
    assert call(v=FAKE + 4) == api.SDA_ERR_INVALID_ARG
    assert call(pt=None) == api.SDA_ERR_INVALID_ARG
    assert call(n_inst=0) == api.SDA_OK and call(n_new=0) == api.SDA_OK  # nothing launched


def _cpu_call_args():
    """Well-formed CPU tensors for a batched decode call (2 instances, 2
    query positions of 3 heads, 40 selected cells, 8 logical pages)."""
    import torch
    from decode_attention_sparse_amd import api
    cells = 256
    pool = api.Pool(torch.zeros((cells, 256), dtype=torch.int8), torch.zeros(cells, dtype=torch.int16),
                    torch.zeros((cells, 256), dtype=torch.int8), torch.zeros(cells, dtype=torch.int16))
    return dict(pool=pool, page_table=torch.zeros((2, 8), dtype=torch.int32),
                sel=torch.zeros((2, 40), dtype=torch.int32), n_sel=torch.zeros(2, dtype=torch.int32),
                max_sel=40, q=torch.zeros((2, 2, 3, 256)), softmax_scale=0.0625, chunk_cells=64,
                out=torch.zeros((2, 2, 3, 256)), lse=torch.zeros((2, 2, 3)))


@pytest.mark.parametrize("change,msg", [
    (dict(n_sel=("dtype", "int64")), "n_sel must have dtype"),
    (dict(q=("dtype", "float64")), "q must have dtype"),
    (dict(q=("shape", (2, 2, 3, 128))), "q has shape"),
    (dict(out=("shape", (2, 2, 3, 128))), "out has shape"),
    (dict(lse=("shape", (2, 2))), "lse has shape"),
    (dict(sel=("dtype", "int64")), "sel must have dtype"),
    (dict(sel=("shape", (3, 40))), "sel has shape"),
    (dict(page_table=("shape", (1, 8))), "page_table has shape"),
    (dict(max_sel=("value", 41)), "max_sel 41 outside"),
    (dict(n_sel=("shape", (3,))), "n_sel has shape"),
    (dict(pool_v=("shape", (128, 256))), "pool.v_codes has shape"),
    (dict(pool_ks=("shape", (100,))), "pool.k_scales has shape"),
    (dict(pool_ks=("dtype", "int32")), "pool.k_scales must have dtype"),
    (dict(), "must be on a GPU"),
])
def test_binding_rejects_bad_tensors(change, msg):
    """The binding checks dtypes, shapes and devices before calling into the
    library, which trusts the sizes it is given (an int64 count read as int32
    pairs or an undersized tensor would be read out of bounds on the GPU).
    Run with CPU tensors: every call must raise ValueError (the last case is
    well formed except for the device)."""
    import torch
    from decode_attention_sparse_amd import api
    a = _cpu_call_args()
    for key, (what, val) in change.items():
        if key.startswith("pool_"):
            pool = a["pool"]
            attr = {"pool_v": "v_codes", "pool_ks": "k_scales"}[key]
            t = getattr(pool, attr)
            setattr(pool, attr, t.to(getattr(torch, val)) if what == "dtype"
                    else torch.zeros(val, dtype=t.dtype))
        elif what == "dtype":
            a[key] = a[key].to(getattr(torch, val))
        elif what == "shape":
            a[key] = torch.zeros(val, dtype=a[key].dtype)
        else:
            a[key] = val
    with pytest.raises(ValueError, match=msg):
        api.decode_attn_batch(**a)


def test_noalloc_rejects_before_launch():
    """sda_decode_attn_batch_noalloc validates like sda_decode_attn_batch and
    refuses a call whose chunk partials exceed the fixed device array, all
    before it touches a device (no GPU here)."""
    lib = api.library()
    p = _pool()
    def call(**kw):
        a = dict(n_inst=2, pt=FAKE, pts=4, nlp=4, sel=FAKE, sels=10, nsel=FAKE, max_sel=10,
                 q=FAKE, n_q=1, nh=12, scale=0.0625, chunk=256, out=FAKE, lse=FAKE, g=None)
        a.update(kw)
        return lib.sda_decode_attn_batch_noalloc(
            C.byref(p), a["n_inst"], a["pt"], a["pts"], a["nlp"], a["sel"], a["sels"], a["nsel"],
            a["max_sel"], a["q"], a["n_q"], a["nh"], a["scale"], a["chunk"], a["out"], a["lse"],
            a["g"], None)
    assert call(nsel=None) == api.SDA_ERR_INVALID_ARG
    assert call(pts=3) == api.SDA_ERR_INVALID_ARG
    assert call(sels=9) == api.SDA_ERR_INVALID_ARG
    assert call(out=None) == api.SDA_ERR_INVALID_ARG
    assert call(q=FAKE + 4) == api.SDA_ERR_INVALID_ARG
    assert call(n_q=5, nh=13) == api.SDA_ERR_UNSUPPORTED
    assert call(chunk=96) == api.SDA_ERR_UNSUPPORTED
    assert call(n_inst=0) == api.SDA_OK
    # 128 instances x 64 rows x 4,096 cells: four chunks per instance, whose
    # partials (33.8 MB) exceed the array
    big = dict(n_inst=128, n_q=4, nh=16, max_sel=4096, sels=4096, chunk=256)
    assert not api.fused_single_launch(128, 4, 16, 4096, 256)
    need = api.workspace_bytes(128, 4, 16, 4096, api.fused_chunk_cells(128, 4096, 256))
    assert need > api.SCRATCH_BYTES
    assert call(**big) == api.SDA_ERR_SCRATCH


def test_qsa_rejects_before_launch():
    """The QSA entry points validate geometry and pointers on the host (no GPU
    here: every call below must fail before anything is launched)."""
    lib = api.library()
    def scores(**kw):
        a = dict(n_inst=2, n_rows=2, n_heads=4, idx_dim=128, R=256, B=512, pooled=FAKE,
                 dead=FAKE, q=FAKE, vis=FAKE, out=FAKE)
        a.update(kw)
        return lib.sda_qsa_block_scores(a["n_inst"], a["n_rows"], a["n_heads"], a["idx_dim"],
                                        a["R"], a["B"], a["pooled"], a["dead"], a["q"],
                                        a["vis"], a["out"], None)
    assert scores(n_rows=0) == api.SDA_ERR_INVALID_ARG
    assert scores(n_rows=9) == api.SDA_ERR_UNSUPPORTED
    assert scores(idx_dim=100) == api.SDA_ERR_UNSUPPORTED        # 400 not a multiple of 64
    assert scores(n_heads=16) == api.SDA_ERR_UNSUPPORTED         # 2048 > 1024
    assert scores(R=100) == api.SDA_ERR_UNSUPPORTED              # not a multiple of 16
    assert scores(R=0) == api.SDA_ERR_INVALID_ARG
    assert scores(B=0) == api.SDA_ERR_INVALID_ARG
    assert scores(B=1 << 24, R=256) == api.SDA_ERR_UNSUPPORTED   # more than 2^31 cells
    assert scores(n_inst=70000) == api.SDA_ERR_UNSUPPORTED
    assert scores(pooled=None) == api.SDA_ERR_INVALID_ARG
    assert scores(q=FAKE + 4) == api.SDA_ERR_INVALID_ARG
    assert scores(n_inst=0) == api.SDA_OK
    def select(**kw):
        a = dict(n_inst=2, n_rows=2, R=256, B=512, sc=FAKE, vis=FAKE, k=64, sel=FAKE,
                 stride=64 * 256, nsel=FAKE)
        a.update(kw)
        return lib.sda_qsa_select(a["n_inst"], a["n_rows"], a["R"], a["B"], a["sc"], a["vis"],
                                  a["k"], a["sel"], a["stride"], a["nsel"], None)
    assert select(k=-1) == api.SDA_ERR_INVALID_ARG
    assert select(k=4097) == api.SDA_ERR_UNSUPPORTED
    assert select(B=16385) == api.SDA_ERR_UNSUPPORTED
    assert select(stride=64 * 256 - 1) == api.SDA_ERR_INVALID_ARG
    assert select(nsel=None) == api.SDA_ERR_INVALID_ARG
    assert select(sel=None) == api.SDA_ERR_INVALID_ARG
    assert select(sc=None) == api.SDA_ERR_INVALID_ARG
    assert select(n_inst=0) == api.SDA_OK
