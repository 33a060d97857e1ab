// extern "C" entry points of libsda.so (declared in include/sda.h):
// host-side validation, workspace layout, and the kernel launches on the
// caller's stream (chunk pass + merge pass, or the chunk kernel's
// single-launch form).  No allocation, no synchronisation, no global state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/sda.h"
#include "sda_internal.h"

// The chunk partials of sda_decode_attn_batch_noalloc: one array per GPU,
// loaded with the library's code object and kept until the process ends.
// In host code its name is only a handle for hipGetSymbolAddress; kernels
// get the device address that call returns (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[SDA_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

struct Layout {
    size_t acc_off, m_off, l_off, total;
    int32_t n_chunks;
};

// Returns SDA_OK and the partials layout, or an error for bad geometry.
int layout_of(int64_t n_inst, int32_t n_q, int32_t n_qheads, int32_t head_dim, int32_t max_sel,
              int32_t chunk_cells, Layout *L) {
    if (n_inst < 0 || n_q < 1 || n_qheads < 1 || max_sel < 0 || chunk_cells < 1)
        return SDA_ERR_INVALID_ARG;
    if (head_dim != SDA_HEAD_DIM) return SDA_ERR_UNSUPPORTED;
    if ((int64_t)n_q * n_qheads > SDA_MAX_ROWS) return SDA_ERR_UNSUPPORTED;
    if (chunk_cells % SDA_CHUNK_ALIGN) return SDA_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)n_q * n_qheads;
    const int64_t n_chunks = (max_sel + (int64_t)chunk_cells - 1) / chunk_cells;
    if (n_chunks > SDA_MAX_CHUNKS) return SDA_ERR_UNSUPPORTED;
    const size_t units = (size_t)n_inst * (size_t)n_chunks * (size_t)rows;
    L->n_chunks = (int32_t)n_chunks;
    L->acc_off = 0;
    L->m_off = align_up(units * head_dim * sizeof(float));
    L->l_off = L->m_off + align_up(units * sizeof(float));
    L->total = L->l_off + align_up(units * sizeof(float));
    if (units == 0) L->total = 0;
    return SDA_OK;
}

enum Passes { kChunk = 1, kMerge = 2, kBoth = 3 };

// (instance, chunk) pairs up to which a chunk pass is one workgroup per CU,
// and the workgroups the chunk kernel keeps resident (two per CU).
constexpr int64_t kLatencyItems = 256;
constexpr int64_t kResidentItems = 512;

// Chunk size the fused call (chunk pass + merge in one call) uses.
//  - A grid of at most kLatencyItems (instance, chunk) pairs is
//    latency-bound, and a workgroup's time grows with the tiles it runs one
//    after another: the call splits the list into the smallest multiple of
//    64 cells that still keeps the grid within kLatencyItems.
//  - Otherwise, with at most kLatencyItems instances: m = kResidentItems /
//    n_inst (at least 2) balanced chunks per instance, at most the caller's
//    number, so the grid fills the two resident workgroups per CU in one
//    round and no workgroup holds a short tail chunk.
//  - Otherwise, a grid of more than kResidentItems pairs would run
//    k = pairs / kResidentItems consecutive chunks per workgroup; the call
//    takes chunks k times the caller's, so that each workgroup leaves one
//    partial instead of k (less partial traffic, a shorter merge).
//  - Otherwise the caller's chunk.
// The merge combines whatever partials the chunk pass leaves.
int32_t fused_chunk_of(int64_t n_inst, int32_t max_sel, int32_t chunk_cells) {
    if (n_inst <= 0 || max_sel <= 0) return chunk_cells;
    auto items = [&](int64_t c) { return n_inst * (((int64_t)max_sel + c - 1) / c); };
    const int64_t pairs = items(chunk_cells);
    if (pairs <= kLatencyItems) {
        for (int32_t c = SDA_CHUNK_ALIGN; c < chunk_cells; c += SDA_CHUNK_ALIGN)
            if (items(c) <= kLatencyItems) return c;
        return chunk_cells;
    }
    const int64_t per_inst = ((int64_t)max_sel + chunk_cells - 1) / chunk_cells;
    if (n_inst <= kLatencyItems) {
        int64_t m = kResidentItems / n_inst;
        if (m > per_inst) m = per_inst;
        const int64_t len = ((int64_t)max_sel + m - 1) / m;  // balanced
        const int64_t c = (len + SDA_CHUNK_ALIGN - 1) / SDA_CHUNK_ALIGN * SDA_CHUNK_ALIGN;
        return c > INT32_MAX ? chunk_cells : (int32_t)c;
    }
    if (pairs > kResidentItems) {
        int64_t k = pairs / kResidentItems;
        if (k > per_inst) k = per_inst;
        const int64_t c = (int64_t)chunk_cells * k;
        return c > INT32_MAX ? chunk_cells : (int32_t)c;
    }
    return chunk_cells;
}

int check_pool(const sda_pool *pool) {
    if (!pool) return SDA_ERR_INVALID_ARG;
    if (pool->page_size != SDA_PAGE_SIZE || pool->head_dim != SDA_HEAD_DIM)
        return SDA_ERR_UNSUPPORTED;
    if (!pool->k_codes || !pool->v_codes || !pool->k_scales || !pool->v_scales)
        return SDA_ERR_INVALID_ARG;
    if (pool->n_phys_pages < 1 || pool->n_phys_pages > ((int64_t)1 << 27))
        return SDA_ERR_INVALID_ARG;
    if (pool->scale_stride < 1 || pool->scale_stride > 64 || pool->reserved != 0)
        return SDA_ERR_INVALID_ARG;
    if (!aligned(pool->k_codes, 16) || !aligned(pool->v_codes, 16) ||
        !aligned(pool->k_scales, 2) || !aligned(pool->v_scales, 2))
        return SDA_ERR_INVALID_ARG;
    return SDA_OK;
}

void set_pool(sda::Params *p, const sda_pool *pool) {
    p->k_codes = pool->k_codes;
    p->k_scales = pool->k_scales;
    p->v_codes = pool->v_codes;
    p->v_scales = pool->v_scales;
    p->scale_stride = pool->scale_stride;
    p->n_phys_pages = pool->n_phys_pages;
}

// A validated decode call: its parameters (all but the partials' pointers),
// the partials' layout and whether it runs as one chunk-kernel launch.
struct Call {
    sda::Params p;
    Layout L;
    bool single;
    int passes;
};

// Host-side validation of a decode call (everything but the workspace) into
// c; SDA_OK with c->p.n_inst == 0 means there is nothing to launch.
int prepare(const sda_pool *pool, int32_t n_inst, const int32_t *page_table, int64_t pt_stride,
            int32_t n_logical_pages, const int32_t *sel, int64_t sel_stride,
            const int32_t *n_sel_dev, int32_t n_sel_host, int32_t max_sel, const float *q,
            int32_t n_q, int32_t n_qheads, float softmax_scale, int32_t chunk_cells, float *out,
            float *lse, int32_t *gather_out, int passes, Call *c) {
    int st = check_pool(pool);
    if (st != SDA_OK) return st;
    Layout &L = c->L;
    st = layout_of(n_inst, n_q, n_qheads, pool->head_dim, max_sel, chunk_cells, &L);
    if (st != SDA_OK) return st;
    // the fused call may run finer chunks (same layout, smaller chunk size)
    const int32_t run_chunk =
        passes == kBoth ? fused_chunk_of(n_inst, max_sel, chunk_cells) : chunk_cells;
    if (run_chunk != chunk_cells &&
        layout_of(n_inst, n_q, n_qheads, pool->head_dim, max_sel, run_chunk, &L) != SDA_OK)
        return SDA_ERR_UNSUPPORTED;
    if (n_logical_pages < 0 || pt_stride < n_logical_pages || sel_stride < max_sel)
        return SDA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale)) return SDA_ERR_INVALID_ARG;
    sda::Params &p = c->p;
    memset(&p, 0, sizeof p);
    c->passes = passes;
    c->single = false;
    if (n_inst == 0) return SDA_OK;
    if (!q || !aligned(q, 16)) return SDA_ERR_INVALID_ARG;
    if ((passes & kMerge) && (!out || !lse || !aligned(out, 16) || !aligned(lse, 4)))
        return SDA_ERR_INVALID_ARG;
    if (n_logical_pages > 0 && !page_table) return SDA_ERR_INVALID_ARG;
    if (max_sel > 0 && !sel) return SDA_ERR_INVALID_ARG;

    set_pool(&p, pool);
    p.page_table = page_table;
    p.pt_stride = pt_stride;
    p.n_logical_pages = n_logical_pages;
    p.sel = sel;
    p.sel_stride = sel_stride;
    p.n_sel_dev = n_sel_dev;
    p.n_sel_host = n_sel_host;
    p.max_sel = max_sel;
    p.q = q;
    p.n_inst = n_inst;
    p.n_rows = n_q * n_qheads;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.chunk = run_chunk;
    p.n_chunks = L.n_chunks;
    p.gather_out = gather_out;
    p.out = out;
    p.lse = lse;
    // a fused call that runs as one launch leaves the partials untouched
    c->single = passes == kBoth && sda::chunk_writes_output(p);
    return SDA_OK;
}

// Bytes of partials a prepared call reads and writes (0 for a single launch).
size_t partial_bytes(const Call &c) { return c.single ? 0 : c.L.total; }

// Launches a prepared call with its partials at workspace (at least
// partial_bytes(c) bytes, 256-byte aligned, when that is not 0).
int launch(Call &c, void *workspace, void *stream) {
    if (c.p.n_inst == 0) return SDA_OK;
    sda::Params &p = c.p;
    char *ws = static_cast<char *>(workspace);
    const bool has = partial_bytes(c) > 0;
    p.acc = has ? reinterpret_cast<float *>(ws + c.L.acc_off) : nullptr;
    p.m = has ? reinterpret_cast<float *>(ws + c.L.m_off) : nullptr;
    p.l = has ? reinterpret_cast<float *>(ws + c.L.l_off) : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // clear a stale error so it is not blamed on us
    if (c.single)
        return sda::launch_chunk_final(p, s) == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
    if ((c.passes & kChunk) && p.n_chunks > 0 && sda::launch_chunk(p, s) != hipSuccess)
        return SDA_ERR_LAUNCH;
    if ((c.passes & kMerge) && sda::launch_merge(p, s) != hipSuccess) return SDA_ERR_LAUNCH;
    return SDA_OK;
}

// A call with the caller's workspace.  The public entry points ask for the
// whole layout's size even when the call is a single launch that does not
// touch it.
int run(const sda_pool *pool, int32_t n_inst, const int32_t *page_table, int64_t pt_stride,
        int32_t n_logical_pages, const int32_t *sel, int64_t sel_stride,
        const int32_t *n_sel_dev, int32_t n_sel_host, int32_t max_sel, const float *q,
        int32_t n_q, int32_t n_qheads, float softmax_scale, int32_t chunk_cells, float *out,
        float *lse, int32_t *gather_out, void *workspace, size_t workspace_bytes, void *stream,
        int passes = kBoth) {
    Call c;
    int st = prepare(pool, n_inst, page_table, pt_stride, n_logical_pages, sel, sel_stride,
                     n_sel_dev, n_sel_host, max_sel, q, n_q, n_qheads, softmax_scale, chunk_cells,
                     out, lse, gather_out, passes, &c);
    if (st != SDA_OK || n_inst == 0) return st;
    if (c.L.total > 0 && (!workspace || workspace_bytes < c.L.total || !aligned(workspace, kAlign)))
        return SDA_ERR_WORKSPACE;
    return launch(c, workspace, stream);
}

// Device address of the current device's scratch array, resolved once per
// device with that device current and kept for later calls.
constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];

int scratch_ptr(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return SDA_ERR_LAUNCH;
        }
        scratch_addr[dev] = p;
    }
    *ptr = scratch_addr[dev];
    return SDA_OK;
}

}  // namespace

extern "C" {

int sda_workspace_bytes(int32_t n_inst, int32_t n_q, int32_t n_qheads, int32_t head_dim,
                        int32_t max_sel, int32_t chunk_cells, size_t *bytes) {
    if (!bytes) return SDA_ERR_INVALID_ARG;
    Layout L, F;
    int st = layout_of(n_inst, n_q, n_qheads, head_dim, max_sel, chunk_cells, &L);
    if (st != SDA_OK) return st;
    st = layout_of(n_inst, n_q, n_qheads, head_dim, max_sel,
                   fused_chunk_of(n_inst, max_sel, chunk_cells), &F);
    if (st != SDA_OK) return st;
    *bytes = L.total > F.total ? L.total : F.total;
    return SDA_OK;
}

int sda_fused_chunk_cells(int32_t n_inst, int32_t max_sel, int32_t chunk_cells,
                          int32_t *fused_chunk_cells) {
    if (!fused_chunk_cells || n_inst < 0 || max_sel < 0 || chunk_cells < 1)
        return SDA_ERR_INVALID_ARG;
    if (chunk_cells % SDA_CHUNK_ALIGN) return SDA_ERR_UNSUPPORTED;
    *fused_chunk_cells = fused_chunk_of(n_inst, max_sel, chunk_cells);
    return SDA_OK;
}

int sda_fused_single_launch(int32_t n_inst, int32_t n_q, int32_t n_qheads, int32_t max_sel,
                            int32_t chunk_cells, int32_t *single_launch) {
    if (!single_launch || n_inst < 0 || max_sel < 0 || chunk_cells < 1 || n_q < 1 ||
        n_qheads < 1)
        return SDA_ERR_INVALID_ARG;
    if (chunk_cells % SDA_CHUNK_ALIGN || (int64_t)n_q * n_qheads > SDA_MAX_ROWS)
        return SDA_ERR_UNSUPPORTED;
    sda::Params p;
    memset(&p, 0, sizeof p);
    p.n_inst = n_inst;
    p.n_rows = n_q * n_qheads;
    p.chunk = fused_chunk_of(n_inst, max_sel, chunk_cells);
    p.n_chunks = (int32_t)(((int64_t)max_sel + p.chunk - 1) / p.chunk);
    *single_launch = sda::chunk_writes_output(p) ? 1 : 0;
    return SDA_OK;
}

int sda_decode_attn_step(const sda_pool *pool, const int32_t *page_table,
                         int32_t n_logical_pages, const int32_t *sel, int32_t n_sel,
                         const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                         int32_t chunk_cells, float *out, float *lse, int32_t *gather_out,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (n_sel < 0) return SDA_ERR_INVALID_ARG;
    return run(pool, 1, page_table, n_logical_pages, n_logical_pages, sel, n_sel, nullptr,
               n_sel, n_sel, q, n_q, n_qheads, softmax_scale, chunk_cells, out, lse, gather_out,
               workspace, workspace_bytes, stream);
}

int sda_decode_attn_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                          int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                          int64_t sel_stride, const int32_t *n_sel, int32_t max_sel,
                          const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                          int32_t chunk_cells, float *out, float *lse, int32_t *gather_out,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (n_inst > 0 && !n_sel) return SDA_ERR_INVALID_ARG;
    return run(pool, n_inst, page_table, pt_stride, n_logical_pages, sel, sel_stride, n_sel, 0,
               max_sel, q, n_q, n_qheads, softmax_scale, chunk_cells, out, lse, gather_out,
               workspace, workspace_bytes, stream);
}

int sda_decode_attn_batch_noalloc(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                                  int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                                  int64_t sel_stride, const int32_t *n_sel, int32_t max_sel,
                                  const float *q, int32_t n_q, int32_t n_qheads,
                                  float softmax_scale, int32_t chunk_cells, float *out,
                                  float *lse, int32_t *gather_out, void *stream) {
    if (n_inst > 0 && !n_sel) return SDA_ERR_INVALID_ARG;
    Call c;
    int st = prepare(pool, n_inst, page_table, pt_stride, n_logical_pages, sel, sel_stride, n_sel,
                     0, max_sel, q, n_q, n_qheads, softmax_scale, chunk_cells, out, lse,
                     gather_out, kBoth, &c);
    if (st != SDA_OK || n_inst == 0) return st;
    const size_t need = partial_bytes(c);
    if (need > SDA_SCRATCH_BYTES) return SDA_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_ptr(&ws);
        if (st != SDA_OK) return st;
    }
    return launch(c, ws, stream);
}

int sda_chunk_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                    int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                    int64_t sel_stride, const int32_t *n_sel, int32_t max_sel, const float *q,
                    int32_t n_q, int32_t n_qheads, float softmax_scale, int32_t chunk_cells,
                    int32_t *gather_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (n_inst > 0 && !n_sel) return SDA_ERR_INVALID_ARG;
    return run(pool, n_inst, page_table, pt_stride, n_logical_pages, sel, sel_stride, n_sel, 0,
               max_sel, q, n_q, n_qheads, softmax_scale, chunk_cells, nullptr, nullptr,
               gather_out, workspace, workspace_bytes, stream, kChunk);
}

int sda_merge_batch(int32_t n_inst, int32_t n_q, int32_t n_qheads, const int32_t *n_sel,
                    int32_t max_sel, int32_t chunk_cells, const void *workspace,
                    size_t workspace_bytes, float *out, float *lse, void *stream) {
    Layout L;
    int st = layout_of(n_inst, n_q, n_qheads, SDA_HEAD_DIM, max_sel, chunk_cells, &L);
    if (st != SDA_OK) return st;
    if (n_inst == 0) return SDA_OK;
    if (!n_sel || !out || !lse || !aligned(out, 16) || !aligned(lse, 4)) return SDA_ERR_INVALID_ARG;
    if (L.total > 0 && (!workspace || workspace_bytes < L.total || !aligned(workspace, kAlign)))
        return SDA_ERR_WORKSPACE;
    sda::Params p;
    memset(&p, 0, sizeof p);
    p.n_sel_dev = n_sel;
    p.max_sel = max_sel;
    p.n_inst = n_inst;
    p.n_rows = n_q * n_qheads;
    p.chunk = chunk_cells;
    p.n_chunks = L.n_chunks;
    char *ws = static_cast<char *>(const_cast<void *>(workspace));
    p.acc = L.total ? reinterpret_cast<float *>(ws + L.acc_off) : nullptr;
    p.m = L.total ? reinterpret_cast<float *>(ws + L.m_off) : nullptr;
    p.l = L.total ? reinterpret_cast<float *>(ws + L.l_off) : nullptr;
    p.out = out;
    p.lse = lse;
    (void)hipGetLastError();
    if (sda::launch_merge(p, static_cast<hipStream_t>(stream)) != hipSuccess) return SDA_ERR_LAUNCH;
    return SDA_OK;
}

int sda_prompt_attn_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                          int64_t pt_stride, int32_t n_logical_pages, const int32_t *pos0,
                          const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                          float *out, float *lse, void *stream) {
    int st = check_pool(pool);
    if (st != SDA_OK) return st;
    if (n_inst < 0 || n_q < 1 || n_qheads < 1) return SDA_ERR_INVALID_ARG;
    if ((int64_t)n_q * n_qheads > SDA_PROMPT_MAX_ROWS) return SDA_ERR_UNSUPPORTED;
    if (n_logical_pages < 1 || pt_stride < n_logical_pages) return SDA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale)) return SDA_ERR_INVALID_ARG;
    if (n_inst == 0) return SDA_OK;
    if (!page_table || !pos0 || !q || !aligned(q, 16) || !out || !aligned(out, 16) || !lse ||
        !aligned(lse, 4))
        return SDA_ERR_INVALID_ARG;
    sda::Params p;
    memset(&p, 0, sizeof p);
    set_pool(&p, pool);
    p.page_table = page_table;
    p.pt_stride = pt_stride;
    p.n_logical_pages = n_logical_pages;
    p.q = q;
    p.n_inst = n_inst;
    p.n_rows = n_q * n_qheads;
    p.n_qheads = n_qheads;
    p.pos0 = pos0;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.out = out;
    p.lse = lse;
    (void)hipGetLastError();
    if (sda::launch_prompt(p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return SDA_ERR_LAUNCH;
    return SDA_OK;
}

int sda_kv_append_batch(const sda_pool_mut *pool, int32_t n_inst, const int32_t *page_table,
                        int64_t pt_stride, int32_t n_logical_pages, const int32_t *pos0,
                        const float *k_new, const float *v_new, int32_t n_new, void *stream) {
    if (!pool) return SDA_ERR_INVALID_ARG;
    const sda_pool view = {pool->k_codes, pool->k_scales, pool->v_codes, pool->v_scales,
                           pool->n_phys_pages, pool->page_size, pool->head_dim,
                           pool->scale_stride, pool->reserved};
    int st = check_pool(&view);
    if (st != SDA_OK) return st;
    if (n_inst < 0 || n_new < 0 || n_logical_pages < 0 || pt_stride < n_logical_pages)
        return SDA_ERR_INVALID_ARG;
    if (n_inst > 65535) return SDA_ERR_UNSUPPORTED;
    if (n_inst == 0 || n_new == 0) return SDA_OK;
    if (!pos0 || !k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
        return SDA_ERR_INVALID_ARG;
    if (n_logical_pages > 0 && !page_table) return SDA_ERR_INVALID_ARG;
    sda::AppendParams p;
    memset(&p, 0, sizeof p);
    p.k_codes = pool->k_codes;
    p.k_scales = pool->k_scales;
    p.v_codes = pool->v_codes;
    p.v_scales = pool->v_scales;
    p.scale_stride = pool->scale_stride;
    p.n_phys_pages = pool->n_phys_pages;
    p.page_table = page_table;
    p.pt_stride = pt_stride;
    p.n_logical_pages = n_logical_pages;
    p.pos0 = pos0;
    p.k_new = k_new;
    p.v_new = v_new;
    p.n_inst = n_inst;
    p.n_new = n_new;
    (void)hipGetLastError();
    if (sda::launch_kv_append(p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return SDA_ERR_LAUNCH;
    return SDA_OK;
}

int sda_qsa_block_scores(int32_t n_inst, int32_t n_rows, int32_t n_heads, int32_t idx_dim,
                         int32_t block_cells, int32_t max_blocks, const float *pooled,
                         const uint8_t *dead, const float *q_idx, const int32_t *n_visible,
                         float *scores, void *stream) {
    if (n_inst < 0 || n_rows < 1 || n_heads < 1 || idx_dim < 1 || block_cells < 1 ||
        max_blocks < 1)
        return SDA_ERR_INVALID_ARG;
    const int64_t hd = (int64_t)n_heads * idx_dim;
    if (n_rows > SDA_QSA_MAX_ROWS || hd % SDA_QSA_HD_ALIGN || hd > SDA_QSA_MAX_HD ||
        block_cells % SDA_PAGE_SIZE || (int64_t)max_blocks * block_cells > INT32_MAX ||
        n_inst > 65535)
        return SDA_ERR_UNSUPPORTED;
    if (n_inst == 0) return SDA_OK;
    if (!pooled || !dead || !q_idx || !n_visible || !scores || !aligned(pooled, 16) ||
        !aligned(q_idx, 16) || !aligned(scores, 4))
        return SDA_ERR_INVALID_ARG;
    sda::QsaParams p;
    memset(&p, 0, sizeof p);
    p.pooled = pooled;
    p.dead = dead;
    p.q_idx = q_idx;
    p.n_visible = n_visible;
    p.scores = scores;
    p.n_inst = n_inst;
    p.n_rows = n_rows;
    p.hd = (int32_t)hd;
    p.block_cells = block_cells;
    p.max_blocks = max_blocks;
    (void)hipGetLastError();
    return sda::launch_qsa_scores(p, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SDA_OK
               : SDA_ERR_LAUNCH;
}

int sda_qsa_select(int32_t n_inst, int32_t n_rows, int32_t block_cells, int32_t max_blocks,
                   const float *scores, const int32_t *n_visible, int32_t k_blocks,
                   int32_t *sel, int64_t sel_stride, int32_t *n_sel, void *stream) {
    if (n_inst < 0 || n_rows < 1 || block_cells < 1 || max_blocks < 1 || k_blocks < 0)
        return SDA_ERR_INVALID_ARG;
    if (n_rows > SDA_QSA_MAX_ROWS || block_cells % SDA_PAGE_SIZE ||
        max_blocks > SDA_QSA_MAX_BLOCKS || k_blocks > SDA_QSA_MAX_K ||
        (int64_t)max_blocks * block_cells > INT32_MAX)
        return SDA_ERR_UNSUPPORTED;
    if (sel_stride < (int64_t)k_blocks * block_cells) return SDA_ERR_INVALID_ARG;
    if (n_inst == 0) return SDA_OK;
    if (!scores || !n_visible || !n_sel || (k_blocks > 0 && !sel)) return SDA_ERR_INVALID_ARG;
    sda::QsaParams p;
    memset(&p, 0, sizeof p);
    p.scores = const_cast<float *>(scores);
    p.n_visible = n_visible;
    p.sel = sel;
    p.n_sel = n_sel;
    p.sel_stride = sel_stride;
    p.n_inst = n_inst;
    p.n_rows = n_rows;
    p.block_cells = block_cells;
    p.max_blocks = max_blocks;
    p.k_blocks = k_blocks;
    (void)hipGetLastError();
    return sda::launch_qsa_select(p, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SDA_OK
               : SDA_ERR_LAUNCH;
}

const char *sda_status_string(int status) {
    switch (status) {
        case SDA_OK: return "SDA_OK";
        case SDA_ERR_INVALID_ARG: return "SDA_ERR_INVALID_ARG: invalid argument";
        case SDA_ERR_UNSUPPORTED: return "SDA_ERR_UNSUPPORTED: unsupported geometry";
        case SDA_ERR_WORKSPACE: return "SDA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case SDA_ERR_LAUNCH: return "SDA_ERR_LAUNCH: kernel launch failed";
        case SDA_ERR_SCRATCH:
            return "SDA_ERR_SCRATCH: the call's chunk partials exceed the library's fixed "
                   "device scratch array (SDA_SCRATCH_BYTES)";
        default: return "unknown sda status";
    }
}

}  // extern "C"
