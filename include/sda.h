/*
 * sda.h -- C ABI of libsda.so: decode-time attention over a selected subset
 * of KV cells held as INT8 K/V pools behind a page table, on MI355X (gfx950).
 *
 * What is computed (Strata PR #2220 page, the decode attention over the QSA
 * selection and its "Kernel (chunk kernel + merge ...)" benchmark; Strata
 * round-9 page, section "R9-gpu-11: four score cells per step in daily INT8
 * attention"):
 *
 *   For every instance i (one sequence x one KV head), every query row
 *   r = t * n_qheads + h (query position t, grouped query head h sharing the
 *   KV head) and every selected list entry j < n_sel[i]:
 *
 *     gather    c = sel[i][j];  p = page_table[i][c / 16];
 *               phys_j = p * 16 + c % 16, or -1 ("masked") when c is outside
 *               [0, 16 * n_logical_pages) or p is outside [0, n_phys_pages)
 *               (page id -1 is the documented way to mask a page)
 *     score     s_j = softmax_scale * k_scale[phys_j] * sum_d q[r][d] * k_code[phys_j][d]
 *     chunk     list positions [c*chunk_cells, (c+1)*chunk_cells) form chunk c;
 *               its partial is m_c = max s_j, l_c = sum e^(s_j - m_c),
 *               acc_c[d] = sum e^(s_j - m_c) * v_scale[phys_j] * v_code[phys_j][d]
 *               over the chunk's unmasked cells (empty: m = -inf, l = 0, acc = 0)
 *     merge     M = max m_c, L = sum l_c e^(m_c - M),
 *               out[r][d] = sum acc_c[d] e^(m_c - M) / L,  lse[r] = M + ln L
 *               (no unmasked cell: out = 0, lse = -inf)
 *
 *   Every query position of an instance attends to the instance's whole
 *   selection (no causal mask between verify positions).  Duplicate list
 *   entries count once each.
 *
 * Two entry points mirror the pages' step (one sequence) and batch (many
 * instances) entry points; both run the chunk pass, then the merge, on the
 * caller's stream (or, when every instance has at most two chunks, one
 * chunk-kernel launch that merges in place: sda_fused_single_launch).  The
 * chunk size is a parameter of the method that changes the result only by
 * rounding; these fused calls choose it from the grid
 * (sda_fused_chunk_cells).
 *
 * Memory and threading contract (all entry points):
 *   - Every array argument is a DEVICE pointer unless marked "host".  The
 *     caller owns all memory; the library never allocates, frees, copies to
 *     the host or synchronises, and keeps no state between calls, so calls
 *     may be captured into a HIP graph and replayed.  (The one exception,
 *     sda_decode_attn_batch_noalloc, keeps its partials in a device array
 *     the library holds per GPU and remembers that array's address.)
 *   - Arguments are validated on the host before anything is launched; a
 *     non-zero status means nothing was launched.  Unsupported geometry
 *     returns SDA_ERR_UNSUPPORTED so that a caller can fall back.
 *   - Launch failures reported by the runtime return SDA_ERR_LAUNCH.
 *   - SDA_OK means that the work was launched, not that it finished well:
 *     launches are asynchronous and no call reads anything back.  One
 *     device-side failure is reported in the outputs instead: the
 *     two-pipeline forms of the chunk pass (a workgroup running two chunks
 *     side by side: the fused decode calls when sda_fused_single_launch
 *     holds and an instance has two chunks, and chunk passes of 17-32 rows
 *     with one chunk per workgroup, in the fused calls and in
 *     sda_chunk_batch) synchronise their waves with bounded waits on LDS
 *     flags; a wait that gives up (tens of milliseconds, never in a correct
 *     run) writes NaN to the out and lse rows of that workgroup, or to the
 *     denominators of its chunk partials, which the merge turns into NaN
 *     rows, and the call has still returned SDA_OK.  A finite output is
 *     therefore part of a successful call's result: a caller that needs
 *     certainty checks out and lse for NaN.
 *   - Device-side contents are trusted for shape (n_sel[i] is clamped to
 *     [0, max_sel]); ids out of range are masked, never dereferenced.
 *   - Outputs (out, lse, gather_out, the workspace, and the pools of
 *     sda_kv_append_batch) must not overlap any other argument's memory.
 *   - Calls on different streams that share a workspace or an output race.
 */
#ifndef SDA_H
#define SDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDA_PAGE_SIZE 16 /* cells per page (the only supported value) */
#define SDA_HEAD_DIM 256 /* dims per head (the only supported value) */
#define SDA_MAX_ROWS 64  /* n_q * n_qheads limit */
#define SDA_CHUNK_ALIGN 64 /* chunk_cells must be a positive multiple of this */
#define SDA_MAX_CHUNKS 65535 /* ceil(max_sel / chunk_cells) limit (one grid dimension) */
#define SDA_PROMPT_MAX_ROWS 3145680 /* n_q * n_qheads limit of sda_prompt_attn_batch (65535 x 48) */

typedef enum {
    SDA_OK = 0,
    SDA_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad stride/alignment */
    SDA_ERR_UNSUPPORTED = -2, /* geometry this library does not implement */
    SDA_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
    SDA_ERR_LAUNCH = -4,      /* the HIP runtime rejected a kernel launch */
    SDA_ERR_SCRATCH = -5      /* sda_decode_attn_batch_noalloc: the call needs more
                                 than SDA_SCRATCH_BYTES of chunk partials */
} sda_status;

/* The INT8 pools, indexed by physical cell = physical page * 16 + slot.
 *   k_codes, v_codes: int8 [n_phys_pages * 16][head_dim], row-major, 16-byte
 *                     aligned; the dequantised value is code * scale.
 *   k_scales, v_scales: IEEE binary16 bit patterns, one scale per physical
 *                     cell: the scales of cell c are k_scales[c * scale_stride]
 *                     and v_scales[c * scale_stride].
 *   scale_stride:     >= 1.  1: two separate arrays.  2 with v_scales =
 *                     k_scales + 1: (K, V) pairs interleaved per cell, so that
 *                     the two scales of a cell share one memory sector (the
 *                     cheaper layout when cells are gathered at random).
 * n_phys_pages must be in [1, 2^27]. */
typedef struct sda_pool {
    const int8_t *k_codes;
    const uint16_t *k_scales;
    const int8_t *v_codes;
    const uint16_t *v_scales;
    int64_t n_phys_pages;
    int32_t page_size;    /* must be SDA_PAGE_SIZE */
    int32_t head_dim;     /* must be SDA_HEAD_DIM */
    int32_t scale_stride; /* elements between the scales of consecutive cells */
    int32_t reserved;     /* must be 0 */
} sda_pool;

/* Workspace needed by one call (host only, no device access).
 * bytes (host out) = size of the chunk partials for chunk_cells or for
 * sda_fused_chunk_cells(n_inst, max_sel, chunk_cells), whichever is larger.
 * Partials are laid out from the start of the workspace as
 *     acc  float [n_inst][n_chunks][R][head_dim]
 *     m    float [n_inst][n_chunks][R]   (natural-log units, -inf if empty)
 *     l    float [n_inst][n_chunks][R]
 * with R = n_q * n_qheads, n_chunks = ceil(max_sel / chunk_cells) (at most
 * SDA_MAX_CHUNKS, else SDA_ERR_UNSUPPORTED), and each
 * of the three arrays starting at a 256-byte aligned offset (acc at 0, m at
 * align256(sizeof acc), l at m + align256(sizeof m)).  After a call these
 * hold the chunk partials of the chunks that instance actually has
 * (c < ceil(n_sel[i] / C)); other entries are unspecified.  C is
 * chunk_cells after sda_chunk_batch, and sda_fused_chunk_cells(...) after
 * sda_decode_attn_step / sda_decode_attn_batch, except after a fused call
 * that runs as a single launch (sda_fused_single_launch), which does not
 * touch the workspace.
 * Returns SDA_OK, SDA_ERR_INVALID_ARG or SDA_ERR_UNSUPPORTED. */
int sda_workspace_bytes(int32_t n_inst, int32_t n_q, int32_t n_qheads, int32_t head_dim,
                        int32_t max_sel, int32_t chunk_cells, size_t *bytes);

/* Chunk size the fused entry points (sda_decode_attn_step / _batch) use for
 * this geometry (host only), with P = n_inst * ceil(max_sel / chunk_cells)
 * (instance, chunk) pairs:
 *   P <= 256: the call is latency-bound; C is the smallest multiple of
 *     SDA_CHUNK_ALIGN cells that keeps n_inst * ceil(max_sel / C) within 256
 *     (the work spreads over more CUs; the merge combines finer partials);
 *   else n_inst <= 256: m = min(512 / n_inst, ceil(max_sel / chunk_cells))
 *     balanced chunks per instance, C = ceil(max_sel / m) rounded up to a
 *     multiple of SDA_CHUNK_ALIGN (one round of two workgroups per CU, no
 *     short tail chunks);
 *   else P > 512: each workgroup of the chunk pass would run k = min(P / 512,
 *     ceil(max_sel / chunk_cells)) consecutive chunks; C = k * chunk_cells,
 *     so that it leaves one partial instead of k;
 *   otherwise C = chunk_cells.
 *   fused_chunk_cells (host out)
 * Returns SDA_OK, SDA_ERR_INVALID_ARG (negative sizes, null output) or
 * SDA_ERR_UNSUPPORTED (chunk_cells not a multiple of SDA_CHUNK_ALIGN). */
int sda_fused_chunk_cells(int32_t n_inst, int32_t max_sel, int32_t chunk_cells,
                          int32_t *fused_chunk_cells);

/* Whether a fused call (sda_decode_attn_step / _batch) of this geometry runs
 * as a single chunk-kernel launch that merges in place and writes out and
 * lse itself, leaving the workspace untouched (host only).  That is the case
 * when C = sda_fused_chunk_cells(n_inst, max_sel, chunk_cells) exceeds
 * SDA_CHUNK_ALIGN and ceil(max_sel / C) is 1, or 2 with 16 < n_q * n_qheads
 * <= 48 (one workgroup runs both chunks of an instance, one gather pipeline
 * each); otherwise the call launches the chunk pass and the merge pass.
 *   single_launch (host out): 1 or 0
 * Returns SDA_OK, SDA_ERR_INVALID_ARG (negative sizes, n_q or n_qheads below
 * 1, null output) or SDA_ERR_UNSUPPORTED (chunk_cells not a multiple of
 * SDA_CHUNK_ALIGN, or more than SDA_MAX_ROWS rows). */
int sda_fused_single_launch(int32_t n_inst, int32_t n_q, int32_t n_qheads, int32_t max_sel,
                            int32_t chunk_cells, int32_t *single_launch);

/* One sequence (one KV head), the pages' single-step entry point.
 *   pool          host pointer to the pool descriptor
 *   page_table    int32 [n_logical_pages] global physical page ids
 *   sel           int32 [n_sel] selected logical cell ids (may be NULL if n_sel == 0)
 *   n_sel         host, >= 0
 *   q             float [n_q][n_qheads][head_dim], 16-byte aligned
 *   n_q, n_qheads host; 1 <= n_q, 1 <= n_qheads, n_q * n_qheads <= SDA_MAX_ROWS
 *   softmax_scale host, finite
 *   chunk_cells   host, positive multiple of SDA_CHUNK_ALIGN
 *   out           float [n_q][n_qheads][head_dim], 16-byte aligned
 *   lse           float [n_q][n_qheads]
 *   gather_out    nullable int32 [n_sel]: physical cell per entry, -1 if masked
 *   workspace     device buffer of at least sda_workspace_bytes(1, ..., n_sel, ...)
 *                 bytes, 256-byte aligned (may be NULL if that size is 0)
 *   stream        hipStream_t (NULL = default stream)
 */
int sda_decode_attn_step(const sda_pool *pool, const int32_t *page_table,
                         int32_t n_logical_pages, const int32_t *sel, int32_t n_sel,
                         const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                         int32_t chunk_cells, float *out, float *lse, int32_t *gather_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Many independent (sequence, KV head) instances sharing one pool, the
 * pages' batch entry point.
 *   n_inst        host, >= 0 (0: nothing is launched)
 *   page_table    int32 [n_inst][pt_stride]; the first n_logical_pages entries
 *                 of each row are used (pt_stride >= n_logical_pages)
 *   sel           int32 [n_inst][sel_stride] (sel_stride >= max_sel)
 *   n_sel         DEVICE int32 [n_inst]: entries used per instance; read on the
 *                 device so that a captured graph replays with new counts;
 *                 clamped to [0, max_sel]
 *   max_sel       host upper bound of n_sel[i]; sizes the grid and workspace
 *   q             float [n_inst][n_q][n_qheads][head_dim]
 *   out           float [n_inst][n_q][n_qheads][head_dim], 16-byte aligned
 *   lse           float [n_inst][n_q][n_qheads]
 *   gather_out    nullable int32 [n_inst][sel_stride]
 *   other arguments as for sda_decode_attn_step, with the workspace sized by
 *   sda_workspace_bytes(n_inst, n_q, n_qheads, head_dim, max_sel, chunk_cells).
 */
int sda_decode_attn_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                          int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                          int64_t sel_stride, const int32_t *n_sel, int32_t max_sel,
                          const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                          int32_t chunk_cells, float *out, float *lse, int32_t *gather_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* sda_decode_attn_batch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and
 * the same results bit for bit.  The chunk partials go to a device array the
 * library holds instead, SDA_SCRATCH_BYTES per GPU, resident from the
 * library's load until the process ends; the call itself allocates nothing.
 *   - The array used is the current device's (hipGetDevice): the stream and
 *     every pointer must belong to that device.  The first call on a device
 *     resolves the array's address (hipGetSymbolAddress); make that first
 *     call outside stream capture.
 *   - A call whose partials exceed SDA_SCRATCH_BYTES returns SDA_ERR_SCRATCH
 *     without launching: the partials of the fused chunk size,
 *     sda_workspace_bytes at chunk_cells = sda_fused_chunk_cells(n_inst,
 *     max_sel, chunk_cells), or 0 when sda_fused_single_launch says the call
 *     is one launch.
 *   - Every call on a GPU shares that GPU's array and leaves its partials
 *     there.  Nothing in it has to start at zero (each chunk pass writes
 *     every partial its merge reads), but calls that overlap on one GPU
 *     (other streams, other host threads) race on it and give wrong results:
 *     serialise them.
 * Returns the statuses of sda_decode_attn_batch except SDA_ERR_WORKSPACE,
 * plus SDA_ERR_SCRATCH (and SDA_ERR_LAUNCH if the array's address cannot be
 * resolved). */
#define SDA_SCRATCH_BYTES ((size_t)32 << 20)
int sda_decode_attn_batch_noalloc(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                                  int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                                  int64_t sel_stride, const int32_t *n_sel, int32_t max_sel,
                                  const float *q, int32_t n_q, int32_t n_qheads,
                                  float softmax_scale, int32_t chunk_cells, float *out,
                                  float *lse, int32_t *gather_out, void *stream);

/* The two passes of sda_decode_attn_batch, callable on their own.
 *
 * sda_chunk_batch runs only the chunk pass: same arguments and validation as
 * sda_decode_attn_batch without out/lse; it leaves the chunk partials in the
 * workspace (layout under sda_workspace_bytes) for each instance's first
 * ceil(n_sel[i] / chunk_cells) chunks.  Partials from several sources can be
 * combined by any log-sum-exp merge; this is also the unit one would shard
 * across devices for a single very long selection.
 *
 * sda_merge_batch runs only the merge pass over partials laid out as
 * sda_workspace_bytes(n_inst, n_q, n_qheads, SDA_HEAD_DIM, max_sel,
 * chunk_cells) describes: n_sel (device, [n_inst]) gives each instance's
 * chunk count as above; out float [n_inst][n_q][n_qheads][head_dim]
 * (16-byte aligned),
 * lse float [n_inst][n_q][n_qheads].
 *
 * Running sda_chunk_batch then sda_merge_batch on one stream with chunk size
 * sda_fused_chunk_cells(n_inst, max_sel, chunk_cells) gives exactly the
 * result of sda_decode_attn_batch with chunk_cells (and its workspace
 * partials, where that call writes them); with chunk_cells itself the result
 * agrees up to rounding. */
int sda_chunk_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                    int64_t pt_stride, int32_t n_logical_pages, const int32_t *sel,
                    int64_t sel_stride, const int32_t *n_sel, int32_t max_sel, const float *q,
                    int32_t n_q, int32_t n_qheads, float softmax_scale, int32_t chunk_cells,
                    int32_t *gather_out, void *workspace, size_t workspace_bytes, void *stream);

int sda_merge_batch(int32_t n_inst, int32_t n_q, int32_t n_qheads, const int32_t *n_sel,
                    int32_t max_sel, int32_t chunk_cells, const void *workspace,
                    size_t workspace_bytes, float *out, float *lse, void *stream);

/* Prompt (many-query) attention over the same pools: a chunk of n_q
 * consecutive query positions per instance, every position attending
 * causally to the instance's logical cells up to and including its own.
 * Strata PR #2220 page, closing note: the prompt attention's parity test
 * takes the decode kernel as its reference (INT8 32K-cell context, 2,048
 * queries per prompt chunk).  Each (position, query head) row is therefore
 * the decode definition at the top of this header with the selection
 * 0, 1, ..., p, where p = pos0[i] + t is the row's position:
 *
 *   out[i][t][h], lse[i][t][h] = decode result of q[i][t][h] over logical
 *   cells 0..p of instance i (cells at or past 16 * n_logical_pages and cells
 *   on pages with id -1 or outside [0, n_phys_pages) are masked; a row with
 *   no unmasked cell, e.g. p < 0, gets out = 0, lse = -inf).
 *
 *   pool          host pointer to the pool descriptor (as above)
 *   n_inst        host, >= 0 (0: nothing is launched)
 *   page_table    int32 [n_inst][pt_stride], n_logical_pages >= 1 used per row
 *   pos0          DEVICE int32 [n_inst]: position of query 0 of each instance
 *                 (read on the device, so a captured graph replays with new
 *                 positions)
 *   q             float [n_inst][n_q][n_qheads][head_dim], 16-byte aligned
 *   n_q, n_qheads host; >= 1, n_q * n_qheads <= SDA_PROMPT_MAX_ROWS
 *   softmax_scale host, finite
 *   out           float [n_inst][n_q][n_qheads][head_dim], 16-byte aligned
 *   lse           float [n_inst][n_q][n_qheads]
 *   stream        hipStream_t (NULL = default stream)
 * No workspace: one kernel computes each row over its whole causal range.
 * Returns SDA_OK, SDA_ERR_INVALID_ARG, SDA_ERR_UNSUPPORTED or SDA_ERR_LAUNCH. */
int sda_prompt_attn_batch(const sda_pool *pool, int32_t n_inst, const int32_t *page_table,
                          int64_t pt_stride, int32_t n_logical_pages, const int32_t *pos0,
                          const float *q, int32_t n_q, int32_t n_qheads, float softmax_scale,
                          float *out, float *lse, void *stream);

/* The pools as the KV append writes them: the same layout and rules as
 * sda_pool, with writable pointers. */
typedef struct sda_pool_mut {
    int8_t *k_codes;
    uint16_t *k_scales;
    int8_t *v_codes;
    uint16_t *v_scales;
    int64_t n_phys_pages;
    int32_t page_size;    /* must be SDA_PAGE_SIZE */
    int32_t head_dim;     /* must be SDA_HEAD_DIM */
    int32_t scale_stride; /* elements between the scales of consecutive cells, in [1, 64] */
    int32_t reserved;     /* must be 0 */
} sda_pool_mut;

/* KV append: quantise new K and V rows to INT8 and write them into the
 * pools, the step that produces what the attention reads.  The pages fix
 * the stored format (INT8 codes, one binary16 scale per cell for K and one
 * for V; Strata PR #2220 page) and list the KV append after the K/V
 * projection (Strata round-9 page, section "R9-gpu-8: one exact launch for
 * QSA K and V"), not the quantiser.  This one is symmetric per-cell absmax,
 * every step in float32:
 *   amax = max_d |x[d]|;  scale = binary16(min(amax / 127, 65504)), rounded
 *   to nearest even;  code[d] = clamp(rint(x[d] / scale), -127, 127) with
 *   ties to even and correctly rounded division; all codes 0 when the scale
 *   is 0 (amax below about 127 * 2^-25).
 * New row t of instance i goes to logical cell c = pos0[i] + t, i.e.
 * physical cell page_table[i][c / 16] * 16 + c % 16 (the attention's page
 * map).  A row whose cell is outside [0, 16 * n_logical_pages) or on a page
 * with id -1 or outside [0, n_phys_pages) is not written.
 *   pool          host pointer, writable pools (as sda_pool)
 *   n_inst        host, in [0, 65535] (0: nothing is launched)
 *   page_table    int32 [n_inst][pt_stride] (may be NULL if n_logical_pages == 0)
 *   pos0          DEVICE int32 [n_inst]
 *   k_new, v_new  float [n_inst][n_new][head_dim], 16-byte aligned, finite
 *                 (non-finite values give unspecified codes)
 *   n_new         host, >= 0
 *   stream        hipStream_t (NULL = default stream)
 * Two new rows that map to the same physical cell (in one call) race: the
 * cell ends up holding one of them.  Returns SDA_OK, SDA_ERR_INVALID_ARG,
 * SDA_ERR_UNSUPPORTED or SDA_ERR_LAUNCH. */
int sda_kv_append_batch(const sda_pool_mut *pool, int32_t n_inst, const int32_t *page_table,
                        int64_t pt_stride, int32_t n_logical_pages, const int32_t *pos0,
                        const float *k_new, const float *v_new, int32_t n_new, void *stream);

/* QSA block scoring and top-k selection: the step that produces the
 * selected cell list (sel, n_sel) the decode entry points read.  The Strata
 * round-9 page (section "R9-gpu-9: QSA_ROWS at five and six queries") gives
 * the scorer's arguments -- pooled block keys, dead flags, indexer queries,
 * per-row extents, the row count and the block capacity -- and its geometry
 * (indexer head dimension, indexer head count, block size); section
 * "R9-gpu-8" names the top-k.  The arithmetic is this library's reading:
 *
 *   block b of an instance holds logical cells [b * R, (b + 1) * R),
 *   R = block_cells;
 *   scores[i][r][b] = sum over indexer heads h of the dot product of
 *                     q_idx[i][r][h][.] and pooled[i][b][h][.] (fp32), or
 *                     -inf when dead[i][b] != 0 or b * R >= n_visible[i][r];
 *   selection: the k_blocks blocks with the highest combined score
 *              max_r scores[i][r][b] (equal scores in increasing block
 *              order, -inf never), in increasing block order, each giving
 *              its cells below E = max_r n_visible[i][r] (clipped to
 *              max_blocks * R): a sorted cell list.
 *
 * sda_qsa_block_scores:
 *   n_inst        host, in [0, 65535] (0: nothing is launched)
 *   n_rows        host, query rows per instance, 1..SDA_QSA_MAX_ROWS
 *   n_heads, idx_dim  host, >= 1; n_heads * idx_dim a multiple of
 *                 SDA_QSA_HD_ALIGN, at most SDA_QSA_MAX_HD
 *   block_cells   host, a positive multiple of SDA_PAGE_SIZE
 *   max_blocks    host, >= 1, max_blocks * block_cells <= 2^31 - 1
 *   pooled        float [n_inst][max_blocks][n_heads][idx_dim], 16-byte aligned
 *   dead          uint8 [n_inst][max_blocks]
 *   q_idx         float [n_inst][n_rows][n_heads][idx_dim], 16-byte aligned
 *   n_visible     DEVICE int32 [n_inst][n_rows]: cells each row can see
 *   scores        float [n_inst][n_rows][max_blocks] (written)
 *   stream        hipStream_t (NULL = default stream)
 * A block no row can use is not read.  Returns SDA_OK, SDA_ERR_INVALID_ARG,
 * SDA_ERR_UNSUPPORTED or SDA_ERR_LAUNCH. */
#define SDA_QSA_MAX_ROWS 8
#define SDA_QSA_HD_ALIGN 64
#define SDA_QSA_MAX_HD 1024
#define SDA_QSA_MAX_BLOCKS 16384
#define SDA_QSA_MAX_K 4096
int sda_qsa_block_scores(int32_t n_inst, int32_t n_rows, int32_t n_heads, int32_t idx_dim,
                         int32_t block_cells, int32_t max_blocks, const float *pooled,
                         const uint8_t *dead, const float *q_idx, const int32_t *n_visible,
                         float *scores, void *stream);

/* sda_qsa_select: top-k selection and expansion to cells (one workgroup per
 * instance, up to eight per instance when there are fewer than 256
 * instances), from scores laid out as sda_qsa_block_scores writes them (any
 * values: -inf is never selected; other non-finite values are unspecified).
 *   n_inst        host, >= 0 (0: nothing is launched)
 *   n_rows, block_cells, n_visible  as above
 *   max_blocks    host, 1..SDA_QSA_MAX_BLOCKS
 *   k_blocks      host, 0..SDA_QSA_MAX_K
 *   sel           int32 [n_inst][sel_stride]: the first n_sel[i] entries are
 *                 written (increasing logical cell ids); the rest untouched
 *   sel_stride    host, >= k_blocks * block_cells
 *   n_sel         int32 [n_inst] (written): cells selected, at most
 *                 k_blocks * block_cells
 * The outputs are exactly the sel, sel_stride and n_sel arguments of
 * sda_decode_attn_batch (with max_sel = k_blocks * block_cells).  Returns
 * SDA_OK, SDA_ERR_INVALID_ARG, SDA_ERR_UNSUPPORTED or SDA_ERR_LAUNCH. */
int sda_qsa_select(int32_t n_inst, int32_t n_rows, int32_t block_cells, int32_t max_blocks,
                   const float *scores, const int32_t *n_visible, int32_t k_blocks,
                   int32_t *sel, int64_t sel_stride, int32_t *n_sel, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *sda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SDA_H */
