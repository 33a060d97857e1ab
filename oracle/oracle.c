/*
 * CPU oracle for decode-time attention over a selected subset of KV cells
 * held as INT8 K/V pools behind a page table.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the tests, the package's smoke check and the bench's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * Everything is plain C with fp64 arithmetic, written as the definition of
 * the result rather than as a fast algorithm.  OpenMP only distributes
 * independent (instance, query row) pairs over host threads; it does not
 * change any arithmetic.
 *
 * Source: Strata PR #2220 page (the decode attention over the QSA selection,
 * "attn_chunk_q8_v3_kernel"): each selected cell is scored against the
 * grouped query heads sharing its KV head, a softmax runs over the selected
 * cells, the INT8 V rows are accumulated into per-chunk partials, and a merge
 * combines the partials into the head output.  The Strata round-9 page
 * (section "R9-gpu-11: four score cells per step in daily INT8 attention",
 * its "Tests and rejection" paragraph) names the partials (accumulators,
 * maxima, denominators), page -1 masking and the 0/1/2/3/63/64/65-cell edge
 * counts.  Readings where the pages are silent:
 *   - one IEEE binary16 scale per physical cell for K and one for V; the
 *     dequantised value is code * scale;
 *   - score = softmax_scale * k_scale * sum_d q[d] * k_code[d];
 *   - page = 16 cells: logical cell c lives at slot c % 16 of logical page
 *     c / 16; physical cell = page_table[c / 16] * 16 + c % 16;
 *   - a page id of -1 (or any id outside [0, n_phys_pages)) masks the cell,
 *     and so does a selected id outside the instance's logical range;
 *   - every query position attends to the whole selection of its instance
 *     (no causal mask between verify positions);
 *   - with no unmasked cell the output is 0 and the log-sum-exp is -inf;
 *   - partial of a chunk (a run of `chunk` consecutive list positions):
 *     m = max score, l = sum exp(score - m), acc = sum exp(score - m) * v_hat;
 *     an all-masked chunk has m = -inf, l = 0, acc = 0;
 *   - merge: M = max m_c, L = sum l_c e^(m_c - M),
 *     out = sum acc_c e^(m_c - M) / L, lse = M + ln L (natural log).
 *
 * Parity pins (tests/test_oracle.py): binary16 decode against numpy on all
 * 65,536 bit patterns; dense result against a textbook softmax-attention
 * built with numpy/scipy on tiny inputs; closed forms (one cell, two cells,
 * identical keys, zero query); invariants (selection order, chunking for
 * several chunk sizes, uniform score shift realised through the inputs,
 * physical page relabelling, masking equals deletion, exact doubling of V
 * scales); brute force over subsets of a tiny pool.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PAGE 16

/* Host threads the parallel loops below may use. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits; exponent 0 encodes
 * subnormals f * 2^-24, exponent 31 encodes inf/nan. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Page-table gather for one selected logical cell.  Returns the physical cell
 * index or -1 when the cell is masked. */
static int64_t gather_one(int32_t c, const int32_t *pt, int64_t n_logical_pages,
                          int64_t n_phys_pages) {
    if (c < 0) return -1;
    int64_t lp = (int64_t)c / ORACLE_PAGE;
    int64_t slot = (int64_t)c % ORACLE_PAGE;
    if (lp >= n_logical_pages) return -1;
    int64_t pp = pt[lp];
    if (pp < 0 || pp >= n_phys_pages) return -1;
    return pp * ORACLE_PAGE + slot;
}

/* Gather for every instance: phys_out[i][j] for j < n_sel[i]; entries from
 * n_sel[i] to sel_stride-1 are left untouched. */
void oracle_gather(int64_t n_inst, const int32_t *sel, int64_t sel_stride,
                   const int32_t *n_sel, const int32_t *page_table, int64_t pt_stride,
                   int64_t n_logical_pages, int64_t n_phys_pages, int64_t *phys_out) {
    for (int64_t i = 0; i < n_inst; ++i)
        for (int64_t j = 0; j < n_sel[i]; ++j)
            phys_out[i * sel_stride + j] =
                gather_one(sel[i * sel_stride + j], page_table + i * pt_stride,
                           n_logical_pages, n_phys_pages);
}

typedef struct {
    const int8_t *k_codes, *v_codes;     /* [cells][head_dim] */
    const uint16_t *k_scales, *v_scales; /* [cells] binary16 bits */
    int64_t n_phys_pages;
    int64_t head_dim;
} pool_t;

/* score of one query row against one physical cell */
static double score(const pool_t *P, const float *qrow, int64_t phys, double sm_scale) {
    const int8_t *k = P->k_codes + phys * P->head_dim;
    double dot = 0.0;
    for (int64_t d = 0; d < P->head_dim; ++d) dot += (double)qrow[d] * (double)k[d];
    return sm_scale * oracle_half_to_double(P->k_scales[phys]) * dot;
}

/* Softmax attention of one query row over list positions [j0, j1) of one
 * instance's selection.  Writes the unnormalised accumulator acc[d]
 * (= sum_j e^(s_j - m) v_hat_j[d]), the maximum m and the denominator l.
 * No unmasked cell: m = -inf, l = 0, acc = 0. */
static void attend_range(const pool_t *P, const float *qrow, const int32_t *sel,
                         int64_t j0, int64_t j1, const int32_t *pt,
                         int64_t n_logical_pages, double sm_scale, double *acc,
                         double *m_out, double *l_out) {
    const int64_t D = P->head_dim;
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        int64_t ph = gather_one(sel[j], pt, n_logical_pages, P->n_phys_pages);
        if (ph < 0) continue;
        double s = score(P, qrow, ph, sm_scale);
        if (s > m) m = s;
    }
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    double l = 0.0;
    if (m != -INFINITY) {
        for (int64_t j = j0; j < j1; ++j) {
            int64_t ph = gather_one(sel[j], pt, n_logical_pages, P->n_phys_pages);
            if (ph < 0) continue;
            double p = exp(score(P, qrow, ph, sm_scale) - m);
            double w = p * oracle_half_to_double(P->v_scales[ph]);
            const int8_t *v = P->v_codes + ph * D;
            l += p;
            for (int64_t d = 0; d < D; ++d) acc[d] += w * (double)v[d];
        }
    }
    *m_out = m;
    *l_out = l;
}

/* Dense result: out[i][r][d] and lse[i][r] for every instance i in
 * `inst_ids` (n_ids of them; NULL means 0..n_inst-1) and every query row
 * r = t * n_qheads + h.  out/lse are indexed by position in the id list.
 * q is float32 [n_inst][n_rows][head_dim]; sel is [n_inst][sel_stride];
 * page_table is [n_inst][pt_stride]. */
void oracle_attend(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                   const uint16_t *v_scales, int64_t n_phys_pages, int64_t head_dim,
                   const int32_t *page_table, int64_t pt_stride, int64_t n_logical_pages,
                   const int32_t *sel, int64_t sel_stride, const int32_t *n_sel,
                   const float *q, int64_t n_rows, double sm_scale, const int64_t *inst_ids,
                   int64_t n_ids, double *out, double *lse) {
    pool_t P = {k_codes, v_codes, k_scales, v_scales, n_phys_pages, head_dim};
    const int64_t D = head_dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_ids * n_rows; ++u) {
        int64_t k = u / n_rows, r = u % n_rows;
        int64_t i = inst_ids ? inst_ids[k] : k;
        double m, l;
        double *o = out + (k * n_rows + r) * D;
        attend_range(&P, q + (i * n_rows + r) * D, sel + i * sel_stride, 0, n_sel[i],
                     page_table + i * pt_stride, n_logical_pages, sm_scale, o, &m, &l);
        if (m == -INFINITY) {
            lse[k * n_rows + r] = -INFINITY; /* o already zero */
        } else {
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
            lse[k * n_rows + r] = m + log(l);
        }
    }
}

/* IEEE binary16 bit pattern of a finite or infinite float, rounded to
 * nearest with ties to even, written out from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; magnitudes below
 * 2^-14 are subnormal multiples of 2^-24; 65520 and above round to
 * infinity.  NaN gives the quiet NaN 0x7e00. */
uint16_t oracle_float_to_half(float x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        double q = rint(ldexp(a, 24)); /* units of 2^-24; 1024 is the smallest normal */
        return sign | (uint16_t)q;
    }
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                  /* a = (2m) * 2^e, 2m in [1, 2) */
    double q = rint((2.0 * m - 1.0) * 1024.0);
    if (q == 1024.0) {
        q = 0.0;
        e += 1;
    }
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)q;
}

/* INT8 quantisation of one new K or V row (the KV append step).  The pages
 * fix only the stored format: int8 codes with one binary16 scale per cell,
 * value = code * scale.  Reading (symmetric per-cell absmax), every step in
 * float32 as a GPU computes it, so that both sides take each integer
 * decision in the same precision:
 *   amax  = max_d |x[d]|
 *   s16   = binary16(min(amax / 127, 65504))   (round to nearest even; the
 *           scale saturates at the largest finite binary16)
 *   s     = the value of s16
 *   code  = clamp(rint(x[d] / s), -127, 127)   (ties to even; all 0 if s = 0)
 * Writes head_dim codes and the scale. */
static void quantise_row(const float *x, int64_t head_dim, int8_t *codes, uint16_t *scale) {
    float amax = 0.0f;
    for (int64_t d = 0; d < head_dim; ++d) {
        float v = fabsf(x[d]);
        if (v > amax) amax = v;
    }
    float s32 = amax / 127.0f;
    if (s32 > 65504.0f) s32 = 65504.0f;
    uint16_t s16 = oracle_float_to_half(s32);
    float s = (float)oracle_half_to_double(s16);
    for (int64_t d = 0; d < head_dim; ++d) {
        float q = 0.0f;
        if (s > 0.0f) {
            q = rintf(x[d] / s);
            if (q > 127.0f) q = 127.0f;
            if (q < -127.0f) q = -127.0f;
        }
        codes[d] = (int8_t)q;
    }
    *scale = s16;
}

/* KV append for one instance: new rows t < n_new go to logical cell
 * c = pos0 + t, i.e. physical cell page_table[c / 16] * 16 + c % 16 (the
 * decode gather's page map); a row whose cell is outside the table or on a
 * masked page (-1 or outside the pool) is not written.  K and V scales of
 * physical cell ph are k_scales[ph * scale_stride], v_scales[ph * scale_stride].
 * k_new, v_new: float32 [n_new][head_dim]. */
void oracle_kv_append(int8_t *k_codes, uint16_t *k_scales, int8_t *v_codes, uint16_t *v_scales,
                      int64_t scale_stride, int64_t n_phys_pages, int64_t head_dim,
                      const int32_t *page_table, int64_t n_logical_pages, int64_t pos0,
                      const float *k_new, const float *v_new, int64_t n_new) {
    for (int64_t t = 0; t < n_new; ++t) {
        int64_t c = pos0 + t;
        if (c < 0 || c > INT32_MAX) continue;
        int64_t ph = gather_one((int32_t)c, page_table, n_logical_pages, n_phys_pages);
        if (ph < 0) continue;
        quantise_row(k_new + t * head_dim, head_dim, k_codes + ph * head_dim,
                     k_scales + ph * scale_stride);
        quantise_row(v_new + t * head_dim, head_dim, v_codes + ph * head_dim,
                     v_scales + ph * scale_stride);
    }
}

/* Prompt (many-query) attention.  Strata PR #2220 page, closing note: the
 * prompt attention's parity test takes the decode kernel as its reference.
 * Reading: query position t of an instance sits at position p = pos0 + t
 * and attends to the instance's logical cells 0, 1, ..., p (its own cell
 * included), i.e. row (t, h) is the decode result above with the selection
 * list 0..p; ids past the page table and masked pages drop out exactly as
 * in the decode definition, and p < 0 leaves nothing (out = 0, lse = -inf).
 * For one instance: page_table [n_logical_pages], q float32
 * [n_q][n_qheads][head_dim]; the positions t listed in t_ids (n_ids of
 * them) and every head h give out[k][h][head_dim] and lse[k][h]. */
void oracle_prompt_attend(const int8_t *k_codes, const uint16_t *k_scales,
                          const int8_t *v_codes, const uint16_t *v_scales,
                          int64_t n_phys_pages, int64_t head_dim, const int32_t *page_table,
                          int64_t n_logical_pages, int64_t pos0, const float *q, int64_t n_q,
                          int64_t n_qheads, double sm_scale, const int64_t *t_ids,
                          int64_t n_ids, double *out, double *lse) {
    pool_t P = {k_codes, v_codes, k_scales, v_scales, n_phys_pages, head_dim};
    const int64_t D = head_dim;
    (void)n_q; /* q rows are indexed by the listed positions */
    /* the selection list 0, 1, ..., p of the latest listed position */
    int64_t p_max = -1;
    for (int64_t k = 0; k < n_ids; ++k)
        if (pos0 + t_ids[k] > p_max) p_max = pos0 + t_ids[k];
    int32_t *list = malloc((size_t)(p_max + 1 > 0 ? p_max + 1 : 1) * sizeof(int32_t));
    for (int64_t j = 0; j <= p_max; ++j) list[j] = (int32_t)j;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_ids * n_qheads; ++u) {
        int64_t k = u / n_qheads, h = u % n_qheads;
        int64_t t = t_ids[k];
        int64_t p = pos0 + t;
        int64_t n_visible = p + 1 > 0 ? p + 1 : 0;
        double m, l;
        double *o = out + u * D;
        attend_range(&P, q + (t * n_qheads + h) * D, list, 0, n_visible, page_table,
                     n_logical_pages, sm_scale, o, &m, &l);
        if (m == -INFINITY) {
            lse[u] = -INFINITY; /* o already zero */
        } else {
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
            lse[u] = m + log(l);
        }
    }
    free(list);
}

/* Chunk partials: for each listed instance, chunk c (list positions
 * [c*chunk, min((c+1)*chunk, n_sel))) and row r: acc[k][c][r][D], m, l
 * ([k][c][r]).  Chunks past the instance's last (c >= ceil(n_sel/chunk)) are
 * written as empty partials. */
void oracle_chunk_partials(const int8_t *k_codes, const uint16_t *k_scales,
                           const int8_t *v_codes, const uint16_t *v_scales,
                           int64_t n_phys_pages, int64_t head_dim, const int32_t *page_table,
                           int64_t pt_stride, int64_t n_logical_pages, const int32_t *sel,
                           int64_t sel_stride, const int32_t *n_sel, const float *q,
                           int64_t n_rows, double sm_scale, int64_t chunk, int64_t n_chunks,
                           const int64_t *inst_ids, int64_t n_ids, double *acc, double *m,
                           double *l) {
    pool_t P = {k_codes, v_codes, k_scales, v_scales, n_phys_pages, head_dim};
    const int64_t D = head_dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_ids * n_chunks * n_rows; ++u) {
        int64_t k = u / (n_chunks * n_rows);
        int64_t c = (u / n_rows) % n_chunks;
        int64_t r = u % n_rows;
        int64_t i = inst_ids ? inst_ids[k] : k;
        int64_t j0 = c * chunk, j1 = j0 + chunk;
        if (j1 > n_sel[i]) j1 = n_sel[i];
        if (j0 > j1) j0 = j1;
        int64_t o = (k * n_chunks + c) * n_rows + r;
        attend_range(&P, q + (i * n_rows + r) * D, sel + i * sel_stride, j0, j1,
                     page_table + i * pt_stride, n_logical_pages, sm_scale, acc + o * D,
                     m + o, l + o);
    }
}

/* Log-sum-exp merge of n_chunks partials for each of n_units (instance,row)
 * units: acc [u][c][D] as laid out by the caller through strides, m and l
 * [u][c].  out [u][D], lse [u].  All-empty: out = 0, lse = -inf. */
void oracle_merge(int64_t n_units, int64_t n_chunks, int64_t head_dim, const double *acc,
                  const double *m, const double *l, double *out, double *lse) {
    const int64_t D = head_dim;
    for (int64_t u = 0; u < n_units; ++u) {
        double M = -INFINITY;
        for (int64_t c = 0; c < n_chunks; ++c)
            if (m[u * n_chunks + c] > M) M = m[u * n_chunks + c];
        double *o = out + u * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            lse[u] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int64_t c = 0; c < n_chunks; ++c) {
            double mc = m[u * n_chunks + c];
            if (mc == -INFINITY) continue; /* empty chunk: contributes nothing */
            double w = exp(mc - M);
            L += l[u * n_chunks + c] * w;
            const double *a = acc + (u * n_chunks + c) * D;
            for (int64_t d = 0; d < D; ++d) o[d] += a[d] * w;
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= L;
        lse[u] = M + log(L);
    }
}

/* ------------------------------------------------------------------------
 * QSA block scorer and top-k selection (the step that produces the selected
 * cell list the attention above reads).
 *
 * Source: Strata round-9 page, section "R9-gpu-9: QSA_ROWS at five and six
 * queries": a block scorer for a few query rows takes pooled block keys,
 * per-block dead flags, indexer queries, per-row extents ("steps"), the row
 * count and the block capacity, and writes block scores; its geometry is an
 * indexer head dimension, an indexer head count and a block size, and its
 * tests compare the full scores and the selected ids (equal keys, dead-tail
 * transitions, partial blocks, several live extents under one capacity).
 * Section "R9-gpu-8" names the top-k that turns the scores into the
 * selection.  The pages fix no arithmetic; the readings taken here:
 *   - block b holds logical cells [b * R, (b + 1) * R) (R = block_cells);
 *   - score of query row r for block b: the sum over indexer heads h of the
 *     dot product of the row's indexer query q[r][h][.] with the block's
 *     pooled key pooled[b][h][.]; -inf when the block is dead or when its
 *     first cell is not visible to the row (b * R >= n_visible[r]);
 *   - selection: each block's combined score is its maximum over the rows
 *     (a block any verify position asks for); the k blocks with the highest
 *     combined scores are taken, equal scores in increasing block order,
 *     blocks at -inf never; the selected blocks, in increasing order, give
 *     their cells below the instance's extent E = max_r n_visible[r]
 *     (clipped to the capacity), so the list is sorted and a block at the
 *     end of the context contributes only its visible cells.
 * ------------------------------------------------------------------------ */

/* scores [n_inst][n_rows][max_blocks] (fp64) from pooled fp32
 * [n_inst][max_blocks][n_heads][idx_dim], dead uint8 [n_inst][max_blocks]
 * (non-zero: dead), q_idx fp32 [n_inst][n_rows][n_heads][idx_dim] and
 * n_visible int32 [n_inst][n_rows]. */
void oracle_qsa_scores(int64_t n_inst, int64_t n_rows, int64_t n_heads, int64_t idx_dim,
                       int64_t max_blocks, int64_t block_cells, const float *pooled,
                       const uint8_t *dead, const float *q_idx, const int32_t *n_visible,
                       double *scores) {
    const int64_t hd = n_heads * idx_dim;
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < n_inst * n_rows; ++u) {
        const int64_t i = u / n_rows; /* row u % n_rows of instance i */
        const float *q = q_idx + u * hd;
        for (int64_t b = 0; b < max_blocks; ++b) {
            double s = -INFINITY;
            if (!dead[i * max_blocks + b] && b * block_cells < (int64_t)n_visible[u]) {
                const float *k = pooled + (i * max_blocks + b) * hd;
                s = 0.0;
                for (int64_t h = 0; h < n_heads; ++h) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < idx_dim; ++d)
                        dot += (double)q[h * idx_dim + d] * (double)k[h * idx_dim + d];
                    s += dot;
                }
            }
            scores[u * max_blocks + b] = s;
        }
    }
}

/* ranking of the blocks by combined score, for qsort: higher first, equal
 * scores in increasing block order */
typedef struct {
    double c;
    int64_t b;
} ranked_t;

static int rank_cmp(const void *x, const void *y) {
    const ranked_t *a = x, *b = y;
    if (a->c > b->c) return -1;
    if (a->c < b->c) return 1;
    return (a->b > b->b) - (a->b < b->b);
}

/* Top-k selection from scores [n_inst][n_rows][max_blocks] (any values; the
 * tests pass the kernel's own fp32 scores as well as the oracle's): writes
 * the selected cells to sel [n_inst][sel_stride] and their count to
 * n_sel [n_inst]. */
void oracle_qsa_select(int64_t n_inst, int64_t n_rows, int64_t max_blocks, int64_t block_cells,
                       const double *scores, const int32_t *n_visible, int64_t k_blocks,
                       int32_t *sel, int64_t sel_stride, int32_t *n_sel) {
    ranked_t *rk = malloc((size_t)(max_blocks > 0 ? max_blocks : 1) * sizeof *rk);
    int64_t *take = malloc((size_t)(max_blocks > 0 ? max_blocks : 1) * sizeof *take);
    for (int64_t i = 0; i < n_inst; ++i) {
        int64_t extent = 0;
        for (int64_t r = 0; r < n_rows; ++r)
            if ((int64_t)n_visible[i * n_rows + r] > extent) extent = n_visible[i * n_rows + r];
        if (extent > max_blocks * block_cells) extent = max_blocks * block_cells;
        for (int64_t b = 0; b < max_blocks; ++b) {
            double c = -INFINITY;
            for (int64_t r = 0; r < n_rows; ++r) {
                double s = scores[(i * n_rows + r) * max_blocks + b];
                if (s > c) c = s;
            }
            rk[b].c = c;
            rk[b].b = b;
            take[b] = 0;
        }
        qsort(rk, (size_t)max_blocks, sizeof *rk, rank_cmp);
        for (int64_t j = 0; j < k_blocks && j < max_blocks && rk[j].c > -INFINITY; ++j)
            take[rk[j].b] = 1;
        int64_t n = 0;
        for (int64_t b = 0; b < max_blocks; ++b) {
            if (!take[b]) continue;
            for (int64_t c = b * block_cells; c < (b + 1) * block_cells && c < extent; ++c) {
                if (n < sel_stride) sel[i * sel_stride + n] = (int32_t)c; /* never past the row */
                ++n;
            }
        }
        n_sel[i] = (int32_t)n;
    }
    free(rk);
    free(take);
}
