/* Runs every function of the fp64 oracle (oracle/oracle.c) once on small
 * seeded inputs with masked pages, out-of-range ids and edge counts, so that
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer sees every
 * code path; one cross-check makes the run meaningful beyond the
 * sanitizers: the merge of the chunk partials equals the direct attention.
 * Prints "ok" and exits 0 when everything held.  Test infrastructure, built
 * and run by tests/test_oracle_sanitized.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_half_to_double(uint16_t h);
uint16_t oracle_float_to_half(float x);
void oracle_gather(int64_t n_inst, const int32_t *sel, int64_t sel_stride, const int32_t *n_sel,
                   const int32_t *page_table, int64_t pt_stride, int64_t n_logical_pages,
                   int64_t n_phys_pages, int64_t *phys_out);
void oracle_attend(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                   const uint16_t *v_scales, int64_t n_phys_pages, int64_t head_dim,
                   const int32_t *page_table, int64_t pt_stride, int64_t n_logical_pages,
                   const int32_t *sel, int64_t sel_stride, const int32_t *n_sel, const float *q,
                   int64_t n_rows, double sm_scale, const int64_t *inst_ids, int64_t n_ids,
                   double *out, double *lse);
void oracle_kv_append(int8_t *k_codes, uint16_t *k_scales, int8_t *v_codes, uint16_t *v_scales,
                      int64_t scale_stride, int64_t n_phys_pages, int64_t head_dim,
                      const int32_t *page_table, int64_t n_logical_pages, int64_t pos0,
                      const float *k_new, const float *v_new, int64_t n_new);
void oracle_prompt_attend(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                          const uint16_t *v_scales, int64_t n_phys_pages, int64_t head_dim,
                          const int32_t *page_table, int64_t n_logical_pages, int64_t pos0,
                          const float *q, int64_t n_q, int64_t n_qheads, double sm_scale,
                          const int64_t *t_ids, int64_t n_ids, double *out, double *lse);
void oracle_chunk_partials(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                           const uint16_t *v_scales, int64_t n_phys_pages, int64_t head_dim,
                           const int32_t *page_table, int64_t pt_stride, int64_t n_logical_pages,
                           const int32_t *sel, int64_t sel_stride, const int32_t *n_sel,
                           const float *q, int64_t n_rows, double sm_scale, int64_t chunk,
                           int64_t n_chunks, const int64_t *inst_ids, int64_t n_ids, double *acc,
                           double *m, double *l);
void oracle_merge(int64_t n_units, int64_t n_chunks, int64_t head_dim, const double *acc,
                  const double *m, const double *l, double *out, double *lse);
void oracle_qsa_scores(int64_t n_inst, int64_t n_rows, int64_t n_heads, int64_t idx_dim,
                       int64_t max_blocks, int64_t block_cells, const float *pooled,
                       const uint8_t *dead, const float *q_idx, const int32_t *n_visible,
                       double *scores);
void oracle_qsa_select(int64_t n_inst, int64_t n_rows, int64_t max_blocks, int64_t block_cells,
                       const double *scores, const int32_t *n_visible, int64_t k_blocks,
                       int32_t *sel, int64_t sel_stride, int32_t *n_sel);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* splitmix64, upper half */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static float unif(void) { return (float)(rnd() >> 8) / 16777216.f * 2.f - 1.f; }

#define FAIL(...)                       \
    do {                                \
        fprintf(stderr, __VA_ARGS__);   \
        fputc('\n', stderr);            \
        return 1;                       \
    } while (0)

int main(void) {
    enum { PAGES = 8, CELLS = PAGES * 16, D = 64, INST = 3, LP = 6, STRIDE = 80, ROWS = 2 };
    /* binary16 both ways */
    for (uint32_t h = 0; h < 65536; ++h) (void)oracle_half_to_double((uint16_t)h);
    const float fs[] = {0.f, -0.f, 1.f, 65504.f, 65520.f, 6e-8f, 1e-30f, -3.5f, INFINITY, NAN};
    for (size_t k = 0; k < sizeof fs / sizeof fs[0]; ++k) (void)oracle_float_to_half(fs[k]);

    /* pool: codes in [-127, 127], scales the binary16 bits of small values */
    int8_t *kc = malloc(CELLS * D), *vc = malloc(CELLS * D);
    uint16_t *ks = malloc(CELLS * 2), *vs = malloc(CELLS * 2);
    for (int e = 0; e < CELLS * D; ++e) {
        kc[e] = (int8_t)((int)(rnd() % 255) - 127);
        vc[e] = (int8_t)((int)(rnd() % 255) - 127);
    }
    for (int c = 0; c < CELLS; ++c) {
        ks[c] = oracle_float_to_half(0.002f + 0.01f * (unif() + 1.f));
        vs[c] = oracle_float_to_half(0.01f + 0.05f * (unif() + 1.f));
    }
    /* page tables: a permutation with a masked page and one past the pool */
    int32_t pt[INST * LP];
    for (int i = 0; i < INST; ++i)
        for (int p = 0; p < LP; ++p) pt[i * LP + p] = (p + 3 * i) % PAGES;
    pt[0 * LP + 2] = -1;
    pt[1 * LP + 4] = PAGES + 5;
    /* lists: counts 0, 37 and 80 (with ids past the logical range and < 0) */
    int32_t sel[INST * STRIDE], n_sel[INST] = {0, 37, STRIDE};
    for (int i = 0; i < INST; ++i)
        for (int j = 0; j < STRIDE; ++j) sel[i * STRIDE + j] = (int32_t)(rnd() % (LP * 16));
    sel[1 * STRIDE + 5] = LP * 16 + 2;
    sel[2 * STRIDE + 9] = -4;
    float q[INST * ROWS * D];
    for (int e = 0; e < INST * ROWS * D; ++e) q[e] = unif();
    const double sm = 1.0 / 8.0;

    int64_t phys[INST * STRIDE];
    oracle_gather(INST, sel, STRIDE, n_sel, pt, LP, LP, PAGES, phys);

    double out[INST * ROWS * D], lse[INST * ROWS];
    oracle_attend(kc, ks, vc, vs, PAGES, D, pt, LP, LP, sel, STRIDE, n_sel, q, ROWS, sm, NULL,
                  INST, out, lse);

    /* chunk partials at chunk 16 and their merge against the direct result */
    enum { CH = 16, NCH = (STRIDE + CH - 1) / CH };
    double *acc = malloc(sizeof(double) * INST * NCH * ROWS * D);
    double *m = malloc(sizeof(double) * INST * NCH * ROWS), *l = malloc(sizeof(double) * INST * NCH * ROWS);
    oracle_chunk_partials(kc, ks, vc, vs, PAGES, D, pt, LP, LP, sel, STRIDE, n_sel, q, ROWS, sm, CH,
                          NCH, NULL, INST, acc, m, l);
    /* [inst][chunk][row] -> [unit = (inst, row)][chunk] */
    double *acc2 = malloc(sizeof(double) * INST * ROWS * NCH * D);
    double *m2 = malloc(sizeof(double) * INST * ROWS * NCH), *l2 = malloc(sizeof(double) * INST * ROWS * NCH);
    for (int i = 0; i < INST; ++i)
        for (int c = 0; c < NCH; ++c)
            for (int r = 0; r < ROWS; ++r) {
                const int src = (i * NCH + c) * ROWS + r, dst = (i * ROWS + r) * NCH + c;
                m2[dst] = m[src];
                l2[dst] = l[src];
                memcpy(acc2 + (size_t)dst * D, acc + (size_t)src * D, sizeof(double) * D);
            }
    double mout[INST * ROWS * D], mlse[INST * ROWS];
    oracle_merge(INST * ROWS, NCH, D, acc2, m2, l2, mout, mlse);
    for (int u = 0; u < INST * ROWS; ++u) {
        if (isinf(lse[u]) != isinf(mlse[u])) FAIL("unit %d: empty in one path only", u);
        if (!isinf(lse[u]) && fabs(lse[u] - mlse[u]) > 1e-9) FAIL("unit %d: lse %g vs %g", u, lse[u], mlse[u]);
        for (int d = 0; d < D; ++d)
            if (fabs(out[u * D + d] - mout[u * D + d]) > 1e-9) FAIL("unit %d dim %d: out differs", u, d);
    }

    /* KV append into a copy of the pool (interleaved scale pairs), then a
     * prompt attention over it */
    int8_t *kc2 = malloc(CELLS * D), *vc2 = malloc(CELLS * D);
    uint16_t *sc2 = malloc(CELLS * 4);
    memcpy(kc2, kc, CELLS * D);
    memcpy(vc2, vc, CELLS * D);
    for (int c = 0; c < CELLS; ++c) {
        sc2[2 * c] = ks[c];
        sc2[2 * c + 1] = vs[c];
    }
    enum { NEW = 20 };
    float kn[NEW * D], vn[NEW * D];
    for (int e = 0; e < NEW * D; ++e) {
        kn[e] = unif() * 4.f;
        vn[e] = unif() * 300.f;
    }
    oracle_kv_append(kc2, sc2, vc2, sc2 + 1, 2, PAGES, D, pt + 2 * LP, LP, 70, kn, vn, NEW);
    enum { NQ = 3, NH = 2 };
    float qp[NQ * NH * D];
    for (int e = 0; e < NQ * NH * D; ++e) qp[e] = unif();
    /* the prompt oracle reads one scale array per pool: split the pairs */
    uint16_t *ks2 = malloc(CELLS * 2), *vs2 = malloc(CELLS * 2);
    for (int c = 0; c < CELLS; ++c) {
        ks2[c] = sc2[2 * c];
        vs2[c] = sc2[2 * c + 1];
    }
    int64_t tids[NQ] = {0, 1, 2};
    double pout[NQ * NH * D], plse[NQ * NH];
    oracle_prompt_attend(kc2, ks2, vc2, vs2, PAGES, D, pt + 2 * LP, LP, 60, qp, NQ, NH, sm, tids, NQ,
                         pout, plse);
    for (int e = 0; e < NQ * NH * D; ++e)
        if (!isfinite(pout[e])) FAIL("prompt output %d not finite", e);

    /* QSA: scores of 2 rows over 12 blocks of 8 cells (a dead block, a row
     * seeing only part), then the top 5 */
    enum { QI = 2, QR = 2, QH = 2, QD = 32, QB = 12, QBC = 8, QK = 5 };
    float pooled[QI * QB * QH * QD], qi[QI * QR * QH * QD];
    for (int e = 0; e < QI * QB * QH * QD; ++e) pooled[e] = unif();
    for (int e = 0; e < QI * QR * QH * QD; ++e) qi[e] = unif();
    uint8_t dead[QI * QB] = {0};
    dead[3] = 1;
    int32_t nvis[QI * QR] = {QB * QBC, 41, 0, 17};
    double scores[QI * QR * QB];
    oracle_qsa_scores(QI, QR, QH, QD, QB, QBC, pooled, dead, qi, nvis, scores);
    int32_t qsel[QI * QB * QBC], qn[QI];
    oracle_qsa_select(QI, QR, QB, QBC, scores, nvis, QK, qsel, QB * QBC, qn);
    if (qn[0] != QK * QBC) FAIL("qsa: instance 0 selected %d cells", qn[0]);
    for (int j = 1; j < qn[0]; ++j)
        if (qsel[j] <= qsel[j - 1]) FAIL("qsa: list not increasing at %d", j);

    free(kc); free(vc); free(ks); free(vs); free(acc); free(m); free(l); free(acc2); free(m2);
    free(l2); free(kc2); free(vc2); free(sc2); free(ks2); free(vs2);
    printf("ok\n");
    return 0;
}
