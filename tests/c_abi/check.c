/*
 * A plain C consumer of libsda.so: no Python, no torch.  It allocates device
 * memory with the HIP runtime, calls the C entry points declared in
 * include/sda.h, and checks the results against the CPU oracle (fp64,
 * oracle/oracle.c), which is linked in as test infrastructure.
 *
 * Checks (one JSON line on stdout; exit status 0 only if all pass):
 *   - sda_decode_attn_batch on three instances (device counts 700, 437 and
 *     0; masked pages on one instance) against oracle_attend: out within
 *     1e-3 + 1e-3 |ref|, lse within 1e-4 + 1e-4 |ref|, -inf lse and zero
 *     output for the empty instance; gather indices equal oracle_gather;
 *   - sda_decode_attn_step on instance 0 equals the batch call bit for bit;
 *   - sda_chunk_batch + sda_merge_batch at sda_fused_chunk_cells(...) equal
 *     the batch call bit for bit;
 *   - a chunk size that is not a multiple of SDA_CHUNK_ALIGN is rejected with
 *     SDA_ERR_UNSUPPORTED before any launch, and sda_status_string names it.
 *
 * Inputs come from splitmix64 (seeded); they have the shapes of the decode
 * workloads (12 query heads, head_dim 256, 16-cell pages behind a permuted
 * page table) and carry none of the method's arithmetic.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sda.h"

/* from oracle/oracle.c (liboracle.so) */
void oracle_attend(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                   const uint16_t *v_scales, int64_t n_phys_pages, int64_t head_dim,
                   const int32_t *page_table, int64_t pt_stride, int64_t n_logical_pages,
                   const int32_t *sel, int64_t sel_stride, const int32_t *n_sel,
                   const float *q, int64_t n_rows, double sm_scale, const int64_t *inst_ids,
                   int64_t n_ids, double *out, double *lse);
void oracle_gather(int64_t n_inst, const int32_t *sel, int64_t sel_stride,
                   const int32_t *n_sel, const int32_t *page_table, int64_t pt_stride,
                   int64_t n_logical_pages, int64_t n_phys_pages, int64_t *phys_out);

enum { N_INST = 3, PAGES = 64, CELLS = PAGES * 16, MAX_SEL = 700, N_Q = 2, N_H = 12,
       ROWS = N_Q * N_H, D = 256, CHUNK = 256 };

static uint64_t rng_state = 0x5DA1C0DEULL;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static int64_t uniform_int(int64_t lo, int64_t hi) { /* [lo, hi] */
    return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}
static void shuffle(int32_t *a, int64_t n) {
    for (int64_t i = n - 1; i > 0; --i) {
        int64_t j = uniform_int(0, i);
        int32_t t = a[i];
        a[i] = a[j];
        a[j] = t;
    }
}
static int cmp_i32(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

#define HIP_OK(x)                                                                 \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

static void *dev_copy(const void *h, size_t n) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n ? n : 1));
    if (n) HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static int failures = 0;
static void fail(const char *what) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
}

int main(void) {
    const int64_t total = (int64_t)N_INST * CELLS;
    int8_t *kc = malloc(total * D), *vc = malloc(total * D);
    uint16_t *ks = malloc(total * 2), *vs = malloc(total * 2);
    int32_t *pt = malloc(sizeof(int32_t) * N_INST * PAGES);
    int32_t *sel = malloc(sizeof(int32_t) * N_INST * MAX_SEL);
    int32_t n_sel[N_INST] = {MAX_SEL, 437, 0};
    float *q = malloc(sizeof(float) * N_INST * ROWS * D);
    for (int64_t e = 0; e < total * D; ++e) {
        kc[e] = (int8_t)uniform_int(-127, 127);
        vc[e] = (int8_t)uniform_int(-127, 127);
    }
    /* binary16 bit patterns between about 0.002 (0x1819) and 0.02 (0x251f) */
    for (int64_t c = 0; c < total; ++c) {
        ks[c] = (uint16_t)uniform_int(0x1819, 0x251f);
        vs[c] = (uint16_t)uniform_int(0x1819, 0x251f);
    }
    for (int i = 0; i < N_INST; ++i) {
        for (int p = 0; p < PAGES; ++p) pt[i * PAGES + p] = i * PAGES + p;
        shuffle(pt + i * PAGES, PAGES);
        int32_t cells[CELLS];
        for (int c = 0; c < CELLS; ++c) cells[c] = c;
        shuffle(cells, CELLS);
        qsort(cells, MAX_SEL, sizeof(int32_t), cmp_i32);
        memcpy(sel + i * MAX_SEL, cells, sizeof(int32_t) * MAX_SEL);
    }
    pt[1 * PAGES + 3] = -1; /* masked pages of instance 1 */
    pt[1 * PAGES + 40] = -1;
    for (int64_t e = 0; e < (int64_t)N_INST * ROWS * D; ++e)
        q[e] = (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 3.0 - 1.5);
    const float sm = 1.0f / 16.0f;

    int8_t *d_kc = dev_copy(kc, total * D), *d_vc = dev_copy(vc, total * D);
    uint16_t *d_ks = dev_copy(ks, total * 2), *d_vs = dev_copy(vs, total * 2);
    int32_t *d_pt = dev_copy(pt, sizeof(int32_t) * N_INST * PAGES);
    int32_t *d_sel = dev_copy(sel, sizeof(int32_t) * N_INST * MAX_SEL);
    int32_t *d_nsel = dev_copy(n_sel, sizeof n_sel);
    float *d_q = dev_copy(q, sizeof(float) * N_INST * ROWS * D);
    const size_t out_n = (size_t)N_INST * ROWS * D, lse_n = (size_t)N_INST * ROWS;
    float *d_out, *d_lse, *d_out2, *d_lse2, *d_out1, *d_lse1;
    int32_t *d_g, *d_g1;
    HIP_OK(hipMalloc((void **)&d_out, out_n * 4));
    HIP_OK(hipMalloc((void **)&d_lse, lse_n * 4));
    HIP_OK(hipMalloc((void **)&d_out2, out_n * 4));
    HIP_OK(hipMalloc((void **)&d_lse2, lse_n * 4));
    HIP_OK(hipMalloc((void **)&d_out1, (size_t)ROWS * D * 4));
    HIP_OK(hipMalloc((void **)&d_lse1, (size_t)ROWS * 4));
    HIP_OK(hipMalloc((void **)&d_g, sizeof(int32_t) * N_INST * MAX_SEL));
    HIP_OK(hipMalloc((void **)&d_g1, sizeof(int32_t) * MAX_SEL));

    sda_pool pool;
    memset(&pool, 0, sizeof pool);
    pool.k_codes = d_kc;
    pool.k_scales = d_ks;
    pool.v_codes = d_vc;
    pool.v_scales = d_vs;
    pool.n_phys_pages = N_INST * PAGES;
    pool.page_size = SDA_PAGE_SIZE;
    pool.head_dim = SDA_HEAD_DIM;
    pool.scale_stride = 1;

    size_t ws_bytes = 0;
    int st = sda_workspace_bytes(N_INST, N_Q, N_H, D, MAX_SEL, CHUNK, &ws_bytes);
    if (st != SDA_OK) fail("sda_workspace_bytes");
    void *d_ws = NULL;
    HIP_OK(hipMalloc(&d_ws, ws_bytes));

    /* the batch entry point */
    st = sda_decode_attn_batch(&pool, N_INST, d_pt, PAGES, PAGES, d_sel, MAX_SEL, d_nsel, MAX_SEL,
                               d_q, N_Q, N_H, sm, CHUNK, d_out, d_lse, d_g, d_ws, ws_bytes, NULL);
    if (st != SDA_OK) fail("sda_decode_attn_batch status");
    /* the step entry point on instance 0 */
    size_t ws1_bytes = 0;
    if (sda_workspace_bytes(1, N_Q, N_H, D, MAX_SEL, CHUNK, &ws1_bytes) != SDA_OK)
        fail("sda_workspace_bytes (step)");
    st = sda_decode_attn_step(&pool, d_pt, PAGES, d_sel, n_sel[0], d_q, N_Q, N_H, sm, CHUNK,
                              d_out1, d_lse1, d_g1, d_ws, ws_bytes, NULL);
    if (st != SDA_OK) fail("sda_decode_attn_step status");
    /* the two passes at the fused call's chunk size */
    int32_t fc = 0;
    if (sda_fused_chunk_cells(N_INST, MAX_SEL, CHUNK, &fc) != SDA_OK) fail("sda_fused_chunk_cells");
    void *d_ws2 = NULL;
    HIP_OK(hipMalloc(&d_ws2, ws_bytes));
    st = sda_chunk_batch(&pool, N_INST, d_pt, PAGES, PAGES, d_sel, MAX_SEL, d_nsel, MAX_SEL, d_q,
                         N_Q, N_H, sm, fc, NULL, d_ws2, ws_bytes, NULL);
    if (st != SDA_OK) fail("sda_chunk_batch status");
    st = sda_merge_batch(N_INST, N_Q, N_H, d_nsel, MAX_SEL, fc, d_ws2, ws_bytes, d_out2, d_lse2,
                         NULL);
    if (st != SDA_OK) fail("sda_merge_batch status");
    /* rejected before any launch */
    st = sda_decode_attn_step(&pool, d_pt, PAGES, d_sel, n_sel[0], d_q, N_Q, N_H, sm, 100,
                              d_out1, d_lse1, NULL, d_ws, ws_bytes, NULL);
    if (st != SDA_ERR_UNSUPPORTED) fail("chunk 100 not rejected as unsupported");
    const char *name = sda_status_string(st);
    if (!name || !*name) fail("sda_status_string");
    HIP_OK(hipDeviceSynchronize());

    float *out = malloc(out_n * 4), *lse = malloc(lse_n * 4), *out2 = malloc(out_n * 4);
    float *lse2 = malloc(lse_n * 4), *out1 = malloc((size_t)ROWS * D * 4), *lse1 = malloc(ROWS * 4);
    int32_t *g = malloc(sizeof(int32_t) * N_INST * MAX_SEL), *g1 = malloc(sizeof(int32_t) * MAX_SEL);
    HIP_OK(hipMemcpy(out, d_out, out_n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, d_lse, lse_n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out2, d_out2, out_n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse2, d_lse2, lse_n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out1, d_out1, (size_t)ROWS * D * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse1, d_lse1, ROWS * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g, d_g, sizeof(int32_t) * N_INST * MAX_SEL, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g1, d_g1, sizeof(int32_t) * MAX_SEL, hipMemcpyDeviceToHost));

    /* the oracle */
    double *ref = malloc(out_n * 8), *ref_lse = malloc(lse_n * 8);
    int64_t *ref_g = malloc(sizeof(int64_t) * N_INST * MAX_SEL);
    oracle_attend(kc, ks, vc, vs, N_INST * PAGES, D, pt, PAGES, PAGES, sel, MAX_SEL, n_sel, q,
                  ROWS, sm, NULL, N_INST, ref, ref_lse);
    oracle_gather(N_INST, sel, MAX_SEL, n_sel, pt, PAGES, PAGES, N_INST * PAGES, ref_g);

    double max_dout = 0.0, max_dlse = 0.0;
    for (size_t e = 0; e < out_n; ++e) {
        double d = fabs((double)out[e] - ref[e]);
        if (!(d <= 1e-3 + 1e-3 * fabs(ref[e]))) { fail("out outside tolerance"); break; }
        if (d > max_dout) max_dout = d;
    }
    for (size_t e = 0; e < lse_n; ++e) {
        if (isinf(ref_lse[e])) {
            if (!(isinf(lse[e]) && lse[e] < 0)) { fail("lse of an empty row is not -inf"); break; }
            continue;
        }
        double d = fabs((double)lse[e] - ref_lse[e]);
        if (!(d <= 1e-4 + 1e-4 * fabs(ref_lse[e]))) { fail("lse outside tolerance"); break; }
        if (d > max_dlse) max_dlse = d;
    }
    for (size_t e = 2 * (size_t)ROWS * D; e < out_n; ++e)
        if (out[e] != 0.0f) { fail("empty instance output is not zero"); break; }
    int g_bad = 0;
    for (int i = 0; i < N_INST; ++i)
        for (int j = 0; j < n_sel[i]; ++j)
            if ((int64_t)g[i * MAX_SEL + j] != ref_g[i * MAX_SEL + j]) ++g_bad;
    if (g_bad) fail("gather indices differ from the oracle");
    if (memcmp(out1, out, (size_t)ROWS * D * 4) || memcmp(lse1, lse, ROWS * 4) ||
        memcmp(g1, g, sizeof(int32_t) * MAX_SEL))
        fail("step entry differs from the batch entry");
    if (memcmp(out2, out, out_n * 4) || memcmp(lse2, lse, lse_n * 4))
        fail("two passes at the fused chunk size differ from the batch entry");

    printf("{\"c_abi_check\": \"%s\", \"instances\": %d, \"rows\": %d, \"fused_chunk\": %d, "
           "\"max_dout\": %.3e, \"max_dlse\": %.3e, \"rejected_status\": \"%s\", \"failures\": %d}\n",
           failures ? "fail" : "ok", N_INST, ROWS, fc, max_dout, max_dlse, name ? name : "", failures);
    return failures ? 1 : 0;
}
