/* The C ABI's host-side logic (argument validation, geometry helpers,
 * status strings) under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every entry point is called with arguments it must reject before any
 * device work (null pointers, negative or oversized counts, bad strides,
 * unsupported geometry), and the host-only helpers are swept over ranges
 * that include their edges.  No GPU is needed: nothing here may launch.
 * Prints "ok" and exits 0 when every call returned the expected status.
 * Test infrastructure, built and run by tests/test_abi_sanitized.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sda.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got, sda_status_string(got), want);
        ++failures;
    }
}

int main(void) {
    static int8_t codes[16 * SDA_HEAD_DIM] __attribute__((aligned(16)));
    static uint16_t scales[32];
    static int32_t pt[8], sel[64], n_sel[2], pos0[2];
    static float q[64 * SDA_HEAD_DIM], out[64 * SDA_HEAD_DIM], lse[64], kv[SDA_HEAD_DIM];
    static uint8_t dead[8];
    char ws[256] __attribute__((aligned(256)));
    sda_pool pool = {codes, scales, codes, scales, 1, SDA_PAGE_SIZE, SDA_HEAD_DIM, 1, 0};
    sda_pool_mut mpool = {codes, scales, codes, scales, 1, SDA_PAGE_SIZE, SDA_HEAD_DIM, 1, 0};

    /* status strings, including unknown codes */
    for (int s = -10; s <= 3; ++s)
        if (!sda_status_string(s) || !sda_status_string(s)[0]) {
            fprintf(stderr, "status string %d empty\n", s);
            ++failures;
        }

    /* geometry helpers over their edges */
    size_t bytes = 0;
    int32_t v = 0;
    const int32_t vals[] = {-1, 0, 1, 63, 64, 65, 255, 256, 4096, 65535, 1 << 20, 2147483647};
    const int nv = (int)(sizeof vals / sizeof vals[0]);
    for (int a = 0; a < nv; ++a)
        for (int b = 0; b < nv; ++b)
            for (int c = 0; c < nv; ++c) {
                (void)sda_workspace_bytes(vals[a], 4, 12, SDA_HEAD_DIM, vals[b], vals[c], &bytes);
                (void)sda_workspace_bytes(2, vals[a] % 70, 12, SDA_HEAD_DIM, vals[b], vals[c], &bytes);
                (void)sda_fused_chunk_cells(vals[a], vals[b], vals[c], &v);
                (void)sda_fused_single_launch(vals[a], 4, 12, vals[b], vals[c], &v);
                (void)sda_fused_single_launch(vals[a], vals[b] % 70, 3, 600, vals[c], &v);
            }
    expect("workspace null out", sda_workspace_bytes(1, 1, 12, SDA_HEAD_DIM, 64, 64, NULL),
           SDA_ERR_INVALID_ARG);
    expect("workspace negative", sda_workspace_bytes(-1, 1, 12, SDA_HEAD_DIM, 64, 64, &bytes),
           SDA_ERR_INVALID_ARG);
    expect("workspace head_dim", sda_workspace_bytes(1, 1, 12, 128, 64, 64, &bytes), SDA_ERR_UNSUPPORTED);
    expect("fused chunk null", sda_fused_chunk_cells(1, 64, 64, NULL), SDA_ERR_INVALID_ARG);
    expect("fused chunk align", sda_fused_chunk_cells(1, 64, 100, &v), SDA_ERR_UNSUPPORTED);
    expect("single launch rows", sda_fused_single_launch(1, 8, 12, 64, 64, &v), SDA_ERR_UNSUPPORTED);

    /* decode entry points: each rejection before any launch */
    expect("step null pool", sda_decode_attn_step(NULL, pt, 1, sel, 1, q, 1, 12, 1.f, 64, out, lse,
                                                  NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    expect("batch null q", sda_decode_attn_batch(&pool, 1, pt, 1, 1, sel, 64, n_sel, 64, NULL, 1, 12,
                                                 1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    expect("batch negative inst", sda_decode_attn_batch(&pool, -1, pt, 1, 1, sel, 64, n_sel, 64, q, 1,
                                                        12, 1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    expect("batch sel stride", sda_decode_attn_batch(&pool, 1, pt, 1, 1, sel, 8, n_sel, 64, q, 1, 12,
                                                     1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    expect("batch rows", sda_decode_attn_batch(&pool, 1, pt, 1, 1, sel, 64, n_sel, 64, q, 8, 12, 1.f,
                                               64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_UNSUPPORTED);
    expect("batch chunk", sda_decode_attn_batch(&pool, 1, pt, 1, 1, sel, 64, n_sel, 64, q, 1, 12, 1.f,
                                                100, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_UNSUPPORTED);
    sda_pool bad = pool;
    bad.page_size = 32;
    expect("batch page size", sda_decode_attn_batch(&bad, 1, pt, 1, 1, sel, 64, n_sel, 64, q, 1, 12,
                                                    1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_UNSUPPORTED);
    bad = pool;
    bad.reserved = 1;
    expect("batch reserved", sda_decode_attn_batch(&bad, 1, pt, 1, 1, sel, 64, n_sel, 64, q, 1, 12,
                                                   1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    bad = pool;
    bad.k_codes = codes + 1;  /* misaligned */
    expect("batch alignment", sda_decode_attn_batch(&bad, 1, pt, 1, 1, sel, 64, n_sel, 64, q, 1, 12,
                                                    1.f, 64, out, lse, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    /* (host pointers stand in for device arrays: nothing is dereferenced) */
    expect("batch no workspace", sda_decode_attn_batch(&pool, 1, pt, 1, 1, sel, 4096, n_sel, 4096, q,
                                                       4, 12, 1.f, 64, out, lse, NULL, NULL, 0, NULL),
           SDA_ERR_WORKSPACE);
    expect("chunk pass null", sda_chunk_batch(&pool, 1, pt, 1, 1, NULL, 64, n_sel, 64, q, 1, 12, 1.f,
                                              64, NULL, ws, sizeof ws, NULL),
           SDA_ERR_INVALID_ARG);
    expect("merge null", sda_merge_batch(1, 1, 12, n_sel, 64, 64, ws, sizeof ws, NULL, lse, NULL),
           SDA_ERR_INVALID_ARG);
    expect("noalloc null pool", sda_decode_attn_batch_noalloc(NULL, 1, pt, 1, 1, sel, 64, n_sel, 64, q,
                                                              1, 12, 1.f, 64, out, lse, NULL, NULL),
           SDA_ERR_INVALID_ARG);

    /* prompt, append and QSA */
    expect("prompt null pos0", sda_prompt_attn_batch(&pool, 1, pt, 1, 1, NULL, q, 1, 12, 1.f, out, lse,
                                                     NULL),
           SDA_ERR_INVALID_ARG);
    expect("prompt rows", sda_prompt_attn_batch(&pool, 1, pt, 1, 1, pos0, q, 0, 12, 1.f, out, lse, NULL),
           SDA_ERR_INVALID_ARG);
    expect("append null rows", sda_kv_append_batch(&mpool, 1, pt, 1, 1, pos0, NULL, kv, 1, NULL),
           SDA_ERR_INVALID_ARG);
    sda_pool_mut mbad = mpool;
    mbad.scale_stride = 65;
    expect("append stride", sda_kv_append_batch(&mbad, 1, pt, 1, 1, pos0, kv, kv, 1, NULL),
           SDA_ERR_INVALID_ARG);
    expect("qsa scores null", sda_qsa_block_scores(1, 1, 4, 128, 256, 8, NULL, dead, q, n_sel, lse,
                                                   NULL),
           SDA_ERR_INVALID_ARG);
    expect("qsa select blocks", sda_qsa_select(1, 1, 256, SDA_QSA_MAX_BLOCKS + 1, lse, n_sel, 4, sel,
                                               64 * 256, n_sel, NULL),
           SDA_ERR_UNSUPPORTED);
    expect("qsa select stride", sda_qsa_select(1, 1, 256, 8, lse, n_sel, 4, sel, 10, n_sel, NULL),
           SDA_ERR_INVALID_ARG);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
