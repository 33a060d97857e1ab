// Cold-cache HBM read ceilings on this GPU for the access shapes of the
// chunk pass: 256-byte code rows gathered at random, 4 KB pages (16 rows)
// gathered at random, a plain sequential read, and the batched decode call's
// own bytes (its code rows, scale pairs, lists, page-table entries and
// queries read, its outputs written; no arithmetic).  Each row-gather measurement
// reads 268 MB or 2.1 GB (16 or 128 tiles of 64 rows per workgroup), the
// sequential one 1 GiB, after evicting the caches by reading a separate
// 1 GiB buffer; after at least 60 ms of untimed launches, the median
// of 21 launches is printed as one JSON line per shape.  Standalone program (no library code); built next to
// libsda.so and run by `bench.py --gather-ceiling`.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

typedef int v4i __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            return 1;                                                              \
        }                                                                          \
    } while (0)

// Workgroup w gathers tiles of 64 rows from both pools: each of its 4 waves
// requests 8 blocks of 4 rows (16 lanes per 256-byte row) before using any.
__global__ __launch_bounds__(256) void row_gather(const int8_t *kp, const int8_t *vp,
                                                  const int *rows, int tiles, int *sink) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
    const int *my = rows + (int64_t)blockIdx.x * tiles * 64;
    v4i acc = {0, 0, 0, 0};
    for (int t = 0; t < tiles; ++t) {
        v4i st[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int k = wave + 4 * it;  // 32 blocks: 16 of K, 16 of V
            const int r = my[t * 64 + 4 * (k & 15) + g];
            st[it] = *reinterpret_cast<const v4i *>((k >= 16 ? vp : kp) + (int64_t)r * 256 + 16 * l16);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) acc ^= st[it];
    }
    if (acc.x == 0x13579bdf) sink[0] = acc.y;
}

// The batched decode call's own reads, with no arithmetic: workgroup
// (instance i, tile t) takes list entries [64 t, 64 t + 64) of instance i,
// looks each up in i's page table, then gathers the cells' K and V code rows
// (wave w: pool w / 2, cells 32 (w % 2) .. + 31, 8 loads of 4 rows in flight)
// and their interleaved (K, V) scale pairs; tile 0 also reads the instance's
// query rows, and each tile writes its share of as many bytes as the
// instance's output rows and log-sum-exps take (16-byte stores).  Small register use, so up to eight workgroups share a
// CU: the time to move exactly the call's bytes at the device's full
// occupancy.
__global__ __launch_bounds__(256) void decode_pattern(const int8_t *kp, const int8_t *vp,
                                                      const uint32_t *scales, const int *pt,
                                                      const int *sel, const v4i *q, int n_sel,
                                                      int pages, int tiles, int q_v4, v4i *out,
                                                      int out_v4, int *sink) {
    const int inst = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
    const int j = min(tile * 64 + lane, n_sel - 1);
    const int c = sel[(int64_t)inst * n_sel + j];
    const int ph = pt[(int64_t)inst * pages + (c >> 4)] * 16 + (c & 15);
    const int8_t *pool = wave >= 2 ? vp : kp;
    v4i st[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int r = __shfl(ph, 32 * (wave & 1) + 4 * it + g);
        st[it] = *reinterpret_cast<const v4i *>(pool + (int64_t)r * 256 + 16 * l16);
    }
    v4i acc = {0, 0, 0, 0};
    if (wave == 0) acc.x = (int)scales[ph];
    if (tile == 0)
        for (int e = threadIdx.x; e < q_v4; e += 256) acc ^= q[(int64_t)inst * q_v4 + e];
#pragma unroll
    for (int it = 0; it < 8; ++it) acc ^= st[it];
    const int share = (out_v4 + tiles - 1) / tiles, e = tile * share + threadIdx.x;
    if (threadIdx.x < share && e < out_v4) out[(int64_t)inst * out_v4 + e] = acc ^ e;
    if (acc.x == 0x13579bdf) sink[0] = acc.y;
}

__global__ __launch_bounds__(256) void seq_read(const v4i *src, int64_t n, int *sink) {
    v4i acc = {0, 0, 0, 0};
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) acc ^= src[e];
    if (acc.x == 0x13579bdf) sink[0] = acc.y;
}

int main() {
    const int64_t inst = 256, cells_per_inst = 32768, cells = inst * cells_per_inst;  // 2 GiB per pool
    const int wgs = 512, max_tiles = 128, max_per = max_tiles * 64;
    int8_t *kp, *vp;
    int *rows, *sink;
    v4i *flush;
    const int64_t flush_n = (1ll << 30) / 16;
    CHECK(hipMalloc(&kp, cells * 256));
    CHECK(hipMalloc(&vp, cells * 256));
    CHECK(hipMalloc(&flush, flush_n * 16));
    CHECK(hipMalloc(&rows, (size_t)wgs * max_per * sizeof(int)));
    CHECK(hipMalloc(&sink, 16));
    CHECK(hipMemset(kp, 1, cells * 256));
    CHECK(hipMemset(vp, 2, cells * 256));
    CHECK(hipMemset(flush, 3, flush_n * 16));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    auto evict = [&] { hipLaunchKernelGGL(seq_read, 2048, 256, 0, 0, flush, flush_n, sink); };
    evict();  // clean lines only from here on
    CHECK(hipDeviceSynchronize());
    // Untimed rounds first, until at least 60 ms of them have run: the first
    // 10-20 ms of sustained HBM traffic run slower than the steady state.
    // Then the median of 21 timed launches.
    auto median_us = [&](auto launch) {
        std::vector<float> v;
        float warm_ms = 0.f;
        for (int rep = 0; rep < 100000 && (warm_ms < 60.f || (int)v.size() < 21); ++rep) {
            evict();
            hipEventRecord(e0);
            launch();
            hipEventRecord(e1);
            hipEventSynchronize(e1);
            float ms = 0.f;
            hipEventElapsedTime(&ms, e0, e1);
            if (warm_ms < 60.f)
                warm_ms += ms + 0.15f;  // with the eviction read before it
            else
                v.push_back(ms * 1e3f);
        }
        std::sort(v.begin(), v.end());
        return v[v.size() / 2];
    };
    // Two launch lengths: 16 tiles per workgroup (268 MB, about 50 us, where
    // the grid's start and drain weigh) and 128 (2.1 GB, about 400 us).
    const char *shape[3] = {"random 256-byte rows", "random 4 KB pages of 16 rows", "sequential rows"};
    std::mt19937_64 rng(7);
    std::vector<int> host((size_t)wgs * max_per);
    for (int tiles : {16, max_tiles}) {
        const int per = tiles * 64;
        const double gather_bytes = (double)wgs * per * 512;
        for (int s = 0; s < 3; ++s) {
            for (int w = 0; w < wgs; ++w) {
                const int64_t base = (int64_t)(w / 2) * cells_per_inst;  // two workgroups per instance
                std::vector<int> c(cells_per_inst);
                for (int j = 0; j < cells_per_inst; ++j) c[j] = j;
                if (s == 0) {
                    std::shuffle(c.begin(), c.end(), rng);
                } else if (s == 1) {
                    std::vector<int> pg(cells_per_inst / 16);
                    for (size_t j = 0; j < pg.size(); ++j) pg[j] = (int)j;
                    std::shuffle(pg.begin(), pg.end(), rng);
                    for (int j = 0; j < per; ++j) c[j] = pg[j / 16] * 16 + (j & 15);
                } else {
                    for (int j = 0; j < per; ++j) c[j] = (w & 1) * per + j;
                }
                for (int j = 0; j < per; ++j) host[(size_t)w * per + j] = (int)(base + c[j]);
            }
            for (size_t j = 0; j < (size_t)wgs * per; ++j)
                if (host[j] < 0 || host[j] >= cells) { fprintf(stderr, "row out of range\n"); return 1; }
            CHECK(hipMemcpy(rows, host.data(), (size_t)wgs * per * sizeof(int), hipMemcpyHostToDevice));
            const float us = median_us([&] { hipLaunchKernelGGL(row_gather, wgs, 256, 0, 0, kp, vp, rows, tiles, sink); });
            printf("{\"shape\": \"%s\", \"tiles_per_workgroup\": %d, \"bytes\": %.0f, \"us\": %.2f, \"GBps\": %.1f}\n",
                   shape[s], tiles, gather_bytes, us, gather_bytes / (us * 1e-6) / 1e9);
            fflush(stdout);
        }
    }
    {
        // batched decode: 256 instances, 2,051 sorted random cells of each
        // instance's 32,768, its 2,048 pages a permutation of its own range
        // of the pool, 48 query rows of 1 KB
        const int n_inst = 256, n_sel = 2051, pages = cells_per_inst / 16, tiles = (n_sel + 63) / 64;
        const int q_v4 = 48 * 256 * 4 / 16, out_v4 = 48 * 257 * 4 / 16;
        std::vector<int> hsel((size_t)n_inst * n_sel), hpt((size_t)n_inst * pages);
        double bytes = 0.0;
        for (int i = 0; i < n_inst; ++i) {
            std::vector<int> c(cells_per_inst), pg(pages);
            for (int j = 0; j < cells_per_inst; ++j) c[j] = j;
            std::shuffle(c.begin(), c.end(), rng);
            std::sort(c.begin(), c.begin() + n_sel);
            for (int j = 0; j < pages; ++j) pg[j] = i * pages + j;
            std::shuffle(pg.begin(), pg.end(), rng);
            std::vector<char> touched(pages, 0);
            for (int j = 0; j < n_sel; ++j) {
                hsel[(size_t)i * n_sel + j] = c[j];
                touched[c[j] >> 4] = 1;
            }
            for (int j = 0; j < pages; ++j) {
                hpt[(size_t)i * pages + j] = pg[j];
                bytes += 4.0 * touched[j];
            }
        }
        // code rows, scale pair and list entry per cell, the query rows, the
        // outputs
        bytes += (double)n_inst * n_sel * (512 + 4 + 4) + (double)n_inst * q_v4 * 16 + (double)n_inst * out_v4 * 16;
        for (size_t e = 0; e < hpt.size(); ++e)
            if (hpt[e] < 0 || (int64_t)hpt[e] * 16 + 15 >= cells) { fprintf(stderr, "page out of range\n"); return 1; }
        for (size_t e = 0; e < hsel.size(); ++e)
            if (hsel[e] < 0 || hsel[e] >= cells_per_inst) { fprintf(stderr, "cell out of range\n"); return 1; }
        int *dsel, *dpt;
        uint32_t *dsc;
        v4i *dq, *dout;
        CHECK(hipMalloc(&dsel, hsel.size() * sizeof(int)));
        CHECK(hipMalloc(&dpt, hpt.size() * sizeof(int)));
        CHECK(hipMalloc(&dsc, cells * sizeof(uint32_t)));
        CHECK(hipMalloc(&dq, (size_t)n_inst * q_v4 * 16));
        CHECK(hipMalloc(&dout, (size_t)n_inst * out_v4 * 16));
        CHECK(hipMemcpy(dsel, hsel.data(), hsel.size() * sizeof(int), hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dpt, hpt.data(), hpt.size() * sizeof(int), hipMemcpyHostToDevice));
        CHECK(hipMemset(dsc, 4, cells * sizeof(uint32_t)));
        CHECK(hipMemset(dq, 5, (size_t)n_inst * q_v4 * 16));
        // the reads alone, then with the writes
        for (int w = 0; w < 2; ++w) {
            const int nv = w ? out_v4 : 0;
            const double b = bytes - (w ? 0.0 : (double)n_inst * out_v4 * 16);
            const float us = median_us([&] {
                hipLaunchKernelGGL(decode_pattern, n_inst * tiles, 256, 0, 0, kp, vp, dsc, dpt, dsel, dq, n_sel,
                                   pages, tiles, q_v4, dout, nv, sink);
            });
            printf("{\"shape\": \"batched decode call's %s (256 x 2051 cells: code rows, scale pairs, lists, "
                   "page table, queries%s)\", \"bytes\": %.0f, \"us\": %.2f, \"GBps\": %.1f}\n",
                   w ? "bytes" : "reads", w ? "; outputs" : "", b, us, b / (us * 1e-6) / 1e9);
            fflush(stdout);
        }
        CHECK(hipFree(dsel));
        CHECK(hipFree(dpt));
        CHECK(hipFree(dsc));
        CHECK(hipFree(dq));
        CHECK(hipFree(dout));
    }
    const int64_t seq_n = (1ll << 30) / 16;
    const float us = median_us([&] { hipLaunchKernelGGL(seq_read, 4096, 256, 0, 0, (const v4i *)kp, seq_n, sink); });
    printf("{\"shape\": \"sequential read\", \"bytes\": %.0f, \"us\": %.2f, \"GBps\": %.1f}\n", (double)seq_n * 16, us,
           seq_n * 16 / (us * 1e-6) / 1e9);
    CHECK(hipDeviceSynchronize());
    return 0;
}
