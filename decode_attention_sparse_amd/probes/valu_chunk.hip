// The pages' two design knobs of the chunk pass, as vector-ALU (no matrix
// core) variants, timed beside the library's MFMA chunk kernel on the same
// inputs.  A measurement program only: none of this is in libsda.so, which
// it loads at run time to time sda_chunk_batch.
//
// Source of the knobs: Strata round-9 page, section "R9-gpu-11: four score
// cells per step in daily INT8 attention" (NC score cells per step reuse the
// query slice; two by default, four was slower on V100), and the Strata
// PR #2220 page (lane-cell scoring, STRATA_ATTN_LANECELL=1, beside the
// warp-per-cell kernels).  Rewritten for wave64:
//   wave_cell<NC>  a wave owns 12 query rows and walks the chunk's cells NC at
//                  a time: each lane holds 4 dims of the 12 query rows in
//                  registers, reads 4 bytes of each K row (one coalesced
//                  256-byte row per cell), and the 12 NC partial sums are
//                  reduced across the 64 lanes by halving exchanges (12 -> 6
//                  -> 3 values per lane, then 4 more levels: 21 lane swaps per
//                  cell instead of 72); probabilities are broadcast from the
//                  lanes that hold them, and each lane accumulates its 4 dims
//                  of the 12 rows.
//   lane_cell      a wave scores 64 cells at once, one per lane: each lane
//                  reads its cell's whole K row and the 12 query rows as LDS
//                  broadcasts, so no cross-lane sum is needed; the
//                  probabilities go to LDS cell-major and the V accumulation
//                  runs as in wave_cell.
// Both write the chunk partials (acc, m, l) in the library's workspace
// layout.  Correctness: instance 0's partials against a host fp64
// computation.  Output: one JSON line per (workload, kernel) with the median
// microseconds of 20 launches (after 3 untimed), back to back.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/sda.h"

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

constexpr int D = 256;
constexpr int RW = 12;  // query rows per wave

struct Work {
    const int8_t *kc, *vc;
    const uint16_t *ks, *vs;  // binary16 scales per physical cell
    const int32_t *pt, *sel;  // [inst][pages], [inst][n]
    const float *q;           // [inst][R][D]
    int n, R, chunk, n_chunks, pages;
    float scale_log2;
    float *acc, *m, *l;  // [inst][n_chunks][R][D], [inst][n_chunks][R]
};

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ int phys_of(const Work &w, int i, int j) {
    const int c = w.sel[(int64_t)i * w.n + j];
    const int pp = w.pt[(int64_t)i * w.pages + (c >> 4)];
    return pp * 16 + (c & 15);
}

// Emits the partial of 12 rows held as acc[r][4 dims per lane], m, l (base 2).
__device__ __forceinline__ void emit(const Work &w, int i, int c, int row0, float (&acc)[RW][4],
                                     const float (&m)[RW], const float (&l)[RW], int lane) {
    for (int r = 0; r < RW; ++r) {
        const int row = row0 + r;
        if (row >= w.R) break;
        const int64_t u = ((int64_t)i * w.n_chunks + c) * w.R + row;
        for (int e = 0; e < 4; ++e) w.acc[u * D + 4 * lane + e] = acc[r][e];
        if (lane == 0) {
            w.m[u] = m[r] == -INFINITY ? -INFINITY : m[r] * 0.69314718f;
            w.l[u] = l[r];
        }
    }
}

// wave_cell: grid (inst, chunk), one wave per 12-row group.
template <int NC>
__global__ __launch_bounds__(256) void wave_cell(Work w) {
    const int i = blockIdx.x, c = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = wave * RW;
    if (row0 >= w.R) return;
    float q[RW][4];
    for (int r = 0; r < RW; ++r)
        for (int e = 0; e < 4; ++e)
            q[r][e] = row0 + r < w.R ? w.q[((int64_t)i * w.R + row0 + r) * D + 4 * lane + e] * w.scale_log2 : 0.f;
    float acc[RW][4] = {}, m[RW], l[RW] = {};
    for (int r = 0; r < RW; ++r) m[r] = -INFINITY;
    const int j0 = c * w.chunk, j1 = min(j0 + w.chunk, w.n);
    for (int j = j0; j < j1; j += NC) {
        // NC cells: partial dots of this lane's 4 dims for the 12 rows
        float s[NC][RW];
        int ph[NC];
        float ksc[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const bool ok = j + k < j1;
            ph[k] = ok ? phys_of(w, i, j + k) : 0;
            const uint32_t kr = *reinterpret_cast<const uint32_t *>(w.kc + (int64_t)ph[k] * D + 4 * lane);
            ksc[k] = ok ? h2f(w.ks[ph[k]]) : 0.f;
            const float kv[4] = {(float)(int8_t)kr, (float)(int8_t)(kr >> 8), (float)(int8_t)(kr >> 16),
                                 (float)(int8_t)(kr >> 24)};
#pragma unroll
            for (int r = 0; r < RW; ++r)
                s[k][r] = q[r][0] * kv[0] + q[r][1] * kv[1] + q[r][2] * kv[2] + q[r][3] * kv[3];
        }
        // halving exchanges: xor 32 keeps 6 rows, xor 16 keeps 3, then full sums
        const bool h32 = lane & 32, h16 = lane & 16;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            float t6[6], t3[3];
#pragma unroll
            for (int e = 0; e < 6; ++e) {
                const float mine = h32 ? s[k][6 + e] : s[k][e];
                const float give = h32 ? s[k][e] : s[k][6 + e];
                t6[e] = mine + __shfl_xor(give, 32);
            }
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const float mine = h16 ? t6[3 + e] : t6[e];
                const float give = h16 ? t6[e] : t6[3 + e];
                t3[e] = mine + __shfl_xor(give, 16);
            }
#pragma unroll
            for (int e = 0; e < 3; ++e)
                for (int x = 8; x >= 1; x >>= 1) t3[e] += __shfl_xor(t3[e], x);
            // lanes of group g = lane >> 4 now hold rows 3g .. 3g + 2: broadcast all 12
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float v = __shfl(t3[r % 3], 16 * (r / 3));
                s[k][r] = (j + k < j1) ? v * ksc[k] : -INFINITY;
            }
        }
        // online softmax over the NC cells, then V
        float p[NC][RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            float mx = m[r];
#pragma unroll
            for (int k = 0; k < NC; ++k) mx = fmaxf(mx, s[k][r]);
            const float corr = mx == -INFINITY ? 1.f : exp2f(m[r] - mx);
            m[r] = mx;
            l[r] *= corr;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] *= corr;
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                p[k][r] = mx == -INFINITY ? 0.f : exp2f(s[k][r] - mx);
                l[r] += p[k][r];
            }
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const uint32_t vr = *reinterpret_cast<const uint32_t *>(w.vc + (int64_t)ph[k] * D + 4 * lane);
            const float vsc = (j + k < j1) ? h2f(w.vs[ph[k]]) : 0.f;
            const float vv[4] = {(float)(int8_t)vr, (float)(int8_t)(vr >> 8), (float)(int8_t)(vr >> 16),
                                 (float)(int8_t)(vr >> 24)};
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float pw = p[k][r] * vsc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(pw, vv[e], acc[r][e]);
            }
        }
    }
    emit(w, i, c, row0, acc, m, l, lane);
}

// lane_cell: grid (inst, chunk), one wave per 12-row group, 64 cells per step.
__global__ __launch_bounds__(256) void lane_cell(Work w) {
    __shared__ float qs[4][RW][D];
    __shared__ float ps[4][64][RW];
    const int i = blockIdx.x, c = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = wave * RW;
    for (int e = threadIdx.x; e < 4 * RW * D; e += 256) {
        const int wv = e / (RW * D), r = (e / D) % RW, d = e % D;
        const int row = wv * RW + r;
        (&qs[0][0][0])[e] = row < w.R ? w.q[((int64_t)i * w.R + row) * D + d] * w.scale_log2 : 0.f;
    }
    __syncthreads();
    if (row0 >= w.R) return;
    float acc[RW][4] = {}, m[RW], l[RW] = {};
    for (int r = 0; r < RW; ++r) m[r] = -INFINITY;
    const int j0 = c * w.chunk, j1 = min(j0 + w.chunk, w.n);
    for (int jb = j0; jb < j1; jb += 64) {
        const int j = jb + lane;
        const bool ok = j < j1;
        const int ph = ok ? phys_of(w, i, j) : 0;
        float s[RW] = {};
        const int8_t *kr = w.kc + (int64_t)ph * D;
        for (int d0 = 0; d0 < D; d0 += 16) {
            int8_t kv[16];
            *reinterpret_cast<int4 *>(kv) = *reinterpret_cast<const int4 *>(kr + d0);
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[r] = fmaf(qs[wave][r][d0 + e], (float)kv[e], s[r]);
        }
        const float ksc = ok ? h2f(w.ks[ph]) : 0.f;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const float sc = ok ? s[r] * ksc : -INFINITY;
            float mx = sc;
            for (int x = 32; x >= 1; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
            mx = fmaxf(mx, m[r]);
            const float corr = mx == -INFINITY ? 1.f : exp2f(m[r] - mx);
            const float p = mx == -INFINITY ? 0.f : exp2f(sc - mx);
            float ps_sum = p;
            for (int x = 32; x >= 1; x >>= 1) ps_sum += __shfl_xor(ps_sum, x);
            l[r] = l[r] * corr + ps_sum;
            m[r] = mx;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] *= corr;
            ps[wave][lane][r] = p * (ok ? h2f(w.vs[ph]) : 0.f);  // cell-major
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const int cells = min(64, j1 - jb);
        for (int k = 0; k < cells; ++k) {
            const int phk = phys_of(w, i, jb + k);
            const uint32_t vr = *reinterpret_cast<const uint32_t *>(w.vc + (int64_t)phk * D + 4 * lane);
            const float vv[4] = {(float)(int8_t)vr, (float)(int8_t)(vr >> 8), (float)(int8_t)(vr >> 16),
                                 (float)(int8_t)(vr >> 24)};
            const float4 *pr = reinterpret_cast<const float4 *>(&ps[wave][k][0]);
            float pw[RW];
            *reinterpret_cast<float4 *>(&pw[0]) = pr[0];
            *reinterpret_cast<float4 *>(&pw[4]) = pr[1];
            *reinterpret_cast<float4 *>(&pw[8]) = pr[2];
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(pw[r], vv[e], acc[r][e]);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    emit(w, i, c, row0, acc, m, l, lane);
}

static float median(std::vector<float> v) {
    std::sort(v.begin(), v.end());
    return v[v.size() / 2];
}

template <typename F>
static float time_us(F launch) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int k = 0; k < 3; ++k) launch();
    CHECK(hipDeviceSynchronize());
    std::vector<float> t;
    for (int k = 0; k < 20; ++k) {
        CHECK(hipEventRecord(e0));
        launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        t.push_back(ms * 1e3f);
    }
    return median(t);
}

int main(int argc, char **argv) {
    const char *lib_path = argc > 1 ? argv[1] : "decode_attention_sparse_amd/libsda.so";
    void *lib = dlopen(lib_path, RTLD_NOW);
    if (!lib) {
        fprintf(stderr, "%s\n", dlerror());
        return 1;
    }
    auto sda_chunk = (decltype(&sda_chunk_batch))dlsym(lib, "sda_chunk_batch");
    auto sda_fused = (decltype(&sda_decode_attn_batch))dlsym(lib, "sda_decode_attn_batch");
    auto sda_ws = (decltype(&sda_workspace_bytes))dlsym(lib, "sda_workspace_bytes");
    auto sda_fcc = (decltype(&sda_fused_chunk_cells))dlsym(lib, "sda_fused_chunk_cells");
    if (!sda_chunk || !sda_fused || !sda_ws || !sda_fcc) {
        fprintf(stderr, "libsda.so lacks an entry point\n");
        return 1;
    }
    // the VALU chunk passes run at the chunk size the library's fused call
    // picks for the stated chunk, so both split the cells the same way
    struct Shape {
        const char *name;
        int inst, n, n_q, stated_chunk;
    } shapes[] = {
        {"pages_kernel_point_1inst_2051cells_4q_12heads", 1, 2051, 4, 256},
        {"pages_kernel_point_1inst_2051cells_1q_12heads", 1, 2051, 1, 256},
        {"batched_decode_256inst_2051cells_4q_12heads", 256, 2051, 4, 1024},
    };
    const int pool_cells = 32768, pages = pool_cells / 16;
    for (Shape sh0 : shapes) {
        struct {
            const char *name;
            int inst, n, R, chunk;
        } sh{sh0.name, sh0.inst, sh0.n, 12 * sh0.n_q, 0};
        if (sda_fcc(sh.inst, sh.n, sh0.stated_chunk, &sh.chunk) != SDA_OK) return 1;
        std::mt19937_64 rng(20261600 + sh.inst);
        const int64_t cells = (int64_t)sh.inst * pool_cells;
        std::vector<int8_t> kc(cells * D), vc(cells * D);
        std::vector<uint16_t> ksc(cells), vsc(cells), sc2(cells * 2);
        std::vector<int32_t> pt((int64_t)sh.inst * pages), sel((int64_t)sh.inst * sh.n), nsel(sh.inst, sh.n);
        std::vector<float> q((int64_t)sh.inst * sh.R * D);
        std::uniform_real_distribution<float> sdist(0.002f, 0.02f);
        std::normal_distribution<float> nd(0.f, 1.f);
        // codes: 8 bytes per draw, -128 folded to -127
        for (auto *v : {&kc, &vc})
            for (size_t e = 0; e < v->size(); e += 8) {
                uint64_t r = rng();
                for (int b = 0; b < 8; ++b, r >>= 8) (*v)[e + b] = (int8_t)std::max<int>((int8_t)(r & 255), -127);
            }
        for (int64_t e = 0; e < cells; ++e) {
            _Float16 a = (_Float16)sdist(rng), b = (_Float16)sdist(rng);
            memcpy(&ksc[e], &a, 2);
            memcpy(&vsc[e], &b, 2);
            sc2[2 * e] = ksc[e];
            sc2[2 * e + 1] = vsc[e];
        }
        for (int i = 0; i < sh.inst; ++i) {
            std::vector<int> perm(pages), pick(pool_cells);
            for (int k = 0; k < pages; ++k) perm[k] = k + i * pages;
            std::shuffle(perm.begin(), perm.end(), rng);
            for (int k = 0; k < pages; ++k) pt[(int64_t)i * pages + k] = perm[k];
            for (int k = 0; k < pool_cells; ++k) pick[k] = k;
            std::shuffle(pick.begin(), pick.end(), rng);
            std::sort(pick.begin(), pick.begin() + sh.n);
            for (int k = 0; k < sh.n; ++k) sel[(int64_t)i * sh.n + k] = pick[k];
        }
        for (auto &x : q) x = nd(rng);
        int8_t *dkc, *dvc;
        uint16_t *dks, *dvs, *dsc2;
        int32_t *dpt, *dsel, *dnsel;
        float *dq, *acc, *m, *l;
        const int nch = (sh.n + sh.chunk - 1) / sh.chunk;
        const int64_t units = (int64_t)sh.inst * nch * sh.R;
        CHECK(hipMalloc(&dkc, kc.size()));
        CHECK(hipMalloc(&dvc, vc.size()));
        CHECK(hipMalloc(&dks, cells * 2));
        CHECK(hipMalloc(&dvs, cells * 2));
        CHECK(hipMalloc(&dsc2, cells * 4));
        CHECK(hipMalloc(&dpt, pt.size() * 4));
        CHECK(hipMalloc(&dsel, sel.size() * 4));
        CHECK(hipMalloc(&dnsel, nsel.size() * 4));
        CHECK(hipMalloc(&dq, q.size() * 4));
        CHECK(hipMalloc(&acc, units * D * 4));
        CHECK(hipMalloc(&m, units * 4));
        CHECK(hipMalloc(&l, units * 4));
        CHECK(hipMemcpy(dkc, kc.data(), kc.size(), hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dvc, vc.data(), vc.size(), hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dks, ksc.data(), cells * 2, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dvs, vsc.data(), cells * 2, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dsc2, sc2.data(), cells * 4, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dpt, pt.data(), pt.size() * 4, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dsel, sel.data(), sel.size() * 4, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dnsel, nsel.data(), nsel.size() * 4, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dq, q.data(), q.size() * 4, hipMemcpyHostToDevice));
        const float sm = 1.f / 16.f;
        Work w{dkc, dvc, dks, dvs, dpt, dsel, dq, sh.n, sh.R, sh.chunk, nch, pages,
               sm * 1.4426950408889634f, acc, m, l};
        const dim3 grid(sh.inst, nch);
        const int threads = 64 * ((sh.R + RW - 1) / RW);
        // host fp64 check of instance 0's partials
        auto check = [&]() {
            CHECK(hipDeviceSynchronize());
            const int64_t u0 = (int64_t)nch * sh.R;
            std::vector<float> ga(u0 * D), gm(u0), gl(u0);
            CHECK(hipMemcpy(ga.data(), acc, u0 * D * 4, hipMemcpyDeviceToHost));
            CHECK(hipMemcpy(gm.data(), m, u0 * 4, hipMemcpyDeviceToHost));
            CHECK(hipMemcpy(gl.data(), l, u0 * 4, hipMemcpyDeviceToHost));
            double worst = 0;
            auto h = [](uint16_t b) { _Float16 f; memcpy(&f, &b, 2); return (double)f; };
            for (int cc = 0; cc < nch; ++cc)
                for (int r = 0; r < sh.R; ++r) {
                    const int j0 = cc * sh.chunk, j1 = std::min(j0 + sh.chunk, sh.n);
                    std::vector<double> s(j1 - j0);
                    double mx = -INFINITY;
                    for (int j = j0; j < j1; ++j) {
                        const int cl = sel[j], ph = pt[cl >> 4] * 16 + (cl & 15);
                        double dot = 0;
                        for (int d = 0; d < D; ++d) dot += (double)q[r * D + d] * kc[(int64_t)ph * D + d];
                        s[j - j0] = dot * h(ksc[ph]) * sm;
                        mx = std::max(mx, s[j - j0]);
                    }
                    double lsum = 0;
                    std::vector<double> a(D, 0.0);
                    for (int j = j0; j < j1; ++j) {
                        const int cl = sel[j], ph = pt[cl >> 4] * 16 + (cl & 15);
                        const double p = std::exp(s[j - j0] - mx);
                        lsum += p;
                        for (int d = 0; d < D; ++d) a[d] += p * h(vsc[ph]) * vc[(int64_t)ph * D + d];
                    }
                    const int64_t u = (int64_t)cc * sh.R + r;
                    const double gsc = std::exp((double)gm[u] - mx);  // this side's reference
                    worst = std::max(worst, std::fabs(gl[u] * gsc - lsum) / lsum);
                    for (int d = 0; d < D; ++d)  // on the scale of the attention output
                        worst = std::max(worst, std::fabs(ga[u * D + d] * gsc - a[d]) / lsum);
                }
            return worst;
        };
        auto report = [&](const char *kname, float us, double err) {
            printf("{\"workload\": \"%s\", \"kernel\": \"%s\", \"us_median\": %.3f, "
                   "\"instances\": %d, \"cells\": %d, \"rows\": %d, \"chunk\": %d, "
                   "\"max_err_instance0\": %.2e}\n",
                   sh.name, kname, us, sh.inst, sh.n, sh.R, sh.chunk, err);
            fflush(stdout);
        };
        float us = time_us([&] { wave_cell<1><<<grid, threads>>>(w); });
        report("wave_cell NC=1", us, check());
        us = time_us([&] { wave_cell<2><<<grid, threads>>>(w); });
        report("wave_cell NC=2", us, check());
        us = time_us([&] { wave_cell<4><<<grid, threads>>>(w); });
        report("wave_cell NC=4", us, check());
        us = time_us([&] { lane_cell<<<grid, 256>>>(w); });
        report("lane_cell", us, check());
        // the library on the same pools: its chunk pass at the same chunk
        // size, then its fused call (chunk pass + merge, or one launch)
        sda_pool pool{dkc, dsc2, dvc, dsc2 + 1, cells / 16, 16, 256, 2, 0};
        size_t wsb = 0;
        if (sda_ws(sh.inst, sh0.n_q, 12, 256, sh.n, sh.chunk, &wsb) != SDA_OK) return 1;
        void *ws;
        float *out, *lse;
        CHECK(hipMalloc(&ws, wsb));
        CHECK(hipMalloc(&out, (size_t)sh.inst * sh.R * D * 4));
        CHECK(hipMalloc(&lse, (size_t)sh.inst * sh.R * 4));
        int st = SDA_OK;
        us = time_us([&] {
            st |= sda_chunk(&pool, sh.inst, dpt, pages, pages, dsel, sh.n, dnsel, sh.n, dq, sh0.n_q,
                            12, sm, sh.chunk, nullptr, ws, wsb, nullptr);
        });
        if (st != SDA_OK) return 1;
        // its partials under the same check (the rows are ordered as here)
        CHECK(hipMemcpy(acc, ws, (size_t)nch * sh.R * D * 4, hipMemcpyDeviceToDevice));
        const size_t a256 = ((size_t)sh.inst * nch * sh.R * D * 4 + 255) / 256 * 256;
        const size_t m256 = ((size_t)sh.inst * nch * sh.R * 4 + 255) / 256 * 256;
        CHECK(hipMemcpy(m, (char *)ws + a256, (size_t)nch * sh.R * 4, hipMemcpyDeviceToDevice));
        CHECK(hipMemcpy(l, (char *)ws + a256 + m256, (size_t)nch * sh.R * 4, hipMemcpyDeviceToDevice));
        report("libsda sda_chunk_batch (MFMA chunk pass)", us, check());
        us = time_us([&] {
            st |= sda_fused(&pool, sh.inst, dpt, pages, pages, dsel, sh.n, dnsel, sh.n, dq, sh0.n_q,
                            12, sm, sh0.stated_chunk, out, lse, nullptr, ws, wsb, nullptr);
        });
        if (st != SDA_OK) return 1;
        report("libsda sda_decode_attn_batch (fused, with merge)", us, 0.0);
        CHECK(hipFree(ws));
        CHECK(hipFree(out));
        CHECK(hipFree(lse));
        for (void *ptr : {(void *)dkc, (void *)dvc, (void *)dks, (void *)dvs, (void *)dsc2, (void *)dpt,
                          (void *)dsel, (void *)dnsel, (void *)dq, (void *)acc, (void *)m, (void *)l})
            CHECK(hipFree(ptr));
    }
    return 0;
}
