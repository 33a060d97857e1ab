// Merge pass: log-sum-exp combination of the chunk partials of one
// (instance, query row) into the head output and its log-sum-exp.
//
// Source: Strata PR #2220 page (chunk partials merged into the final output);
// Strata round-9 page, section "R9-gpu-11" (accumulators, maxima and
// denominators are the partials; the softmax merge order is fixed).
//
// Lane l owns head dimensions [4l, 4l + 4): one 16-byte load per chunk and
// lane, a 1 KB coalesced row per wave.  Rows with at most four chunks are
// merged four rows per wave with every load in flight (merge_few_kernel);
// rows with up to eight get one wave each and rows with more are split over
// the four waves of a workgroup (merge_kernel).  The first batch of
// accumulator rows is requested before the maximum over the chunk maxima is
// known, so a short merge costs one round trip to memory.  Wave sums are
// added in a fixed order through LDS, which keeps the result deterministic.
#include "sda_internal.h"

namespace sda {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));


// KW = waves that share one row's chunks.  KW = 4: workgroup = one (instance,
// row), wave w takes chunks c = w (mod 4) (long merges).  KW = 1: workgroup =
// four rows of one instance, one wave per row (short merges, where a row has
// only a few chunks and splitting them would leave waves idle).  KB =
// accumulator rows each wave requests at once (a row of up to KW * KB chunks
// is one round trip); the chunk order of the sums does not depend on it.
template <int KW, int KB>
__global__ __launch_bounds__(256) void merge_kernel(Params p) {
    constexpr int kBatch = KB;
    __shared__ v4f part_o[KW > 1 ? KW - 1 : 1][64];
    __shared__ float part_l[KW > 1 ? KW - 1 : 1];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x;  // instance (x: the grid dimension without a 64K limit)
    const int r = KW == 1 ? 4 * blockIdx.y + wave : blockIdx.y;
    const int share = KW == 1 ? 0 : wave;
    const int R = p.n_rows;
    if (KW == 1 && r >= R) return;
    const int n = count_of(p, i);
    const int nch = (n + p.chunk - 1) / p.chunk;
    const int64_t row0 = (int64_t)i * p.n_chunks * R + r;  // chunk c of this row: row0 + c * R
    const float *acc_l = p.acc + row0 * kDim + 4 * lane;

    // Loads are issued for clamped chunk ids (always inside this instance's
    // partials) and chunks past the end get weight 0, so no load is behind a
    // branch.
    v4f a[kBatch];
    float mc[kBatch], lc[kBatch];
    auto load_batch = [&](int c0) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int c = c0 + KW * k;
            const int64_t e = (int64_t)(c < nch ? c : nch - 1) * R;
            a[k] = *reinterpret_cast<const v4f *>(acc_l + e * kDim);
            const float m = p.m[row0 + e];
            mc[k] = c < nch ? m : -INFINITY;
            lc[k] = p.l[row0 + e];
        }
    };

    float M = -INFINITY, L = 0.f;
    v4f o = (v4f){0.f, 0.f, 0.f, 0.f};
    if (share < nch) {
        load_batch(share);  // in flight while the maximum is formed
        for (int c = lane; c < nch; c += 64) M = fmaxf(M, p.m[row0 + (int64_t)c * R]);
        M = wave_max(M);
        for (int c0 = share;;) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                // a chunk with no unmasked cell (m = -inf) has weight 0
                const float w = merge_weight(mc[k], M);
                L = fmaf(lc[k], w, L);
                o = merge_acc(o, w, a[k]);
            }
            c0 += KW * kBatch;
            if (c0 >= nch) break;
            load_batch(c0);
        }
    }

    if (KW > 1) {
        if (wave > 0) {
            part_o[wave - 1][lane] = o;
            if (lane == 0) part_l[wave - 1] = L;
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < KW - 1; ++w) {
            o += part_o[w][lane];
            L += part_l[w];
        }
    }
    v4f *out = reinterpret_cast<v4f *>(p.out + ((int64_t)i * R + r) * kDim) + lane;
    if (!(L > 0.f)) {  // no unmasked cell in any chunk
        *out = (v4f){0.f, 0.f, 0.f, 0.f};
        if (lane == 0) p.lse[(int64_t)i * R + r] = -INFINITY;
        return;
    }
    *out = o * (1.f / L);
    if (lane == 0) p.lse[(int64_t)i * R + r] = M + logf(L);
}

// Rows of at most NC chunks: each wave merges kRowsPerWave rows (workgroup =
// 4 waves = 16 rows of one instance) and issues every load of its rows at
// once, so a merge of a few partials per row is one round trip for a quarter
// of the waves.  Per row the arithmetic is merge_kernel<1>'s, chunk by chunk.
constexpr int kRowsPerWave = 4;

template <int NC>
__global__ __launch_bounds__(256) void merge_few_kernel(Params p) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x;
    const int R = p.n_rows;
    const int r0 = (4 * blockIdx.y + wave) * kRowsPerWave;
    if (r0 >= R) return;
    const int n = count_of(p, i);
    const int nch = (n + p.chunk - 1) / p.chunk;  // at most NC here
    v4f a[kRowsPerWave][NC];
    float mc[kRowsPerWave][NC], lc[kRowsPerWave][NC];
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
        const int r = r0 + q < R ? r0 + q : R - 1;  // rows past the end: loaded, not stored
        const int64_t row0 = (int64_t)i * p.n_chunks * R + r;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c < nch) {  // uniform across the workgroup
                a[q][c] = *reinterpret_cast<const v4f *>(p.acc + (row0 + (int64_t)c * R) * kDim +
                                                         4 * lane);
                mc[q][c] = p.m[row0 + (int64_t)c * R];
                lc[q][c] = p.l[row0 + (int64_t)c * R];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
        if (r0 + q >= R) break;
        float M = -INFINITY, L = 0.f;
        v4f o = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c < nch) M = fmaxf(M, mc[q][c]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c < nch) {
                const float w = merge_weight(mc[q][c], M);
                L = fmaf(lc[q][c], w, L);
                o = merge_acc(o, w, a[q][c]);
            }
        }
        const int64_t u = (int64_t)i * R + r0 + q;
        v4f *out = reinterpret_cast<v4f *>(p.out + u * kDim) + lane;
        if (!(L > 0.f)) {  // no unmasked cell in any chunk
            *out = (v4f){0.f, 0.f, 0.f, 0.f};
            if (lane == 0) p.lse[u] = -INFINITY;
        } else {
            *out = o * (1.f / L);
            if (lane == 0) p.lse[u] = M + logf(L);
        }
    }
}

}  // namespace

hipError_t launch_merge(const Params &p, hipStream_t s) {
    if (p.n_chunks <= 2) {
        merge_few_kernel<2><<<dim3(p.n_inst, (p.n_rows + 15) / 16), dim3(256), 0, s>>>(p);
        return hipGetLastError();
    }
    if (p.n_chunks <= 4) {
        merge_few_kernel<4><<<dim3(p.n_inst, (p.n_rows + 15) / 16), dim3(256), 0, s>>>(p);
        return hipGetLastError();
    }
    // rows with more than eight chunks split them over four waves, each
    // requesting its share at once (up to 48 chunks in one round trip)
    const dim3 long_grid(p.n_inst, p.n_rows);
    if (p.n_chunks > 32)
        merge_kernel<4, 12><<<long_grid, dim3(256), 0, s>>>(p);
    else if (p.n_chunks > 16)
        merge_kernel<4, 8><<<long_grid, dim3(256), 0, s>>>(p);
    else if (p.n_chunks > 8)
        merge_kernel<4, 4><<<long_grid, dim3(256), 0, s>>>(p);
    else
        merge_kernel<1, 8><<<dim3(p.n_inst, (p.n_rows + 3) / 4), dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace sda
