// Merge pass: log-sum-exp combination of the chunk partials of one
// (instance, query row) into the head output and its log-sum-exp.
//
// Source: Strata PR #2220 page (chunk partials merged into the final output);
// Strata round-9 page, section "R9-gpu-11" (accumulators, maxima and
// denominators are the partials; the softmax merge order is fixed).
//
// One workgroup of 256 threads per (row, instance); thread d owns head
// dimension d.  The chunk maxima and denominators are read by every thread
// (same address, served as a broadcast), the accumulators once each,
// coalesced along d.
#include "sda_internal.h"

namespace sda {
namespace {

__global__ __launch_bounds__(kDim) void merge_kernel(Params p) {
    const int r = blockIdx.x;
    const int i = blockIdx.y;
    const int d = threadIdx.x;
    const int R = p.n_rows;
    const int n = count_of(p, i);
    const int nch = (n + p.chunk - 1) / p.chunk;
    const int64_t row0 = (int64_t)i * p.n_chunks * R + r;  // chunk c at row0 + c*R
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, p.m[row0 + (int64_t)c * R]);
    float *o = p.out + ((int64_t)i * R + r) * kDim;
    if (M == -INFINITY) {
        o[d] = 0.f;
        if (d == 0) p.lse[(int64_t)i * R + r] = -INFINITY;
        return;
    }
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < nch; ++c) {
        const float mc = p.m[row0 + (int64_t)c * R];
        if (mc == -INFINITY) continue;  // chunk with no unmasked cell
        const float w = expf(mc - M);
        L = fmaf(p.l[row0 + (int64_t)c * R], w, L);
        acc = fmaf(p.acc[(row0 + (int64_t)c * R) * kDim + d], w, acc);
    }
    o[d] = acc / L;
    if (d == 0) p.lse[(int64_t)i * R + r] = M + logf(L);
}

}  // namespace

hipError_t launch_merge(const Params &p, hipStream_t s) {
    dim3 grid(p.n_rows, p.n_inst), block(kDim);
    merge_kernel<<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace sda
