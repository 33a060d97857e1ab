// Chunk pass, plain vector-ALU version (fp32 FMA, LDS-staged tiles).
//
// One workgroup per (chunk, instance).  Per tile of kTile selected cells:
// gather through the page table, stage the INT8 K/V rows and scales in LDS,
// score every (row, cell) pair in fp32, run the online softmax per row in
// base-2 units, and accumulate p * v_scale * v_code into per-row
// accumulators held by the thread that owns each head dimension.  The
// chunk's (acc, m, l) partial is written at the end.
//
// Source: Strata PR #2220 page (chunk kernel: score the grouped query heads
// per selected cell, online softmax, value loop into chunk partials).
#include "sda_internal.h"

namespace sda {
namespace {

constexpr int kTile = 32;
constexpr int kThreads = 256;

template <int RMAX>
__global__ __launch_bounds__(kThreads) void chunk_valu_kernel(Params p) {
    const int c = blockIdx.x;
    const int i = blockIdx.y;
    const int n = count_of(p, i);
    const int j_begin = c * p.chunk;
    if (j_begin >= n) return;  // this instance has fewer chunks
    const int j_end = min(j_begin + p.chunk, n);
    const int R = p.n_rows;
    const int t = threadIdx.x;

    __shared__ int4 k_tile[kTile][kDim / 16];
    __shared__ int4 v_tile[kTile][kDim / 16];
    __shared__ float s_tile[RMAX][kTile];
    __shared__ float p_tile[RMAX][kTile];
    __shared__ int phys[kTile];
    __shared__ float ks[kTile], vs[kTile];
    __shared__ float corr_s[RMAX];

    const int32_t *pt = p.page_table + (int64_t)i * p.pt_stride;
    const int32_t *sel = p.sel + (int64_t)i * p.sel_stride;
    const float *qi = p.q + (int64_t)i * R * kDim;

    float o[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) o[r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;  // owned by threads t < R

    for (int j0 = j_begin; j0 < j_end; j0 += kTile) {
        const int cnt = min(kTile, j_end - j0);
        if (t < kTile) {
            int ph = -1;
            if (t < cnt) {
                ph = gather_cell(p, pt, sel[j0 + t]);
                if (p.gather_out) p.gather_out[(int64_t)i * p.sel_stride + j0 + t] = ph;
            }
            phys[t] = ph;
            ks[t] = ph >= 0 ? half_bits_to_float(p.k_scales[ph]) : 0.f;
            vs[t] = ph >= 0 ? half_bits_to_float(p.v_scales[ph]) : 0.f;
        }
        __syncthreads();
        for (int e = t; e < kTile * (kDim / 16); e += kThreads) {
            const int cell = e / (kDim / 16), part = e % (kDim / 16);
            const int ph = phys[cell];
            int4 kv = make_int4(0, 0, 0, 0), vv = kv;
            if (ph >= 0) {
                kv = reinterpret_cast<const int4 *>(p.k_codes + (int64_t)ph * kDim)[part];
                vv = reinterpret_cast<const int4 *>(p.v_codes + (int64_t)ph * kDim)[part];
            }
            k_tile[cell][part] = kv;
            v_tile[cell][part] = vv;
        }
        __syncthreads();
        // scores in base-2 units
        for (int e = t; e < R * kTile; e += kThreads) {
            const int r = e / kTile, cell = e % kTile;
            float s = -INFINITY;
            if (phys[cell] >= 0) {
                const float4 *qr = reinterpret_cast<const float4 *>(qi + (int64_t)r * kDim);
                const int8_t *kr = reinterpret_cast<const int8_t *>(&k_tile[cell][0]);
                float dot = 0.f;
                for (int d4 = 0; d4 < kDim / 4; ++d4) {
                    const float4 qv = qr[d4];
                    dot = fmaf(qv.x, (float)kr[4 * d4 + 0], dot);
                    dot = fmaf(qv.y, (float)kr[4 * d4 + 1], dot);
                    dot = fmaf(qv.z, (float)kr[4 * d4 + 2], dot);
                    dot = fmaf(qv.w, (float)kr[4 * d4 + 3], dot);
                }
                s = dot * ks[cell] * p.scale_log2;
            }
            s_tile[r][cell] = s;
        }
        __syncthreads();
        // online softmax, one thread per row
        if (t < R) {
            float tmax = -INFINITY;
            for (int cell = 0; cell < kTile; ++cell) tmax = fmaxf(tmax, s_tile[t][cell]);
            const float m_new = fmaxf(m_run, tmax);
            float corr = 1.f, lsum = 0.f;
            if (m_new != -INFINITY) {
                corr = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
                for (int cell = 0; cell < kTile; ++cell) {
                    const float s = s_tile[t][cell];
                    const float pr = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
                    lsum += pr;
                    p_tile[t][cell] = pr * vs[cell];
                }
            } else {
                for (int cell = 0; cell < kTile; ++cell) p_tile[t][cell] = 0.f;
            }
            l_run = l_run * corr + lsum;
            m_run = m_new;
            corr_s[t] = corr;
        }
        __syncthreads();
        // value accumulation, one thread per head dimension
        {
            const int d = t;
#pragma unroll
            for (int r = 0; r < RMAX; ++r)
                if (r < R) o[r] *= corr_s[r];
            for (int cell = 0; cell < cnt; ++cell) {
                const float v = (float)reinterpret_cast<const int8_t *>(&v_tile[cell][0])[d];
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (r < R) o[r] = fmaf(p_tile[r][cell], v, o[r]);
            }
        }
        __syncthreads();
    }
    const int64_t base = ((int64_t)i * p.n_chunks + c) * R;
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
        if (r < R) p.acc[(base + r) * kDim + t] = o[r];
    if (t < R) {
        // base-2 maximum back to natural-log units
        p.m[base + t] = (m_run == -INFINITY) ? -INFINITY : m_run * 0.69314718055994531f;
        p.l[base + t] = l_run;
    }
}

}  // namespace

hipError_t launch_chunk_valu(const Params &p, hipStream_t s) {
    dim3 grid(p.n_chunks, p.n_inst), block(kThreads);
    if (p.n_rows <= 16)
        chunk_valu_kernel<16><<<grid, block, 0, s>>>(p);
    else if (p.n_rows <= 32)
        chunk_valu_kernel<32><<<grid, block, 0, s>>>(p);
    else if (p.n_rows <= 48)
        chunk_valu_kernel<48><<<grid, block, 0, s>>>(p);
    else
        chunk_valu_kernel<64><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace sda
