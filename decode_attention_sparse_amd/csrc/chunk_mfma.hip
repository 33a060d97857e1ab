// Chunk pass on the gfx950 matrix cores (int8 MFMA with exact digit splits).
//
// Source: Strata PR #2220 page -- per selected cell, score the grouped query
// heads that share the KV head, run an online softmax, accumulate the INT8 V
// rows into the chunk partial (running max, denominator, accumulator).  The
// page's CUDA kernels (shared-memory query slices, 32-lane warp reductions,
// cell-major probabilities) are prior art; this kernel is laid out for
// CDNA4 wave64 matrix cores instead.
//
// Workgroup = one (chunk, instance), RB = ceil(rows / 16) waves; wave w owns
// query rows [16w, 16w + 16) for the whole chunk, so every softmax statistic
// of a row lives in one wave.  Cells are processed in tiles of 64.
//
// Exactness of the contractions.  The INT8 codes are used as they are; the
// fp32 operands are split into int8 digits so that the int8 MFMA (exact
// int32 accumulation) reproduces fp32-accurate products:
//   QK  q_r[d] = sigma_r * (a + b/2^8 + c/2^16), sigma_r = max|q_r| / 127,
//       a in [-127,127], b, c in [-128,127] (round-to-nearest digits with
//       carry); S = sigma_r * ((2^8 A + B) / 2^8 + C / 2^16) where A, B, C
//       are the exact integer dot products of the digits with the K codes
//       (2^8 A + B is accumulated in one int32 register: the A products are
//       shifted left by 8 between the two MFMA groups; |2^8 A + B| < 2^30).
//   PV  p'_rj = p_rj * v_scale_j in [0, max], split per tile and row as
//       tau * (a + b/2^8), tau = tile max / 127, a in [0,127], b in
//       [-128,127]; the tile's (2^8 A + B) int32 sums are converted once and
//       folded into the fp32 accumulator with the online-softmax correction.
// The q split keeps 23 significant bits (fp32-level); the probability split
// keeps 15 bits relative to the tile's largest weighted probability.
//
// Data movement.  Each tile's 64 K rows and 64 V rows (256 B each) go from
// HBM straight into LDS with global_load_lds (16 B per lane, no VGPR hop),
// double-buffered so that tile t+1 is in flight while tile t computes.  K
// rows are read back with ds_read_b128 as the A operand of S^T = K Q^T; V
// rows are read back transposed with ds_read_b64_tr_b8 as the A operand of
// O^T = V^T P^T.  16-byte chunks are XOR-swizzled per row to spread banks.
// The page-table gather (selected id -> physical cell) and the scale loads
// run once per segment of up to 512 cells into LDS.
#include "sda_internal.h"

namespace sda {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kTile = 64;      // cells per tile (the K extent of one PV MFMA)
constexpr int kSeg = 512;      // cells gathered into LDS at a time
constexpr int kRow = kDim;     // bytes per code row

// physical 16-byte chunk of logical chunk x in code row c of a tile
__device__ __forceinline__ int swz_k(int c) { return c & 7; }
__device__ __forceinline__ int swz_v(int c) { return (c & 3) | ((c >> 2) & 4); }

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max4(float x) {  // over lanes l, l^16, l^32, l^48
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_sum4(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Stage tile `t` (segment-relative) of K and V code rows into LDS buffer
// `b`.  32 instructions of 1 KB (4 rows each), dealt round-robin to waves.
template <int RB>
__device__ __forceinline__ void issue_tile(const Params &p, const int *phys_s, int t,
                                           int8_t *kb, int8_t *vb, int wave,
                                           int lane) {
#pragma unroll
    for (int it = 0; it < (32 + RB - 1) / RB; ++it) {
        const int k = wave + it * RB;
        if (k >= 32) break;
        const int kk = k & 15;
        const int row = 4 * kk + (lane >> 4);
        int ph = phys_s[t * kTile + row];
        ph = ph < 0 ? 0 : ph;  // masked: any valid row, its score is -inf
        const bool is_v = k >= 16;
        const int lc = (lane & 15) ^ (is_v ? swz_v(row) : swz_k(row));
        const int8_t *src = (is_v ? p.v_codes : p.k_codes) + (int64_t)ph * kRow + lc * 16;
        int8_t *dst = (is_v ? vb : kb) + kk * 1024;
        __builtin_amdgcn_global_load_lds((const void *)src, (void LDS_AS *)(dst), 16, 0, 0);
    }
}

template <int RB>
__global__ __launch_bounds__(64 * RB) void chunk_mfma_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) int8_t kbuf[2][kTile * kRow];
    __shared__ __attribute__((aligned(16))) int8_t vbuf[2][kTile * kRow];
    __shared__ __attribute__((aligned(16))) int phys_s[kSeg];
    __shared__ __attribute__((aligned(16))) float ks_s[kSeg];
    __shared__ __attribute__((aligned(16))) float vs_s[kSeg];
    __shared__ __attribute__((aligned(16))) float bias_s[kSeg];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;     // lane group: k-set of the MFMA operands
    const int l16 = lane & 15;   // row (of this wave's 16) owned by this lane
    const int c = blockIdx.x;
    const int i = blockIdx.y;
    const int n = count_of(p, i);
    const int j_begin = c * p.chunk;
    if (j_begin >= n) return;  // this instance has fewer chunks
    const int j_end = min(j_begin + p.chunk, n);
    const int R = p.n_rows;
    const int row = wave * 16 + l16;
    const int32_t *pt = p.page_table + (int64_t)i * p.pt_stride;
    const int32_t *sel = p.sel + (int64_t)i * p.sel_stride;

    // ---- query digits: B operands of S^T = K Q^T for rows 16*wave + l16,
    // dims 64s + 16g + e (byte e of slab s)
    v4i qa[4], qb[4], qc[4];
    float coef_q;  // sigma_r * scale_log2 / 2^8
    {
        float qv[4][16];
        float mx = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                v4f v = {0.f, 0.f, 0.f, 0.f};
                if (row < R)
                    v = *reinterpret_cast<const v4f *>(p.q + ((int64_t)i * R + row) * kDim +
                                                       64 * s + 16 * g + 4 * e4);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    qv[s][4 * e4 + u] = v[u];
                    mx = fmaxf(mx, fabsf(v[u]));
                }
            }
        }
        mx = wave_max4(mx);
        const float inv = mx > 0.f ? 127.f / mx : 0.f;
        coef_q = (mx / 127.f) * p.scale_log2 * (1.f / 256.f);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                unsigned pa = 0, pb = 0, pc = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x = qv[s][4 * w + u] * inv;
                    float a = rintf(x);
                    const float r1 = (x - a) * 256.f;
                    float b = rintf(r1);
                    float cc = rintf((r1 - b) * 256.f);
                    if (cc > 127.f) { cc -= 256.f; b += 1.f; }
                    if (b > 127.f) { b -= 256.f; a += 1.f; }
                    pa |= ((unsigned)(int)a & 0xffu) << (8 * u);
                    pb |= ((unsigned)(int)b & 0xffu) << (8 * u);
                    pc |= ((unsigned)(int)cc & 0xffu) << (8 * u);
                }
                qa[s][w] = (int)pa;
                qb[s][w] = (int)pb;
                qc[s][w] = (int)pc;
            }
        }
    }

    float m_run = -INFINITY;  // running max of this lane's row (base-2 units)
    float l_part = 0.f;       // this lane's share of the row denominator
    v4f o[16];                // O^T[16db + 4g + u][row]
#pragma unroll
    for (int db = 0; db < 16; ++db) o[db] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int seg0 = j_begin; seg0 < j_end; seg0 += kSeg) {
        const int seg_cnt = min(kSeg, j_end - seg0);
        const int seg_tiles = (seg_cnt + kTile - 1) / kTile;
        __syncthreads();  // LDS of the previous segment no longer read
        {
            // batched gather: all selected ids, then all page-table entries,
            // then all scales, so each thread waits for three round trips
            constexpr int kPer = (kSeg + 64 * RB - 1) / (64 * RB);
            const int lim = seg_tiles * kTile;
            int ids[kPer], ph[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int jj = threadIdx.x + k * 64 * RB;
                ids[k] = (jj < seg_cnt) ? sel[seg0 + jj] : -1;
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) ph[k] = gather_cell(p, pt, ids[k]);
            uint16_t kh[kPer], vh[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int q0 = ph[k] < 0 ? 0 : ph[k];
                kh[k] = p.k_scales[q0];
                vh[k] = p.v_scales[q0];
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int jj = threadIdx.x + k * 64 * RB;
                if (jj < lim) {
                    const bool ok = ph[k] >= 0;
                    phys_s[jj] = ph[k];
                    ks_s[jj] = ok ? half_bits_to_float(kh[k]) : 0.f;
                    vs_s[jj] = ok ? half_bits_to_float(vh[k]) : 0.f;
                    bias_s[jj] = ok ? 0.f : -INFINITY;
                    if (p.gather_out && jj < seg_cnt)
                        p.gather_out[(int64_t)i * p.sel_stride + seg0 + jj] = ph[k];
                }
            }
        }
        __syncthreads();
        issue_tile<RB>(p, phys_s, 0, kbuf[0], vbuf[0], wave, lane);

        for (int t = 0; t < seg_tiles; ++t) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile t staged by every wave; tile t-1 no longer read
            if (t + 1 < seg_tiles)
                issue_tile<RB>(p, phys_s, t + 1, kbuf[(t + 1) & 1], vbuf[(t + 1) & 1], wave,
                               lane);
            const int8_t *kb = kbuf[t & 1];
            const int8_t *vb = vbuf[t & 1];
            const int cb0 = t * kTile + 4 * g;  // this lane's first cell in the segment arrays

            // ---- scores S^T[cell = 16cb + 4g + u][row], base-2 units
            v4f sc[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int cell = 16 * cb + l16;
                v4i ka[4];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    ka[s] = *reinterpret_cast<const v4i *>(
                        kb + cell * kRow + (((4 * s + g) ^ swz_k(cell)) << 4));
                v4i ab = {0, 0, 0, 0}, cc = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < 4; ++s) ab = mfma_i8(ka[s], qa[s], ab);
                ab = ab << 8;
#pragma unroll
                for (int s = 0; s < 4; ++s) ab = mfma_i8(ka[s], qb[s], ab);
#pragma unroll
                for (int s = 0; s < 4; ++s) cc = mfma_i8(ka[s], qc[s], cc);
                const v4f ks = *reinterpret_cast<const v4f *>(&ks_s[cb0 + 16 * cb]);
                const v4f bs = *reinterpret_cast<const v4f *>(&bias_s[cb0 + 16 * cb]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float tq = fmaf((float)cc[u], 1.f / 256.f, (float)ab[u]);
                    sc[cb][u] = fmaf(tq, ks[u] * coef_q, bs[u]);
                }
            }

            // ---- online softmax (row max over the tile: 16 cells here, 4 lane groups)
            float tmax = -INFINITY;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int u = 0; u < 4; ++u) tmax = fmaxf(tmax, sc[cb][u]);
            tmax = wave_max4(tmax);
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            float psum = 0.f, pmax = 0.f;
            v4f pw[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const v4f vs = *reinterpret_cast<const v4f *>(&vs_s[cb0 + 16 * cb]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float pr = __builtin_amdgcn_exp2f(sc[cb][u] - m_use);
                    psum += pr;
                    pw[cb][u] = pr * vs[u];
                    pmax = fmaxf(pmax, pw[cb][u]);
                }
            }
            l_part = fmaf(l_part, corr, psum);
            pmax = wave_max4(pmax);
            const float inv_tau = pmax > 0.f ? 127.f / pmax : 0.f;
            const float tau2 = pmax * (1.f / (127.f * 256.f));

            // ---- probability digits: byte e = 4cb + u <-> cell 16cb + 4g + u
            v4i pa, pb;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                unsigned wa = 0, wb = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float x = pw[cb][u] * inv_tau;
                    const float a = rintf(x);
                    const float b = fminf(rintf(fmaf(x - a, 256.f, 128.f)), 255.f);
                    wa |= (unsigned)a << (8 * u);
                    wb |= (unsigned)b << (8 * u);
                }
                pa[cb] = (int)wa;
                pb[cb] = (int)(wb ^ 0x80808080u);  // offset-128 bytes -> signed digits
            }

            // ---- O^T += V^T P^T for 16 blocks of 16 dims
            const int tb = l16 >> 1, th = l16 & 1;  // source role in the transposed read
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                v4i va;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int e = 8 * r + tb;
                    const int cell = ((e >> 2) << 4) + 4 * g + (e & 3);
                    const int8_t *src = vb + cell * kRow + ((db ^ swz_v(cell)) << 4) + 8 * th;
                    const v2i h = __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i LDS_AS *)(src));
                    va[2 * r] = h[0];
                    va[2 * r + 1] = h[1];
                }
                v4i acc = mfma_i8(va, pa, (v4i){0, 0, 0, 0});
                acc = acc << 8;
                acc = mfma_i8(va, pb, acc);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[db][u] = fmaf((float)acc[u], tau2, o[db][u] * corr);
            }
        }
    }

    const float l_row = wave_sum4(l_part);
    if (row < R) {
        const int64_t base = ((int64_t)i * p.n_chunks + c) * R + row;
        float *dst = p.acc + base * kDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 16; ++db) *reinterpret_cast<v4f *>(dst + 16 * db) = o[db];
        if (g == 0) {
            // base-2 maximum back to natural-log units
            p.m[base] = (m_run == -INFINITY) ? -INFINITY : m_run * 0.69314718055994531f;
            p.l[base] = l_row;
        }
    }
}

}  // namespace

hipError_t launch_chunk(const Params &p, hipStream_t s) {
    dim3 grid(p.n_chunks, p.n_inst);
    const int rb = (p.n_rows + 15) / 16;
    switch (rb) {
        case 1: chunk_mfma_kernel<1><<<grid, 64, 0, s>>>(p); break;
        case 2: chunk_mfma_kernel<2><<<grid, 128, 0, s>>>(p); break;
        case 3: chunk_mfma_kernel<3><<<grid, 192, 0, s>>>(p); break;
        default: chunk_mfma_kernel<4><<<grid, 256, 0, s>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace sda
