// QSA block scoring and top-k selection: the step that produces the
// selected cell list the chunk pass reads.
//
// Source: Strata round-9 page, section "R9-gpu-9: QSA_ROWS at five and six
// queries" (a block scorer over pooled block keys, dead flags, indexer
// queries and per-row extents, for a few query rows; its tests compare the
// scores and the selected ids), and section "R9-gpu-8" (the top-k that
// follows).  The arithmetic is this library's reading of them:
//   score[r][b] = sum over indexer heads h of q_idx[r][h] . pooled[b][h],
//                 -inf if block b is dead or b * R >= n_visible[r];
//   selection   = the k blocks with the highest max_r score[r][b], equal
//                 scores in increasing block order, -inf never; their cells
//                 below max_r n_visible[r], in increasing order.
//
// qsa_scores_kernel: a memory-bound product of each block's pooled key (one
// fp32 vector of n_heads * idx_dim) with the rows' queries.  Sixteen lanes
// share a block: each loads 16 consecutive bytes of every 256-byte slab of
// the key (one coalesced 256-byte segment per load instruction), multiplies
// them with the rows' matching query values (held in LDS, read as
// broadcasts), and the 16 partial sums of a row meet through lane swaps.
// Blocks no row can use (dead, or past every row's extent) are not read.
//
// qsa_select_kernel: one workgroup per instance, or up to eight in grids
// of fewer than 256 instances, each computing the same selection and
// writing its share of the cell list (with one workgroup per instance the
// writes took a quarter of the kernel's time).  The scores are loaded a few
// blocks per thread at a time, all rows at once, and become
// order-preserving 32-bit keys in LDS (0 for -inf); a radix select over
// four 8-bit digits (a 256-bin histogram per digit, the digit found by a
// suffix scan across one wave) gives the key of the k-th largest block and
// how many blocks with exactly that key are taken; a scan in block order
// then marks the selected blocks (all larger keys, and the first of the
// equal ones), a second scan gives each its offset in the cell list, and
// each wave writes the cells of one block at a time with coalesced stores.
#include <algorithm>

#include "sda_internal.h"

namespace sda {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kScoreThreads = 256;        // 16 lanes per block, 16 blocks at a time
// blocks per workgroup: one per 16 lanes, so that a workgroup makes one
// pass and the grid is as wide as the blocks (64 blocks per workgroup,
// four passes, took 19.8 against 17.3 us at 64 x 512 blocks)
constexpr int kScoreBlocksPerGroup = kScoreThreads / 16;
constexpr int kSelectThreads = 256;
constexpr int kKeyBatch = 4;  // blocks per thread whose scores are loaded together

// Sum over the 16 lanes of a row of lanes (xor swaps within the row).
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 8, 16);
    return x;
}

template <int NR>
__global__ __launch_bounds__(kScoreThreads) void qsa_scores_kernel(QsaParams p) {
    extern __shared__ __attribute__((aligned(16))) float q_s[];  // [NR][hd]
    const int i = blockIdx.y;
    const int hd = p.hd;
    const int slabs = hd / 64;
    // the rows' queries into LDS (rows past n_rows as zeros)
    for (int e = threadIdx.x; e < NR * hd; e += kScoreThreads) {
        const int r = e / hd;
        q_s[e] = r < p.n_rows ? p.q_idx[((int64_t)i * p.n_rows + r) * hd + (e - r * hd)] : 0.f;
    }
    __syncthreads();
    int vis[NR];
    int vmax = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        vis[r] = r < p.n_rows ? p.n_visible[(int64_t)i * p.n_rows + r] : 0;
        vmax = max(vmax, vis[r]);
    }
    const int j = threadIdx.x & 15;         // lane within the block's 16
    const int grp = threadIdx.x >> 4;       // which of the 16 blocks in flight
    const int b0 = blockIdx.x * kScoreBlocksPerGroup;
    for (int bb = grp; bb < kScoreBlocksPerGroup; bb += kScoreThreads / 16) {
        const int b = b0 + bb;
        if (b >= p.max_blocks) break;
        const bool dead = p.dead[(int64_t)i * p.max_blocks + b] != 0;
        const int64_t first = (int64_t)b * p.block_cells;
        float acc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = 0.f;
        if (!dead && first < vmax) {  // a block no row can use is not read
            const float *key = p.pooled + ((int64_t)i * p.max_blocks + b) * hd + 4 * j;
            for (int s = 0; s < slabs; ++s) {
                const v4f k = *reinterpret_cast<const v4f *>(key + 64 * s);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const v4f qv = *reinterpret_cast<const v4f *>(&q_s[r * hd + 64 * s + 4 * j]);
                    acc[r] = fmaf(k[0], qv[0], acc[r]);
                    acc[r] = fmaf(k[1], qv[1], acc[r]);
                    acc[r] = fmaf(k[2], qv[2], acc[r]);
                    acc[r] = fmaf(k[3], qv[3], acc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float s = sum16(acc[r]);
            if (j == r && r < p.n_rows)
                p.scores[((int64_t)i * p.n_rows + r) * p.max_blocks + b] =
                    (!dead && first < vis[r]) ? s : -INFINITY;
        }
    }
}

// Order-preserving key of a combined score: larger score, larger key;
// -inf (and anything not above it) 0; -0 and +0 the same key.
__device__ __forceinline__ unsigned key_of(float c) {
    if (!(c > -INFINITY)) return 0u;
    const unsigned u = __float_as_uint(c + 0.f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one value per thread over the workgroup (in thread
// order); returns this thread's prefix and the total through *total.
__device__ __forceinline__ int block_scan(int v, int *part, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) part[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelectThreads / 64; ++w) {
        const int pw = part[w];
        base += w < wave ? pw : 0;
        all += pw;
    }
    __syncthreads();
    *total = all;
    return base + x - v;
}

__global__ __launch_bounds__(kSelectThreads) void qsa_select_kernel(QsaParams p) {
    __shared__ unsigned keys[kQsaMaxBlocks];
    __shared__ int hist[256];
    __shared__ int sel_block[kQsaMaxK], sel_off[kQsaMaxK];
    __shared__ int part[kSelectThreads / 64];
    __shared__ int pick[2];  // digit found, rank left
    const int i = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int B = p.max_blocks;
    // The loads below take clamped indices (a row past n_rows reads the last
    // row again, a block past B block B - 1; neither changes a maximum), so
    // that none is conditional and all are in flight at once.
    const int last_row = p.n_rows - 1;
    // combined scores as keys, kKeyBatch blocks per thread at a time; live
    // blocks counted
    const float *sc = p.scores + (int64_t)i * p.n_rows * B;
    auto load = [&](int b0, float (&c)[kKeyBatch]) {
#pragma unroll
        for (int k = 0; k < kKeyBatch; ++k) c[k] = -INFINITY;
#pragma unroll
        for (int r = 0; r < kQsaMaxRows; ++r)
#pragma unroll
            for (int k = 0; k < kKeyBatch; ++k)
                c[k] = fmaxf(c[k], sc[(int64_t)min(r, last_row) * B +
                                      min(b0 + k * kSelectThreads, B - 1)]);
    };
    int live = 0;
    auto put = [&](int b0, const float (&c)[kKeyBatch]) {
#pragma unroll
        for (int k = 0; k < kKeyBatch; ++k) {
            const int b = b0 + k * kSelectThreads;
            if (b < B) {
                const unsigned key = key_of(c[k]);
                keys[b] = key;
                live += key != 0u;
            }
        }
    };
    float c0[kKeyBatch];
    load(tid, c0);
    // lane r < n_rows: row r's extent (loaded beside the first scores, used
    // after the keys)
    int nv = p.n_visible[(int64_t)i * p.n_rows + min(lane, last_row)];
    put(tid, c0);
    for (int b0 = tid + kKeyBatch * kSelectThreads; b0 < B; b0 += kKeyBatch * kSelectThreads) {
        float c[kKeyBatch];
        load(b0, c);
        put(b0, c);
    }
    // the largest over lanes 0..7 (rows past n_rows repeat the last row)
#pragma unroll
    for (int d = 1; d < kQsaMaxRows; d <<= 1) nv = max(nv, __shfl_xor(nv, d, kQsaMaxRows));
    const int64_t extent = min((int64_t)max(__shfl(nv, 0), 0), (int64_t)B * p.block_cells);
    int n_live;
    (void)block_scan(live, part, &n_live);  // (also orders the key writes before the reads below)
    const int kk = min(p.k_blocks, n_live);

    // radix select: the key T of the kk-th largest, and how many keys equal
    // to T are taken (rank, 1..count(T))
    unsigned prefix = 0;
    int rank = kk;
    for (int pass = 0; pass < 4 && kk > 0; ++pass) {
        const int shift = 24 - 8 * pass;
        const unsigned hi_mask = pass == 0 ? 0u : ~0u << (shift + 8);
        for (int d = tid; d < 256; d += kSelectThreads) hist[d] = 0;
        __syncthreads();
        for (int b = tid; b < B; b += kSelectThreads) {
            const unsigned k = keys[b];
            if (k != 0u && (k & hi_mask) == (prefix & hi_mask))
                atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255 - 4l .. 252 - 4l, high to low; suffix
            // sums over the lanes give, for each digit, the count of keys
            // with a larger digit
            int h[4], s = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = hist[255 - 4 * lane - e];
                s += h[e];
            }
            int x = s;  // inclusive scan from lane 0 (digit 255) upwards
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(x, d);
                if (lane >= d) x += y;
            }
            int above = x - s;  // keys with a digit larger than this lane's first
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (above < rank && rank <= above + h[e]) {
                    pick[0] = 255 - 4 * lane - e;
                    pick[1] = rank - above;
                }
                above += h[e];
            }
        }
        __syncthreads();
        prefix |= (unsigned)pick[0] << shift;
        rank = pick[1];
        __syncthreads();
    }
    const unsigned T = prefix;

    // this thread's contiguous range of blocks; marks in block order
    const int per = (B + kSelectThreads - 1) / kSelectThreads;
    const int lo = min(tid * per, B), hi = min(lo + per, B);
    int n_eq = 0;
    for (int b = lo; b < hi; ++b) n_eq += (kk > 0 && keys[b] == T);
    int total;
    int eq_before = block_scan(n_eq, part, &total);
    int n_sel_blocks = 0, n_cells = 0;
    for (int b = lo; b < hi; ++b) {
        const unsigned k = keys[b];
        bool s = false;
        if (kk > 0 && k > T) s = true;
        if (kk > 0 && k == T) s = eq_before++ < rank;
        const int64_t c0 = (int64_t)b * p.block_cells;
        const int cnt = s ? (int)max((int64_t)0, min((int64_t)p.block_cells, extent - c0)) : 0;
        keys[b] = s ? 1u : 0u;  // from here on: selected or not
        n_sel_blocks += s;
        n_cells += cnt;
    }
    int blocks_total, cells_total;
    int slot = block_scan(n_sel_blocks, part, &blocks_total);
    int off = block_scan(n_cells, part, &cells_total);
    // (the selection has exactly min(k, live) blocks; the bounds below only
    // keep every store inside its array whatever the scores hold)
    for (int b = lo; b < hi; ++b) {
        if (keys[b] == 0u) continue;
        const int64_t c0 = (int64_t)b * p.block_cells;
        const int cnt = (int)max((int64_t)0, min((int64_t)p.block_cells, extent - c0));
        if (slot < kQsaMaxK) {
            sel_block[slot] = b;
            sel_off[slot] = off;
        }
        ++slot;
        off += cnt;
    }
    __syncthreads();
    // cells of each selected block, one block per wave at a time: four
    // consecutive cells per lane in one 16-byte store where the block's
    // place in the list is 16-byte aligned and it lies wholly inside the
    // list, single cells otherwise
    int32_t *out = p.sel + (int64_t)i * p.sel_stride;
    const bool base_aligned = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    const int split = gridDim.y;  // workgroups sharing this instance's writes
    for (int s = wave + (kSelectThreads / 64) * blockIdx.y; s < min(blocks_total, kQsaMaxK);
         s += (kSelectThreads / 64) * split) {
        const int b = sel_block[s];
        const int off = sel_off[s];
        const int64_t c0 = (int64_t)b * p.block_cells;
        const int cnt = (int)max((int64_t)0, min((int64_t)p.block_cells, extent - c0));
        if (base_aligned && (off & 3) == 0 && (cnt & 3) == 0 && off + (int64_t)cnt <= p.sel_stride) {
            for (int c = 4 * lane; c < cnt; c += 256) {
                const int v = (int)(c0 + c);
                *reinterpret_cast<int4 *>(out + off + c) = make_int4(v, v + 1, v + 2, v + 3);
            }
        } else {
            for (int c = lane; c < cnt; c += 64)
                if (off + (int64_t)c < p.sel_stride) out[off + c] = (int32_t)(c0 + c);
        }
    }
    if (tid == 0 && blockIdx.y == 0) p.n_sel[i] = cells_total;
}

}  // namespace

hipError_t launch_qsa_scores(const QsaParams &p, hipStream_t s) {
    const dim3 grid((p.max_blocks + kScoreBlocksPerGroup - 1) / kScoreBlocksPerGroup, p.n_inst);
    const int nr = p.n_rows <= 1 ? 1 : p.n_rows <= 2 ? 2 : p.n_rows <= 4 ? 4 : 8;
    const size_t lds = (size_t)nr * p.hd * sizeof(float);
    switch (nr) {
        case 1: qsa_scores_kernel<1><<<grid, kScoreThreads, lds, s>>>(p); break;
        case 2: qsa_scores_kernel<2><<<grid, kScoreThreads, lds, s>>>(p); break;
        case 4: qsa_scores_kernel<4><<<grid, kScoreThreads, lds, s>>>(p); break;
        default: qsa_scores_kernel<8><<<grid, kScoreThreads, lds, s>>>(p); break;
    }
    return hipGetLastError();
}

hipError_t launch_qsa_select(const QsaParams &p, hipStream_t s) {
    // grids of fewer than 256 instances: up to eight workgroups per
    // instance (one per CU at this LDS size), each computing the same
    // selection and writing its share of the selected blocks' cells
    const int per_wg = kSelectThreads / 64;
    int split = (int)std::max<int64_t>(1, std::min<int64_t>(8, 256 / std::max(1, p.n_inst)));
    split = std::max(1, std::min(split, (p.k_blocks + per_wg - 1) / per_wg));
    qsa_select_kernel<<<dim3(p.n_inst, split), kSelectThreads, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace sda
