// Chunk pass on the gfx950 matrix cores (int8 MFMA with exact digit splits).
//
// Source: Strata PR #2220 page -- per selected cell, score the grouped query
// heads that share the KV head, run an online softmax, accumulate the INT8 V
// rows into the chunk partial (running max, denominator, accumulator).  The
// page's CUDA kernels (shared-memory query slices, 32-lane warp reductions,
// cell-major probabilities) are prior art; this kernel is laid out for
// CDNA4 wave64 matrix cores instead.
//
// Workgroup = one (instance, chunk) -- or several consecutive chunks of one
// instance when the grid is large -- with DS * RB + 1 waves: compute wave w
// owns query rows [16 (w / DS), 16 (w / DS) + 16) for the whole chunk (and
// 256 / DS of the head dimensions), so every softmax statistic of a row
// lives in one wave; one more wave is the producer: it runs the gather and
// stages all code rows (the compute waves issue no global loads and hold no
// staging registers).  Cells are processed in tiles of 64.  The compute
// waves' state and per-tile step (RowBlock) are shared by all launches:
//   chunk_mfma_kernel<RB, DS, false>           the pipelined chunk pass below
//                                              (chunk partials);
//   chunk_mfma_kernel<2, 1, false, 2>          the same for two 16-row
//                                              groups, two pipelines (a
//                                              chunk or run of chunks each)
//                                              per workgroup, so that the
//                                              compute waves sit on four
//                                              SIMDs;
//   chunk_mfma_kernel<RB, DS, false, 1, true>  the same for calls with one
//                                              chunk per instance, writing
//                                              the normalised outputs;
//   chunk_mfma_kernel<RB, 1, false, 2, true>   calls with two chunks per
//                                              instance: two pipelines per
//                                              workgroup, merged in LDS;
//   chunk_tile_kernel<RB, DS>                  one-tile chunks in latency-
//                                              bound grids (the tile staged
//                                              at once, no pipeline; a
//                                              workgroup per 16-row group
//                                              in the smallest grids);
//   chunk_mfma_kernel<RB, 1, true>             prompt attention: the
//                                              pipelined pass over an
//                                              implicit causal cell list.
//
// Exactness of the contractions.  The INT8 codes are used as they are; the
// fp32 operands are split into int8 digits so that the int8 MFMA (exact
// int32 accumulation) reproduces fp32-accurate products:
//   QK  q[d] = sigma * (a + b/2^8 + c/2^16), sigma = max |q| over the wave's
//       16 rows / 127, a in [-127,127], b, c in [-128,127] (the nearest
//       multiple of 2^-16 written in balanced base-256 digits).  S = sigma *
//       ((2^8 A + B) / 2^8 + C / 2^16) with A, B, C the exact integer dot
//       products of the digits with the K codes, each accumulated by its own
//       MFMA chain; 2^8 A + B is formed in int32 (|.| < 2^30) before the
//       conversion to fp32.  Score errors are at fp32 level relative to the
//       wave's largest score.
//   PV  x = p * v_scale / tau in [0, 127], tau = (the tile's largest
//       v_scale) / 127 (p <= 1: it is taken against the tile's own maximum,
//       and the factor from there to the running maximum goes with the
//       tile's sums into the accumulator); X = rint(2^16 x) in [0, 127 * 2^16] is
//       written as 2^16 a + 2^8 b + c (a in [0,127], b, c in [-128,127]);
//       the tile's sums over cells of a, b and c times v_code (three MFMAs)
//       are exact in int32, 2^8 A + B is formed in int32 (|.| < 2^29), and
//       2^8 (2^8 A + B) + C is folded into the fp32 accumulator once per
//       tile, the low sum arriving biased (no conversion).  Each weight is
//       represented to 2^-24 of the tile's largest possible weight (its
//       largest V scale), whatever the spread of the V scales across tiles.
//
// Pipeline.  Iteration t of the tile loop computes the scores of tile t+1
// while it runs the softmax and the V accumulation of tile t, so matrix-core
// and vector work of neighbouring tiles interleave within a wave.  Loads run
// ahead of use: selected ids of tile t+4, page-table entries of tile t+3,
// scales and K rows of tile t+2, V rows of tile t+1.  Code rows (256 B) are
// loaded into VGPRs with 16-byte loads (16 lanes per row) and written to LDS
// rows padded to 272 B, double-buffered; the padding and a row permutation
// (lds_row) spread the K and the transposed V reads over the 64 LDS banks,
// with immediate offsets.  K rows feed
// S^T = K Q^T through ds_read_b128; V rows are read transposed with
// ds_read_b64_tr_b8 to feed O^T = V^T P^T.
//
// Online-softmax rescaling without a branch: the accumulator is kept in a
// frame scaled by F = product of the per-tile corrections (O = F * O_frame);
// each tile adds its contribution times 1/F, and the frame is renormalised
// (a wave-uniform, rare branch) only when F drops below 2^-64.
#include "sda_internal.h"

namespace sda {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kTile = 64;            // cells per tile (the K extent of one PV MFMA)
constexpr int kStride = kDim + 16;   // LDS bytes per code row (padded)
constexpr int kBuf = kTile * kStride;
constexpr int kRows = kTile / 4;     // 1 KB staging loads per tile and pool (4 rows each)
constexpr float kRound = 8388608.f;  // 2^23: adding it rounds [0, 2^23) to integers in the low bits
// The low P.V digit leaves the matrix cores biased: its MFMA starts from
// kLoBits (an inline constant: the bits of the float 1/(2 pi)) instead of 0,
// and ends at kLoBits + n, which read as a float is (kLoUnits + n) 2^-26
// exactly for |n| <= 2^21 (the float's binade is [1/8, 1/4) and its mantissa
// field, 2,292,099, is at least 2^21 from both ends), so the sum needs no
// int-to-float conversion; the offset, kLoUnits = 2^23 + 2,292,099 units of
// 2^-26, is taken out once per tile.
constexpr int kLoBits = 0x3E22F983;
constexpr float kLoUnit = 0.15915494f;  // kLoUnits 2^-26, the float kLoBits
constexpr float kTwo26 = 67108864.f;
// The low q.k digit's MFMA chain starts from kMagicBits (1.5 * 2^23 as a
// float): its int32 sum C, |C| <= 256 * 128 * 128 = 2^22, ends at
// kMagicBits + C, which read as a float is 1.5 * 2^23 + C exactly; over 2^8
// that is kScoreOffset + C / 2^8, and the producers store each cell's bias
// less kScoreOffset * k_scale (exact: k_scale has 11 significant bits).
constexpr int kMagicBits = 0x4B400000;
constexpr float kScoreOffset = 49152.f;  // 1.5 * 2^23 / 2^8
constexpr float kRenorm = 5.421010862427522e-20f;  // 2^-64
constexpr int64_t kResidentWorkgroups = 512;        // 256 CUs x 2 workgroups (LDS-limited)
constexpr int64_t kLatencyWorkgroups = 256;         // grids up to one workgroup per CU

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The tile's weight scale, from the producer wave that stages its V scales
// (lane = cell, vsf its V scale, 0 for a masked cell): with vmax the
// largest V scale of the tile, W = 127 * 2^16 / vmax (0 if vmax is 0); cell
// c's slot gets vsf * W (a probability p <= 1 times it is the P.V weight on
// the digit grid, at most 127 * 2^16), and *inv_w gets 1 / W (0 if W is 0).
// Every producer form calls this, so all forms share the bits.
__device__ __forceinline__ void put_v_scales(float *vs_slot, float *inv_w, float vsf, int lane) {
    const float vmax = wave_max(vsf);
    const float W = vmax > 0.f ? (65536.f * 127.f) * __builtin_amdgcn_rcpf(vmax) : 0.f;
    vs_slot[lane] = vsf * W;
    if (lane == 0) *inv_w = vmax * (1.f / (65536.f * 127.f));
}

// Sum over the four lanes l, l^16, l^32, l^48 (one query row), with the
// gfx950 lane swaps (VALU, no LDS round trip); max4 is its maximum.
__device__ __forceinline__ float sum4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS row of the QK operand index 16*cb + l: a permutation within the tile
// (odd cell blocks exchange their two halves of 8 rows) laid out for 64 LDS
// banks of 4 bytes.  With 272-byte rows a row starts 4 banks after the
// previous one, so rows 16 apart share banks: the 16 lanes of a K read take
// 16 consecutive rows (distinct), and the 32 lanes of a transposed V read,
// which take rows from an even and an odd cell block, get rows that differ
// modulo 16.  (Exchanging groups of 4 instead, the layout for 32 banks, had
// twice the prompt kernel's counted bank conflicts.)
__device__ __forceinline__ int lds_row(int cb, int l) { return 16 * cb + (l ^ (8 * (cb & 1))); }

// LDS layout of tiles staged by LDS-DMA loads (the prompt kernel with no
// producer wave): such a load writes 64 lanes x 16 bytes contiguously, so
// one instruction stages 4 code rows.  Tile cell c (block b = c / 4) sits at
// kDmaBlock b + 64 sigma(b) + 256 (c % 4), and its 16-byte granule G
// (bytes 16 G .. 16 G + 15) at slot G ^ (c % 4) of that row.  The blocks'
// shifts sigma spread the rows that one read instruction touches over the 64
// banks: for K reads (16 consecutive cells, one granule) sigma_K(b) = b % 4;
// for the transposed V reads (cells 0-7 and 16-23, or 8-15 and 24-31, of a
// 32-cell half, one granule) sigma_V(b) = (b & 1) | (((b >> 2) & 1) << 1).
constexpr int kDmaBlock = 1280;           // 1 KB of rows and room for the shift
constexpr int kDmaBuf = 16 * kDmaBlock;   // one tile of K or V rows
__host__ __device__ constexpr int dma_sigma_k(int b) { return b & 3; }
__host__ __device__ constexpr int dma_sigma_v(int b) { return (b & 1) | (((b >> 2) & 1) << 1); }
__host__ __device__ constexpr int dma_row_k(int c) {
    return kDmaBlock * (c >> 2) + 64 * dma_sigma_k(c >> 2) + 256 * (c & 3);
}
__host__ __device__ constexpr int dma_row_v(int c) {
    return kDmaBlock * (c >> 2) + 64 * dma_sigma_v(c >> 2) + 256 * (c & 3);
}

// The state of one compute wave: query digits, per-lane LDS offsets, and the
// running softmax statistics and accumulator of its 16 query rows (for the
// head dimensions [256 dh / DS, 256 (dh + 1) / DS) it owns, kDB = 16 / DS
// blocks of 16).  step() is one tile; both kernels run exactly this sequence
// per chunk, so a chunk's partial does not depend on the kernel or launch.
template <int kDB, bool kDma = false>
struct RowBlock {
    // LDS bytes between the K rows of consecutive 16-cell blocks
    static constexpr int kCbStride = kDma ? 4 * kDmaBlock : 16 * kStride;
    v4i qa[4], qb[4], qc[4];  // query digits: B operands of S^T = K Q^T
    float coef;  // sigma * |scale_log2| / 2^8: S (base 2) = coef * (AB + C / 2^8) * k_scale
    int k_off0, k_off1, v_off, m_off0, m_off1;
    int v_offj[kDma ? 4 : 1];  // DMA layout: V read offsets for 16-dim blocks db % 4 = j
    int w_off;     // this pipeline's offset in the arrays of 1 / W (wave-uniform)
    float m_run;   // running max of this lane's row (base-2 units)
    float l_part;  // this lane's share of the row denominator
    float frame;   // O = frame * (o - obias)
    float obias;   // the offset o carries from the biased low P.V digit
    v4f o[kDB];    // O^T[16 (kDB dh + db) + 4g + u][row] / frame + obias
    v4f su[4];     // scores of the tile the softmax runs on next: u, S = coef * u

    // qrow: this lane's query row, read at dims 64s + 16g + e (byte e of
    // slab s); a row past the end (valid false) passes any readable row and
    // gets digits 0.  The loads are unconditional, so all sixteen are in
    // flight at once.  The sign of the softmax scale is folded into the
    // digits so that coef >= 0 and max commutes with it.
    __device__ __forceinline__ void init(const float *qrow, bool valid, float scale_log2, int g,
                                         int l16) {
        v4f qv[4][4];
        float mx = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                qv[s][w] = *reinterpret_cast<const v4f *>(qrow + 64 * s + 16 * g + 4 * w);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fabsf(qv[s][w][u]));
        // a row past the end counts as zeros: out of the maximum, and its
        // digits come out 0 (its values are multiplied by 0)
        mx = wave_max(valid ? mx : 0.f);
        const float inv_row =
            mx > 0.f ? (scale_log2 < 0.f ? -65536.f : 65536.f) * 127.f / mx : 0.f;
        const float inv = valid ? inv_row : 0.f;
        // clamped away from 0 so that masked cells (-inf) never meet a zero factor
        coef = fmaxf((mx / 127.f) * fabsf(scale_log2) * (1.f / 256.f), 1e-30f);
        // X = round(q * 127 * 2^16 / max) = 2^16 a + 2^8 b + c with balanced
        // digits b, c in [-128, 127] (a in [-127, 127]).  Then X + 2^7 =
        // 2^8 (2^8 a + b) + (c + 2^7) and X + 2^7 + 2^15 = 2^16 a + 2^8 (b +
        // 2^7) + (c + 2^7) with the added digits in [0, 255], so the two's
        // complement bytes are c = byte 0 of X, b = byte 1 of X + 2^7 and
        // a = byte 2 of X + 2^7 + 2^15; each operand gathers one such byte
        // of four values (byte permutes).
        auto gather = [](const unsigned (&v)[4], unsigned byte) {
            const unsigned sel = 0x0c0c0400u + byte * 0x0101u;  // bytes 0, 1: v[0], v[1]
            const unsigned lo = __builtin_amdgcn_perm(v[1], v[0], sel);
            const unsigned hi = __builtin_amdgcn_perm(v[3], v[2], sel);
            return (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                unsigned x0[4], x1[4], x2[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int X = (int)rintf(qv[s][w][u] * inv);
                    x0[u] = (unsigned)X;
                    x1[u] = (unsigned)(X + 128);
                    x2[u] = (unsigned)(X + 32896);
                }
                qc[s][w] = gather(x0, 0);
                qb[s][w] = gather(x1, 1);
                qa[s][w] = gather(x2, 2);
            }
        }
        // per-lane constant LDS offsets (everything else is an immediate):
        const int tb = l16 >> 1, th = l16 & 1;
        if constexpr (kDma) {
            // K operand of cell block cb, slab s: cell 16 cb + l16, granule
            // 4s + g, at dma_row_k(l16) + 16 ((4s + g) ^ (l16 % 4)) + cb
            // kCbStride = (constant) + 64 s
            k_off0 = k_off1 = dma_row_k(l16) + 16 * (g ^ (l16 & 3));
            // transposed V read of cell c = 16 (tb >> 2) + 4g + (tb & 3) (and c
            // + 32), bytes 16 db + 8 th: granule db at slot db ^ (c % 4), so
            // the offset depends on db % 4 (one per value) and on db / 4
            // (an immediate 64 (db / 4))
            const int c = 16 * (tb >> 2) + 4 * g + (tb & 3);
#pragma unroll
            for (int j = 0; j < 4; ++j) v_offj[j] = dma_row_v(c) + 16 * (j ^ (c & 3)) + 8 * th;
            v_off = 0;
            // this lane's S cells (cb, 4g + u) are tile cells 16 cb + 4g + u
            m_off0 = m_off1 = 4 * g;
        } else {
            // K operand of cell block cb, slab s: row lds_row(cb, l16), bytes 64s + 16g
            k_off0 = lds_row(0, l16) * kStride + 16 * g;
            k_off1 = (lds_row(1, l16) - 16) * kStride + 16 * g;
            // transposed V read: source role (b, h) = (l16 >> 1, l16 & 1) reads row
            // lds_row(2r + (b >> 2), 4g + (b & 3)), bytes 16db + 8h
            v_off = lds_row(tb >> 2, 4 * g + (tb & 3)) * kStride + 8 * th;
            // this lane's S cells (cb, 4g + u) live in LDS rows lds_row(cb, 4g + u)
            m_off0 = lds_row(0, 4 * g);
            m_off1 = lds_row(1, 4 * g) - 16;
        }
        w_off = 0;
        reset();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) su[cb] = (v4f){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }

    // Moves this lane's LDS offsets to another pipeline's buffers: code rows
    // kv bytes on, scale and bias slots sc elements on, the 1 / W values sw
    // on.  (Not for the causal form, whose mask compares the slot offsets
    // with cell indices.)
    __device__ __forceinline__ void shift(int kv, int sc, int sw) {
        k_off0 += kv;
        k_off1 += kv;
        v_off += kv;
        m_off0 += sc;
        m_off1 += sc;
        w_off += sw;
    }

    __device__ __forceinline__ void reset() {
        m_run = -INFINITY;
        l_part = 0.f;
        frame = 1.f;
        obias = 0.f;
#pragma unroll
        for (int db = 0; db < kDB; ++db) o[db] = (v4f){0.f, 0.f, 0.f, 0.f};
    }

    // Block db of the accumulator, O^T / frame: o without its offset.
    __device__ __forceinline__ v4f acc(int db) const { return o[db] - obias; }

    // One step of the pipeline: the softmax and V accumulation of the tile
    // whose scores are in su (V rows vb, V scales vs), and the scores of the
    // next tile (K rows kb, K scales ks, biases bias_t) into su.  kCausal:
    // cells of the next tile past index lim (this lane's row's last visible
    // cell, counted from the tile's first cell) are masked too.  The two
    // halves are independent (score() and stats() + accumulate()), so the
    // matrix-core and vector work of neighbouring tiles interleave; a
    // pipeline's first step runs only the scores, its last only the
    // accumulation, and a one-tile chunk the two one after the other
    // (tile()), with the same arithmetic.
    template <bool kCausal = false>
    __device__ __forceinline__ void step(const int8_t *kb, const float *ks_t, const float *bias_t,
                                         const int8_t *vb, const float *vs_t, const float *vw_t, int dh,
                                         int lim = 0) {
        // the softmax of the current tile first, so that its scores are dead
        // before the next tile's arrive (one set of score registers)
        const Digits d = prepare(stats(), vs_t, vw_t);
        __builtin_amdgcn_sched_barrier(0);
        score<kCausal>(su, kb, ks_t, bias_t, lim);
        pv(d, vb, dh);
    }

    // A whole one-tile chunk: its scores, then their softmax and V
    // accumulation.
    __device__ __forceinline__ void tile(const int8_t *kb, const float *ks_t, const float *bias_t,
                                         const int8_t *vb, const float *vs_t, const float *vw_t, int dh) {
        score(su, kb, ks_t, bias_t);
        accumulate(stats(), vb, vs_t, vw_t, dh);
    }

    // Softmax statistics of the tile whose scores are in su: the running max
    // moves to include it; the frame and the reference max it implies.  The
    // tile's probabilities are taken against its own maximum t_use (its
    // largest is 1, so its weights use the whole digit grid however far the
    // tile lies below the running maximum) and scaled back by
    // 2^(t_use - running max) <= 1 in the accumulator's factor and the
    // denominator (prepare()).
    struct Stats {
        float corr, frame_new, t_use;
    };
    __device__ __forceinline__ Stats stats() {
        float tmax = -INFINITY;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int u = 0; u < 4; ++u) tmax = fmaxf(tmax, su[cb][u]);
        tmax = max4(tmax);
        tmax = (tmax == -INFINITY) ? -INFINITY : tmax * coef;  // base-2 tile max
        const float m_new = fmaxf(m_run, tmax);
        Stats st;
        st.corr = __builtin_amdgcn_exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
        st.frame_new = (m_run == -INFINITY) ? 1.f : frame * st.corr;
        // (+inf for a row with no visible cell in the tile: every score is
        // -inf, so its probabilities come out 0 all the same)
        st.t_use = (tmax == -INFINITY) ? INFINITY : tmax;
        m_run = m_new;
        return st;
    }

    // Scores of a tile: u = (AB + C/2^8) * k_scale + bias, into sn (kCausal
    // and lim as in step()).
    template <bool kCausal = false>
    __device__ __forceinline__ void score(v4f (&sn)[4], const int8_t *kb, const float *ks_t,
                                          const float *bias_t, int lim = 0) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) sn[cb] = score_block(cb, kb, ks_t, bias_t);
        if constexpr (kCausal) {
            if (__any(lim < kTile - 1)) {  // only tiles that reach past some row's position
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int mo = 16 * cb + ((cb & 1) ? m_off1 : m_off0);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (mo + u > lim) sn[cb][u] = -INFINITY;
                }
            }
        }

    }

    // The scores of this lane's 4 cells of cell block cb (cells 16 cb to
    // 16 cb + 15 of the tile).
    __device__ __forceinline__ v4f score_block(int cb, const int8_t *kb, const float *ks_t,
                                               const float *bias_t) {
        const int8_t *kp = kb + ((cb & 1) ? k_off1 : k_off0) + cb * kCbStride;
        v4i ka[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const v4i *>(kp + 64 * s);
        v4i aa = {0, 0, 0, 0}, bb = {0, 0, 0, 0};
        v4i cc = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            aa = mfma_i8(ka[s], qa[s], aa);
            bb = mfma_i8(ka[s], qb[s], bb);
            cc = mfma_i8(ka[s], qc[s], cc);
        }
        const v4i ab = (aa << 8) + bb;  // 2^8 A + B, |.| < 2^30
        const int mo = 16 * cb + ((cb & 1) ? m_off1 : m_off0);
        const v4f ks = *reinterpret_cast<const v4f *>(ks_t + mo);
        const v4f bs = *reinterpret_cast<const v4f *>(bias_t + mo);
        v4f sn;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float tq = fmaf(__int_as_float(cc[u]), 1.f / 256.f, (float)ab[u]);
            sn[u] = fmaf(tq, ks[u], bs[u]);
        }
        return sn;
    }

    // tile() with the scoring shared by the DS waves that hold the same 16
    // rows: wave dh scores cell blocks (4 / DS) dh to (4 / DS) (dh + 1) - 1
    // and the blocks meet in LDS (xs: 4 blocks x 64 lanes for this row
    // group), so every wave goes on with the scores tile() computes, bit for
    // bit.  Contains a workgroup barrier that every wave must reach.
    template <int DS>
    __device__ __forceinline__ void tile_shared(const int8_t *kb, const float *ks_t,
                                                const float *bias_t, const int8_t *vb,
                                                const float *vs_t, const float *vw_t, int dh, v4f *xs,
                                                int lane) {
        constexpr int kPer = 4 / DS;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int cb = kPer * dh + k;
            xs[64 * cb + lane] = score_block(cb, kb, ks_t, bias_t);
        }
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) su[cb] = xs[64 * cb + lane];
        accumulate(stats(), vb, vs_t, vw_t, dh);
    }

    // Softmax and V accumulation of the tile whose scores are in su (its
    // statistics st from stats()): probabilities, their digits, O^T += V^T P^T.
    __device__ __forceinline__ void accumulate(const Stats &st, const int8_t *vb,
                                               const float *vs_t, const float *vw_t, int dh) {
        const Digits d = prepare(st, vs_t, vw_t);
        __builtin_amdgcn_sched_barrier(0);  // as in step(): the halves apart
        pv<true>(d, vb, dh);
    }

    // The probabilities' digits of a tile and their scale (the softmax half
    // of accumulate()), then the products with the V rows (its P.V half).
    struct Digits {
        v4i xa, xb, xc;
        float tau3l;
    };
    __device__ __forceinline__ Digits prepare(const Stats &st, const float *vs_t, const float *vw_t) {
        const float t_use = st.t_use, corr = st.corr, frame_new = st.frame_new;
        // ---------------- probabilities and their digits for the current tile
        // weights w = p * v_scale on the tile's grid: X = rint(p * v_scale *
        // W) with W = 127 * 2^16 / (the tile's largest V scale) (the slot
        // holds v_scale * W per cell, and 1 / W after them; p <= 1 against
        // the tile's maximum, so X <= 127 * 2^16 < 2^23; a rounding above 1
        // by an ulp still stays below 2^23 and leaves a = 127) lands in the
        // low bits of fma(p, v_scale W, 2^23):
        // X = 2^16 a + 2^8 b + c with balanced digits b, c in [-128, 127] (a
        // in [0, 127]): c = byte 0 of X, b = byte 1 of X + 2^7, a = byte 2 of
        // X + 2^7 + 2^15 (bit 23 of the float pattern, the exponent's lowest
        // bit, is 0 in [2^23, 2^24)).  Byte 1 of X + 2^7 + 2^15 is b + 2^7
        // modulo 2^8: b is read there, its top bit flipped.
        float psum = 0.f;
        v4i xa, xb, xc;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int mo = 16 * cb + ((cb & 1) ? m_off1 : m_off0);
            const v4f vw = *reinterpret_cast<const v4f *>(vs_t + mo);
            unsigned xs[4], x2[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(su[cb][u], coef, -t_use));
                psum += pr;
                xs[u] = __float_as_uint(fmaf(pr, vw[u], kRound));
                x2[u] = xs[u] + 32896u;
            }
            const unsigned c01 = __builtin_amdgcn_perm(xs[1], xs[0], 0x0c0c0400u);
            const unsigned c23 = __builtin_amdgcn_perm(xs[3], xs[2], 0x04000c0cu);
            const unsigned b01 = __builtin_amdgcn_perm(x2[1], x2[0], 0x0c0c0501u);
            const unsigned b23 = __builtin_amdgcn_perm(x2[3], x2[2], 0x05010c0cu);
            const unsigned a01 = __builtin_amdgcn_perm(x2[1], x2[0], 0x0c0c0602u);
            const unsigned a23 = __builtin_amdgcn_perm(x2[3], x2[2], 0x06020c0cu);
            xa[cb] = (int)(a01 | a23);
            xb[cb] = (int)((b01 | b23) ^ 0x80808080u);
            xc[cb] = (int)(c01 | c23);
        }
        // the tile's factor to the running maximum, the same for the row's
        // four lanes (0 for a row with no visible cell in the tile: it adds
        // nothing)
        const float scale = t_use == INFINITY ? 0.f : __builtin_amdgcn_exp2f(t_use - m_run);
        l_part = fmaf(psum, scale, l_part * corr);

        // rare: fold the frame into the accumulator before it gets too small
        frame = frame_new;
        if (__any(frame < kRenorm)) {
#pragma unroll
            for (int db = 0; db < kDB; ++db) o[db] *= frame;
            obias *= frame;
            frame = 1.f;
        }
        // tau3 = scale / (W frame), kept as tau3l = 2^26 tau3 and tau3h = 2^8 tau3
        const float tau3l = ((kTwo26 * vw_t[w_off]) * __builtin_amdgcn_rcpf(frame)) * scale;
        return Digits{xa, xb, xc, tau3l};
    }

    // kAlone: a tile with no scoring beside it (the last of a chunk, or the
    // single-tile kernel): groups of four 16-dim blocks are kept apart, so
    // that the compiler does not issue all the products first and hold every
    // block's sums at once.
    template <bool kAlone = false>
    __device__ __forceinline__ void pv(const Digits &d, const int8_t *vb, int dh) {
        const v4i xa = d.xa, xb = d.xb, xc = d.xc;
        const float tau3l = d.tau3l, tau3h = (1.f / 262144.f) * tau3l;
        // ---------------- O^T += V^T P^T for this wave's blocks of 16 dims
        const int8_t *vp = vb + v_off + 16 * kDB * dh;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            // this lane's 8 bytes of V rows (cells) at dims 16 (kDB dh + db):
            // padded rows, or the DMA layout (kDB dh is a multiple of 4, so
            // the granule's slot is kDB dh + 4 (db / 4) + ((db % 4) ^ (c % 4)))
            const int8_t *v0 = kDma ? vb + v_offj[db & 3] + 16 * kDB * dh + 64 * (db >> 2) : vp + 16 * db;
            const int8_t *v1 = kDma ? v0 + 8 * kDmaBlock : v0 + 32 * kStride;
            const v2i h0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i LDS_AS *)v0);
            const v2i h1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i LDS_AS *)v1);
            const v4i va = {h0[0], h0[1], h1[0], h1[1]};
            const v4i hi = mfma_i8(va, xa, (v4i){0, 0, 0, 0});
            const v4i mid = mfma_i8(va, xb, (v4i){0, 0, 0, 0});
            const v4i lo = mfma_i8(va, xc, (v4i){kLoBits, kLoBits, kLoBits, kLoBits});
            // sum of X * v_code = 2^8 T + LO, with T = 2^8 HI + MID exact in
            // int32 (|T| < 2^29, |LO| <= 64 * 128 * 128 = 2^20); LO arrives
            // biased, (kLoUnits + LO) 2^-26 as a float
            const v4i top = (hi << 8) + mid;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                o[db][u] = fmaf((float)top[u], tau3h, fmaf(__int_as_float(lo[u]), tau3l, o[db][u]));
            if constexpr (kAlone)
                if ((db & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        obias = fmaf(kLoUnit, tau3l, obias);  // kLoUnits tau3
        if constexpr (kAlone) {
            // the sums are complete here: otherwise the compiler may move
            // their conversions past the following barrier, next to the
            // partial's stores, and hold every block's sums until then
#pragma unroll
            for (int db = 0; db < kDB; ++db) __asm__ volatile("" : "+v"(o[db]));
            __asm__ volatile("" : "+v"(obias));
        }
    }

    // The partial's maximum: the base-2 running maximum back in natural-log
    // units.
    __device__ __forceinline__ float m_nat() const {
        return (m_run == -INFINITY) ? -INFINITY : m_run * 0.69314718055994531f;
    }

    // The chunk partial of this lane's row at unit index base (instance,
    // chunk, row) of the workspace.  Every lane of the wave must call it.
    __device__ __forceinline__ void emit(const Params &p, int64_t base, int row, int g, int dh) {
        const float l_row = sum4(l_part);
        if (row < p.n_rows) {
            float *dst = p.acc + base * kDim + 16 * kDB * dh + 4 * g;
#pragma unroll
            for (int db = 0; db < kDB; ++db) *reinterpret_cast<v4f *>(dst + 16 * db) = acc(db) * frame;
            if (g == 0 && dh == 0) {
                p.m[base] = m_nat();
                p.l[base] = l_row;
            }
        }
    }

    // The normalised result of this lane's row (out_row nullptr: a row past
    // the end), with the operations the merge applies to a single partial:
    // out = acc * (1 / l), lse = m + ln l; no visible cell: out = 0,
    // lse = -inf.  Every lane of the wave must call it.
    __device__ __forceinline__ void finish(float *out_row, float *lse_row, int g, int dh) {
        const float l_row = sum4(l_part);
        if (!out_row) return;
        float *dst = out_row + 16 * kDB * dh + 4 * g;
        if (!(l_row > 0.f)) {
#pragma unroll
            for (int db = 0; db < kDB; ++db)
                *reinterpret_cast<v4f *>(dst + 16 * db) = (v4f){0.f, 0.f, 0.f, 0.f};
            if (g == 0 && dh == 0) *lse_row = -INFINITY;
            return;
        }
        const float inv = 1.f / l_row;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
            *reinterpret_cast<v4f *>(dst + 16 * db) = (acc(db) * frame) * inv;
        if (g == 0 && dh == 0) *lse_row = m_run * 0.69314718055994531f + logf(l_row);
    }
};

// LDS flags between the roles of one pipeline in a two-pipeline workgroup
// (in place of the workgroup barrier, which would make each step of both
// pipelines wait for the slower of the two).  A flag holds the last step its
// writer completed; a release store after that step's LDS accesses, an
// acquire load before the reader's.  Waits are bounded: past kSpinLimit polls
// the wait gives up and reports it, so a wait can never hang the GPU (the
// kernel then writes NaN for the rows; no correct run comes near the bound,
// which is tens of milliseconds).
constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ void flag_post(int *flag, int step) {
    __hip_atomic_store(flag, step, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ bool flag_wait(const int *flag, int step) {
#pragma clang loop unroll(disable)
    for (int spin = 0; spin < kSpinLimit; ++spin) {
        // uniform (every lane reads the same flag): a scalar loop exit, so
        // the wait adds no divergent control flow around the step
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v >= step) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// DS = number of compute waves per 16-row group, each accumulating
// O^T for 256 / DS of the head dimensions (every one of them scores the
// whole tile).  DS = 1: two workgroups per CU (LDS-limited; with RB = 1 that
// is one wave per SIMD), for grids that fill the chip.  DS = 2: half the
// V accumulation per wave, which shortens each step of a small,
// latency-bound grid (one workgroup per CU).
//
// kPrompt = false: decode.  Workgroup (blockIdx.x, blockIdx.y) = instance i,
// chunks [cpw * y, cpw * y + cpw) of its list; emits chunk partials.
// kFinal (decode calls whose every instance has at most SP chunks): the
// workgroup runs all of instance i's chunks and writes the head outputs
// itself.  SP = 1: its one chunk.  SP = 2: two pipelines side by side
// (pipeline h: chunk h, its own producer wave, compute waves and LDS),
// synchronised through LDS flags rather than the workgroup barrier; the two
// partials are merged in LDS.  Either way the merge pass's arithmetic
// (merge_weight, merge_acc) turns the partials into outputs, so the result
// is the two passes' bit for bit, without the partials' round trip through
// memory or a second launch.
// kPrompt = true: prompt attention.  Workgroup (i, y) = the 16 RB query rows
// starting at row 16 RB y of instance i (rows are position-major, so a
// workgroup holds a few consecutive positions); the cell list is implicit
// (logical cells 0, 1, 2, ... up to the workgroup's last position), each
// row masks the cells past its own position, and the rows are normalised in
// place of a partial (one chunk spans the whole causal range).
template <int RB, int DS, bool kPrompt, int SP = 1, bool kFinal = false, bool kMulti = false>
__global__ __launch_bounds__(64 * SP * (DS * RB + 1))
__attribute__((amdgpu_waves_per_eu((RB == 1 || DS > 1) ? 1 : 2, 2)))
void chunk_mfma_kernel(Params p, int cpw) {
    static_assert(SP == 1 || (SP == 2 && !kPrompt && DS == 1 && RB >= 2 && RB <= 3),
                  "two pipelines: decode, 2 or 3 row groups");
    static_assert(!(kMulti && kFinal), "several chunks per workgroup: partials");
    static_assert(!(kPrompt && kFinal), "the prompt form always writes its rows");
    static_assert(!kMulti || !kPrompt, "several chunks per workgroup: decode partials");
    static_assert(SP == 1 || RB * 8 * 64 * 16 <= 2 * kBuf,
                  "the hand-over fits a pipeline's K (and V) buffers");
    constexpr int kPipe = DS * RB + 1;  // waves per pipeline
    constexpr int kProducer = DS * RB;  // the producer's role index in a pipeline
    constexpr int kDB = 16 / DS;        // 16-dim blocks of O^T per compute wave
    __shared__ __attribute__((aligned(1024))) int8_t kbuf_p[SP][2][kBuf];
    __shared__ __attribute__((aligned(1024))) int8_t vbuf_p[SP][2][kBuf];
    // physical cell of tile cell 16k + r at [slot][4r + k]
    __shared__ __attribute__((aligned(16))) int phys_p[SP][4][kTile];
    __shared__ __attribute__((aligned(16))) float ks_p[SP][4][kTile];
    __shared__ __attribute__((aligned(16))) float vs_p[SP][4][kTile];
    __shared__ float vw_p[SP][4];  // per slot: 1 / W of the tile (put_v_scales)
    __shared__ __attribute__((aligned(16))) float bias_p[SP][4][kTile];
    // two pipelines: per pipeline, the producer's last completed step and each
    // compute wave's; a flag that any wait gave up
    __shared__ int ready_f[SP], done_f[SP][DS * RB], stuck_f;

    // wave index: uniform, so that the role and pipeline branches are scalar
    const int wv = SP == 1 ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Pipeline and role within it (kProducer: the producer; one pipeline: the
    // last wave).  The hardware deals a workgroup's waves to the four SIMDs
    // of its CU in a fixed cyclic order, so waves k and k + 4 share a SIMD;
    // two pipelines lay out their roles so that the compute waves spread
    // over the SIMDs: pipelines of three make the last two waves the
    // producers (the four compute waves on four SIMDs; with each pipeline's
    // three waves consecutive, some SIMD would hold two compute waves and
    // another none), pipelines of four put pipeline 1's producer first
    // (waves 3 and 4: the six compute waves two, two, one and one).
    const int pipe = SP == 1 ? 0 : kPipe == 3 ? (wv < 4 ? wv / 2 : wv - 4) : wv / kPipe;
    const int wave = SP == 1 ? wv : kPipe == 3 ? (wv < 4 ? wv % 2 : kProducer)
                                               : (pipe == 0 ? wv : (wv - 1) % kPipe);
    const int lane = threadIdx.x & 63;
    int8_t (&kbuf)[2][kBuf] = kbuf_p[pipe];
    int8_t (&vbuf)[2][kBuf] = vbuf_p[pipe];
    int (&phys_s)[4][kTile] = phys_p[pipe];
    float (&ks_s)[4][kTile] = ks_p[pipe];
    float (&vs_s)[4][kTile] = vs_p[pipe];
    float (&bias_s)[4][kTile] = bias_p[pipe];
    const int g = lane >> 4;    // lane group: k-set of the MFMA operands
    const int l16 = lane & 15;  // this lane's row within the wave's 16 rows
    const int i = blockIdx.x;   // instance (fastest: full chunks are dispatched first)
    const int R = p.n_rows;
    int c0 = 0, j_begin = 0, j_end, tpc, row0 = 0;
    int n_iter = 0;  // pipeline steps (the tile count of the longest pipeline)
    int64_t pos0 = 0;
    if constexpr (kFinal) {
        // pipeline h runs chunk h (cells [h C, h C + C) clipped to the count);
        // an instance with fewer chunks leaves a pipeline with no tiles, which
        // still takes every step (no early exit: every wave meets the
        // workgroup's barriers) and contributes nothing
        const int n = count_of(p, i);
        c0 = pipe;
        j_begin = pipe * p.chunk;
        j_end = max(j_begin, min(j_begin + p.chunk, n));
        tpc = 1 << 30;
        n_iter = (min(p.chunk, n) + kTile - 1) / kTile;  // pipeline 0's
    } else if constexpr (!kPrompt && SP == 1) {
        // This workgroup runs chunks [c0, c0 + cpw) of instance i as one
        // stream of tiles: the gather pipeline runs on across chunk
        // boundaries, and the compute waves emit a partial at the end of
        // each chunk.
        c0 = blockIdx.y * cpw;
        const int n = count_of(p, i);
        j_begin = c0 * p.chunk;
        if (j_begin >= n) return;  // this instance has fewer chunks
        j_end = (int)min((int64_t)j_begin + (int64_t)cpw * p.chunk, (int64_t)n);
        tpc = p.chunk / kTile;  // tiles per chunk
    } else if constexpr (!kPrompt) {
        // Two pipelines, each its own cpw chunks from (2 y + h) cpw and its
        // partials: the two independent workgroups of the one-pipeline form
        // in one, so that the waves' placement on the SIMDs is fixed (see
        // the roles above).  A pipeline past the instance's chunks has no
        // tiles and emits nothing; the pipelines share no step, so it just
        // ends.
        const int n = count_of(p, i);
        if ((int64_t)blockIdx.y * SP * cpw * p.chunk >= n) return;  // both pipelines empty
        c0 = (blockIdx.y * SP + pipe) * cpw;
        j_begin = (int)min((int64_t)c0 * p.chunk, (int64_t)n);
        j_end = (int)min((int64_t)j_begin + (int64_t)cpw * p.chunk, (int64_t)n);
        tpc = kMulti ? p.chunk / kTile : 1 << 30;  // one chunk: its partial after the loop
    } else {
        // rows [row0, row0 + 16 RB) sit at positions pos0 + r / n_qheads; the
        // cells run to the last of them, clipped to the page table
        row0 = blockIdx.y * (16 * RB);
        pos0 = p.pos0[i];
        const int last_row = min(row0 + 16 * RB, R) - 1;
        const int64_t last = pos0 + last_row / p.n_qheads;
        j_end = (int)max((int64_t)0, min(last + 1, (int64_t)p.n_logical_pages * kPage));
        tpc = 1 << 30;  // one chunk: no partial inside the loop
    }
    const int n_tiles = (j_end - j_begin + kTile - 1) / kTile;
    if constexpr (!kFinal) n_iter = n_tiles;
    // the last list entry, the target of the clamped list loads (a pipeline
    // with no tiles reads a valid entry: a final-output call has max_sel > 0)
    const int j_last = (kFinal || SP > 1) ? max(j_end - 1, 0) : j_end - 1;

    // scale slots read before their first write hold finite values
    for (int e = threadIdx.x; e < SP * 4 * kTile; e += 64 * SP * kPipe) {
        (&ks_p[0][0][0])[e] = 0.f;
        (&vs_p[0][0][0])[e] = 0.f;
        (&bias_p[0][0][0])[e] = -INFINITY;
        if (e < SP * 4) (&vw_p[0][0])[e] = 0.f;
    }
    if constexpr (SP > 1) {
        if (threadIdx.x < SP * (DS * RB + 1)) {
            const int h = threadIdx.x / (DS * RB + 1), w = threadIdx.x % (DS * RB + 1);
            if (w == DS * RB)
                ready_f[h] = -100;  // below every step a wait asks for
            else
                done_f[h][w] = -100;
        }
        if (threadIdx.x == 0) stuck_f = 0;
    }
    __syncthreads();

    // Both roles run n_iter + 4 iterations with one barrier each.  Iteration
    // t: the producer loads the selected ids of tile t+4, the page-table
    // entries of tile t+3, the scales and K rows of tile t+2 and the V rows of
    // tile t+1 and writes them to LDS; the compute waves score tile t+1 and
    // run the softmax and V accumulation of tile t from LDS written earlier.
    if (wave == kProducer) {
        const int32_t *pt = p.page_table + (int64_t)i * p.pt_stride;
        const int32_t *sel = p.sel + (int64_t)i * p.sel_stride;
        // page table, or (with no logical pages, when every cell is masked) any
        // readable int so that the unconditional loads below stay in bounds
        const int32_t *pt_or_sel = p.n_logical_pages > 0 ? pt : sel;
        int sel3 = -1;  // selected id of tile t+3 (this lane's cell)
        int ph2 = -1;   // physical cell of tile t+2
        for (int t = -4; t < n_iter; ++t) {
            const bool ld_k = (t + 2 >= 0) && (t + 2 < n_tiles);
            const bool ld_v = (t + 1 >= 0) && (t + 1 < n_tiles);
            // gather loads: unconditional, from clamped (always valid) addresses,
            // so that none of them is consumed before the end of the step; the
            // per-lane validity is applied when the values are used
            const bool ld_s = (t + 4 < n_tiles);
            const int j4 = j_begin + (t + 4) * kTile + lane;
            const int lp3 = sel3 >> 4;
            const bool id_ok = sel3 >= 0 && lp3 < p.n_logical_pages;
            const int64_t sc2 = (int64_t)(ph2 < 0 ? 0 : ph2) * p.scale_stride;
            const unsigned kh2 = p.k_scales[sc2];
            const unsigned vh2 = p.v_scales[sc2];
            const int pte3 = pt_or_sel[id_ok ? lp3 : 0];
            const int sel4 = kPrompt ? j4 : sel[j4 < j_end ? j4 : j_last];
            // then the code rows: load (k, c) covers rows 16k + l16, bytes
            // 64c + 16g, so each lane needs the physical cells of 4 rows only
            // (one 16-byte LDS read) and every load uses an immediate offset
            v4i kst[kRows], vst[kRows];
            if (ld_k) {
                const v4i ph4 = *reinterpret_cast<const v4i *>(&phys_s[(t + 2) & 3][4 * l16]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int8_t *src = p.k_codes + (int64_t)(ph4[k] < 0 ? 0 : ph4[k]) * kDim + 16 * g;
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        kst[4 * k + cc] = *reinterpret_cast<const v4i *>(src + 64 * cc);
                }
            }
            if (ld_v) {
                const v4i ph4 = *reinterpret_cast<const v4i *>(&phys_s[(t + 1) & 3][4 * l16]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int8_t *src = p.v_codes + (int64_t)(ph4[k] < 0 ? 0 : ph4[k]) * kDim + 16 * g;
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        vst[4 * k + cc] = *reinterpret_cast<const v4i *>(src + 64 * cc);
                }
            }
            // two pipelines: the compute waves must be done with step t - 1,
            // whose buffers this step overwrites (the loads above are in
            // flight meanwhile)
            if constexpr (SP > 1) {
                if (t >= 0) {
                    bool ok = true;
#pragma unroll
                    for (int w = 0; w < DS * RB; ++w) ok &= flag_wait(&done_f[pipe][w], t - 1);
                    if (!ok) stuck_f = 1;
                }
            }
            // complete: code rows to LDS (row 16k + l16, bytes 64c + 16g)
            if (ld_k) {
                int8_t *kb = kbuf[(t + 2) & 1] + l16 * kStride + 16 * g;
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        *reinterpret_cast<v4i *>(kb + 16 * k * kStride + 64 * cc) = kst[4 * k + cc];
            }
            if (ld_v) {
                int8_t *vb = vbuf[(t + 1) & 1] + l16 * kStride + 16 * g;
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        *reinterpret_cast<v4i *>(vb + 16 * k * kStride + 64 * cc) = vst[4 * k + cc];
            }
            if (ld_k) {
                const int m2 = (t + 2) & 3;
                const bool ok = ph2 >= 0;
                const float ksf = ok ? half_bits_to_float((uint16_t)kh2) : 0.f;
                const float vsf = ok ? half_bits_to_float((uint16_t)vh2) : 0.f;
                ks_s[m2][lane] = ksf;
                put_v_scales(vs_s[m2], &vw_p[pipe][m2], vsf, lane);
                bias_s[m2][lane] = ok ? -kScoreOffset * ksf : -INFINITY;
            }
            if (t + 3 >= 0 && t + 3 < n_tiles) {
                int ph = -1;
                if (id_ok && pte3 >= 0 && (int64_t)pte3 < p.n_phys_pages) ph = (pte3 << 4) | (sel3 & 15);
                phys_s[(t + 3) & 3][4 * l16 + g] = ph;  // cell 16g + l16
                const int j3 = j_begin + (t + 3) * kTile + lane;
                if (!kPrompt && p.gather_out && j3 < j_end)
                    p.gather_out[(int64_t)i * p.sel_stride + j3] = ph;
                ph2 = ph;
            }
            sel3 = (ld_s && j4 < j_end) ? sel4 : -1;
            if constexpr (SP > 1) {
                flag_post(&ready_f[pipe], t);  // this step's LDS writes are done (every lane
                                               // stores the same value)
                __builtin_amdgcn_sched_barrier(0);  // keep steps apart, as the barrier did
            } else {
                __syncthreads();
            }
        }
        if constexpr (kFinal && SP > 1) {  // the end of both pipelines, then the compute waves' hand-over
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ======================= compute waves =======================
    const int row = (wave / DS) * 16 + l16;  // this lane's query row
    const int dh = wave % DS;                // its share of the head dimensions
    RowBlock<kDB> rb;
    const int64_t grow = (int64_t)i * R + row0 + row;  // row in [n_inst][n_rows]
    const bool row_ok = row0 + row < R;
    rb.init(p.q + (row_ok ? grow : (int64_t)i * R + row0) * kDim, row_ok, p.scale_log2, g, l16);
    // the steps below address pipeline 0's buffers; the lane offsets carry
    // the pipeline (one add here instead of a base register per buffer)
    if constexpr (SP > 1) rb.shift(pipe * 2 * kBuf, pipe * 4 * kTile, pipe * 4);
    // prompt: this row's last visible cell (its position)
    const int64_t lim_row = kPrompt ? pos0 + (row0 + row) / p.n_qheads : 0;
    // Steps t = -4 .. n_iter - 1, one barrier each (the producer's count).
    // The halves of step t are the scores of tile t + 1 and the softmax and
    // V accumulation of tile t: step -1 runs only the former, step
    // n_tiles - 1 only the latter, steps past a shorter pipeline's tiles
    // neither; each form has a loop of its own (no branch inside a step).
    auto sync = [&]() {
        if constexpr (SP == 1)
            __syncthreads();
        else
            __builtin_amdgcn_sched_barrier(0);  // keep steps apart, as the barrier did
    };
    // two pipelines: step t reads what the producer wrote in its step t - 1
    // (and earlier)
    auto begin_step = [&](int t) {
        if constexpr (SP > 1)
            if (!flag_wait(&ready_f[pipe], t - 1)) stuck_f = 1;
    };
    auto end_step = [&](int t) {
        if constexpr (SP > 1) flag_post(&done_f[pipe][wave], t);  // this step's LDS reads are done
        sync();
    };
    // end of a chunk (tile t its last): emit its partial, start afresh
    auto emit = [&](int t) {
        if constexpr (!kPrompt && !kFinal) {
            const int c = kMulti ? c0 + t / tpc : c0;
            // two pipelines: a wait that gave up (never in a correct run)
            // poisons the partial, so that the merged rows come out NaN
            if constexpr (SP > 1)
                if (*reinterpret_cast<volatile int *>(&stuck_f)) rb.l_part = NAN;
            rb.emit(p, ((int64_t)i * p.n_chunks + c) * R + row, row, g, dh);
            rb.reset();
        }
    };
    // prompt: the mask limit of tile t + 1, whose first cell is j_begin + 64 (t + 1)
    auto lim_next = [&](int t) {
        return kPrompt ? (int)max((int64_t)-1, min(lim_row - (j_begin + (int64_t)(t + 1) * kTile),
                                                   (int64_t)kTile))
                       : 0;
    };
    for (int t = -4; t < -1; ++t) sync();
    begin_step(-1);
    if (n_tiles > 0) rb.template score<kPrompt>(rb.su, kbuf_p[0][0], ks_p[0][0], bias_p[0][0], lim_next(-1));
    end_step(-1);
    for (int t = 0; t < n_tiles - 1; ++t) {
        begin_step(t);
        rb.template step<kPrompt>(kbuf_p[0][(t + 1) & 1], ks_p[0][(t + 1) & 3], bias_p[0][(t + 1) & 3],
                                  vbuf_p[0][t & 1], vs_p[0][t & 3], &vw_p[0][t & 3], dh, lim_next(t));
        if constexpr (kMulti)
            if ((t + 1) % tpc == 0) emit(t);
        end_step(t);
    }
    if (n_tiles > 0) {
        const int t = n_tiles - 1;
        begin_step(t);
        rb.accumulate(rb.stats(), vbuf_p[0][t & 1], vs_p[0][t & 3], &vw_p[0][t & 3], dh);
        end_step(t);
    }
    for (int t = n_tiles; t < n_iter; ++t) {
        begin_step(t);
        end_step(t);
    }
    if (n_tiles > 0) emit(n_tiles - 1);  // the (last) chunk's partial
    if constexpr (kPrompt) {
        // the row's output address formed only here, from an opaque copy of
        // the row index: hoisted above the tile loop it would hold two 64-bit
        // pointers across it
        int r_late = row;
        __asm__ volatile("" : "+v"(r_late));
        const int64_t g_late = (int64_t)i * R + row0 + r_late;
        rb.finish(row_ok ? p.out + g_late * kDim : nullptr, p.lse + g_late, g, dh);
    }
    if constexpr (kFinal) {
        // each pipeline's partial as the chunk pass would emit it: acc = o *
        // frame, m = m_nat(), l = the row sum
        const float l_row = sum4(rb.l_part);
        const float m_row = rb.m_nat();
        // pipeline 1 hands its partial over through its own staging buffers,
        // idle since the last step's barrier: wave w's accumulator block db
        // at [w][db % 8][lane] of its K buffers (db < 8) or V buffers (8 KB
        // per wave in each), m and l by row in its scale slots
        auto xslot = [&](int db) {
            float *base = reinterpret_cast<float *>(db < kDB / 2 ? &kbuf_p[SP - 1][0][0]
                                                                 : &vbuf_p[SP - 1][0][0]);
            return reinterpret_cast<v4f *>(base) + (wave * (kDB / 2) + db % (kDB / 2)) * 64 + lane;
        };
        float *xm = &ks_p[SP - 1][0][0];
        float *xl = &vs_p[SP - 1][0][0];
        if constexpr (SP > 1) {
            __syncthreads();  // both pipelines' steps are over: their buffers are idle
            if (pipe == 1) {
#pragma unroll
                for (int db = 0; db < kDB; ++db) *xslot(db) = rb.acc(db) * rb.frame;
                if (g == 0) {
                    xm[row] = m_row;
                    xl[row] = l_row;
                }
            }
            __syncthreads();
            if (pipe == 1) return;
            if (stuck_f) {  // a wait gave up (never in a correct run): poison the rows
                if (row_ok) {
                    float *dst = p.out + grow * kDim + 16 * kDB * dh + 4 * g;
#pragma unroll
                    for (int db = 0; db < kDB; ++db)
                        *reinterpret_cast<v4f *>(dst + 16 * db) = (v4f){NAN, NAN, NAN, NAN};
                    if (g == 0) p.lse[grow] = NAN;
                }
                return;
            }
        }
        if (!row_ok) return;
        // the merge of the instance's nch partials, chunk by chunk
        const int nch = (count_of(p, i) + p.chunk - 1) / p.chunk;  // at most SP
        float mc[SP], lc[SP];
        mc[0] = m_row;
        lc[0] = l_row;
        if constexpr (SP > 1) {
            mc[1] = xm[row];
            lc[1] = xl[row];
        }
        float M = -INFINITY;
#pragma unroll
        for (int c = 0; c < SP; ++c)
            if (c < nch) M = fmaxf(M, mc[c]);
        float L = 0.f, w[SP];
#pragma unroll
        for (int c = 0; c < SP; ++c) {
            w[c] = 0.f;
            if (c < nch) {
                w[c] = merge_weight(mc[c], M);
                L = fmaf(lc[c], w[c], L);
            }
        }
        float *dst = p.out + grow * kDim + 16 * kDB * dh + 4 * g;
        const bool any = L > 0.f;
        const float inv = any ? 1.f / L : 0.f;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            v4f o = (v4f){0.f, 0.f, 0.f, 0.f};
            if (0 < nch) o = merge_acc(o, w[0], rb.acc(db) * rb.frame);
            if constexpr (SP > 1)
                if (1 < nch) o = merge_acc(o, w[1], *xslot(db));
            *reinterpret_cast<v4f *>(dst + 16 * db) = any ? o * inv : (v4f){0.f, 0.f, 0.f, 0.f};
        }
        if (g == 0 && dh == 0) p.lse[grow] = any ? M + logf(L) : -INFINITY;
    }
}

constexpr int kPtLdsPages = 2048;  // page tables up to this size are staged whole (8 KB)

// One producer wave stages tile cells [j0, j0 + 64) of instance i (entries
// from j_end on are masked): the list entries and the page-table entries,
// then the scales and the K and V code rows together.  With pt_s (a page
// table of at most kPtLdsPages entries) the whole page-table row is loaded
// into LDS in the same round trip as the list entries, so the lookup is an
// LDS read: two dependent round trips to memory instead of three.  LDS
// layout as in the pipelined kernel (row r = tile cell r, padded rows;
// scales and bias by cell).
__device__ __forceinline__ void stage_tile(const Params &p, int32_t *gather_out, int i, int j0,
                                           int j_end, int lane, int8_t *kb, int8_t *vb, float *ks, float *vs,
                                           float *vw,
                                           float *bias, int *pt_s) {
    const int g = lane >> 4, l16 = lane & 15;
    const int32_t *pt = p.page_table + (int64_t)i * p.pt_stride;
    const int32_t *sel = p.sel + (int64_t)i * p.sel_stride;
    const int32_t *pt_or_sel = p.n_logical_pages > 0 ? pt : sel;
    const int j = j0 + lane;
    const int c = j < j_end ? sel[j] : -1;
    const int lp = c >> 4;
    const bool id_ok = c >= 0 && lp < p.n_logical_pages;
    int pte;
    if (pt_s) {
        // the whole row, every load issued before the first LDS write (one
        // round trip): 16-byte pieces when the row is 16-byte aligned, else
        // single entries
        const int nlp = p.n_logical_pages;
        if ((reinterpret_cast<uintptr_t>(pt) & 15) == 0) {
            v4i t[kPtLdsPages / 256];
#pragma unroll
            for (int k = 0; k < kPtLdsPages / 256; ++k) {
                const int e = 4 * lane + 256 * k;
                if (e + 4 <= nlp) t[k] = *reinterpret_cast<const v4i *>(pt + e);
            }
#pragma unroll
            for (int k = 0; k < kPtLdsPages / 256; ++k) {
                const int e = 4 * lane + 256 * k;
                if (e + 4 <= nlp) *reinterpret_cast<v4i *>(pt_s + e) = t[k];
            }
            const int e = (nlp & ~3) + lane;  // the last nlp % 4 entries
            if (e < nlp) pt_s[e] = pt[e];
        } else {
            int t[kPtLdsPages / 64];
#pragma unroll
            for (int k = 0; k < kPtLdsPages / 64; ++k) {
                const int e = lane + 64 * k;
                if (e < nlp) t[k] = pt[e];
            }
#pragma unroll
            for (int k = 0; k < kPtLdsPages / 64; ++k) {
                const int e = lane + 64 * k;
                if (e < nlp) pt_s[e] = t[k];
            }
        }
        // the wave's own LDS writes, read back by other lanes of the wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        pte = id_ok ? pt_s[lp] : 0;
    } else {
        pte = pt_or_sel[id_ok ? lp : 0];
    }
    int ph = -1;
    if (id_ok && pte >= 0 && (int64_t)pte < p.n_phys_pages) ph = (pte << 4) | (c & 15);
    if (gather_out && j < j_end) gather_out[(int64_t)i * p.sel_stride + j] = ph;
    const int64_t sc = (int64_t)(ph < 0 ? 0 : ph) * p.scale_stride;
    const unsigned kh = p.k_scales[sc];
    const unsigned vh = p.v_scales[sc];
    // load (k, cc) covers row 16k + l16, bytes 64cc + 16g; a masked cell
    // reads cell 0 (its score is -inf)
    v4i kst[kRows], vst[kRows];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int pr = __shfl(ph, 16 * k + l16);
        const int64_t off = (int64_t)(pr < 0 ? 0 : pr) * kDim + 16 * g;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            kst[4 * k + cc] = *reinterpret_cast<const v4i *>(p.k_codes + off + 64 * cc);
            vst[4 * k + cc] = *reinterpret_cast<const v4i *>(p.v_codes + off + 64 * cc);
        }
    }
    const bool ok = ph >= 0;
    const float ksf = ok ? half_bits_to_float((uint16_t)kh) : 0.f;
    const float vsf = ok ? half_bits_to_float((uint16_t)vh) : 0.f;
    ks[lane] = ksf;
    put_v_scales(vs, vw, vsf, lane);
    bias[lane] = ok ? -kScoreOffset * ksf : -INFINITY;
    int8_t *kd = kb + l16 * kStride + 16 * g;
    int8_t *vd = vb + l16 * kStride + 16 * g;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            *reinterpret_cast<v4i *>(kd + 16 * k * kStride + 64 * cc) = kst[4 * k + cc];
            *reinterpret_cast<v4i *>(vd + 16 * k * kStride + 64 * cc) = vst[4 * k + cc];
        }
}

// Chunks of one tile (64 cells) in a latency-bound grid: workgroup =
// (instance, chunk, row group z), holding the 16 RB query rows from row
// 16 RB z on, with DS * RB compute waves and one producer wave
// that stages the tile in three round trips (the pipelined kernel takes five
// steps for one tile).  The compute waves then score the tile and run its
// softmax and V accumulation (RowBlock::tile: the arithmetic the pipelined
// kernel applies to a one-tile chunk; with DS = 2 the two waves of a row
// group each score half the cell blocks and exchange them in LDS,
// RowBlock::tile_shared), so the partial is bit for bit the same whichever
// kernel or workgroup holds a row.
//
// kGrouped: one workgroup per (tile, row group), launched as a
// one-dimensional grid of ceil(T / 8) * 8 * G workgroups (T tiles, G row
// groups).  Workgroups go to the 8 XCDs in turn by linear id, so the id is
// mapped to make the G workgroups of a tile share an XCD: each tile is then
// gathered from memory into one L2 and staged again from there, instead of
// once per row group.  Ids past the last tile exit at once.
template <int RB, int DS, bool kGrouped = false>
__global__ __launch_bounds__(64 * (DS * RB + 1))
__attribute__((amdgpu_waves_per_eu(2, 2)))  // at most 256 registers: no AGPR copies
void chunk_tile_kernel(Params p) {
    constexpr int kProducer = DS * RB;
    constexpr int kDB = 16 / DS;
    constexpr bool kShared = DS > 1;  // the DS waves of a row group share its scoring
    __shared__ __attribute__((aligned(16))) v4f xs[kShared ? RB * 4 * 64 : 1];
    __shared__ __attribute__((aligned(1024))) int8_t kbuf[kBuf];
    __shared__ __attribute__((aligned(1024))) int8_t vbuf[kBuf];
    __shared__ __attribute__((aligned(16))) float ks_s[kTile];
    __shared__ __attribute__((aligned(16))) float vs_s[kTile];
    __shared__ float vw_s[1];
    __shared__ __attribute__((aligned(16))) float bias_s[kTile];
    __shared__ __attribute__((aligned(16))) int pt_s[kPtLdsPages];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    int i = blockIdx.x;  // instance
    int c = blockIdx.y;  // chunk = tile
    int z = 0;           // row group
    if constexpr (kGrouped) {
        const int n_groups = (p.n_rows + 16 * RB - 1) / (16 * RB);
        const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
        const int item = (k / n_groups) * 8 + xcd;  // the XCD's (k / G)-th tile
        if (item >= p.n_inst * p.n_chunks) return;
        i = item / p.n_chunks;
        c = item % p.n_chunks;
        z = k % n_groups;
    }
    const int n = count_of(p, i);
    const int j_begin = c * kTile;
    if (j_begin >= n) return;  // this instance has fewer chunks
    const int j_end = min(j_begin + kTile, n);

    if (wave == kProducer) {
        // every row group's workgroup stages the tile; one writes gather_out
        stage_tile(p, z == 0 ? p.gather_out : nullptr, i, j_begin, j_end, lane, kbuf,
                   vbuf, ks_s, vs_s, vw_s, bias_s, p.n_logical_pages <= kPtLdsPages ? pt_s : nullptr);
        __syncthreads();
        if constexpr (kShared) __syncthreads();  // the compute waves' score exchange
        return;
    }
    const int g = lane >> 4, l16 = lane & 15;
    const int row = (z * RB + wave / DS) * 16 + l16;
    const int dh = wave % DS;
    const int R = p.n_rows;
    RowBlock<kDB> rb;
    rb.init(p.q + ((int64_t)i * R + (row < R ? row : 0)) * kDim, row < R, p.scale_log2, g, l16);
    __syncthreads();
    if constexpr (kShared)
        rb.template tile_shared<DS>(kbuf, ks_s, bias_s, vbuf, vs_s, vw_s,
                                    __builtin_amdgcn_readfirstlane(dh),
                                    xs + 256 * (wave / DS), lane);
    else
        rb.tile(kbuf, ks_s, bias_s, vbuf, vs_s, vw_s, dh);
    rb.emit(p, ((int64_t)i * p.n_chunks + c) * R + row, row, g, dh);
}

// Prompt attention with no producer wave: one workgroup of eight compute
// waves per CU holds six 16-row groups (96 rows).  Waves 0-3 take groups 0-3
// whole; waves 4-7 take groups 4 and 5 two waves each, each wave scoring two
// of a tile's four 16-cell blocks (the blocks meet in LDS) and accumulating
// 128 of the 256 dimensions.  The hardware puts waves k and k + 4 on one
// SIMD, so every SIMD runs one whole group and half of another: the vector
// and matrix work is even over the four SIMDs (with two workgroups of three
// groups and a producer, two SIMDs carry two groups each and two carry one).
// Every wave stages part of each tile with LDS-DMA loads (no staging
// registers): in step t waves 0-3 four 1 KB blocks each of K rows of tile
// t + 2, waves 4-7 four of V rows of tile t + 1; wave 4 also maps tile t + 3's
// cells to physical cells (into LDS, for those loads) and loads its scales.
// The instance's page-table row is read into LDS once.  Each step ends with the
// waves' own loads complete and one workgroup barrier.  Step t: softmax and
// V accumulation of tile t, scores of tile t + 1 (as in the pipelined
// kernel).  The arithmetic per row is RowBlock's, so a row's result is the
// other prompt form's up to the order of the cells within a tile.
constexpr int kDmaWaves = 8;
constexpr int kDmaRows = 96;  // six 16-row groups

// One LDS-DMA load: each lane's 16 bytes at src to LDS lds_dst + 16 lane
// (lds_dst wave-uniform).  Written as inline assembly so that the compiler
// does not see an LDS write in flight: it would otherwise wait for the load
// before every LDS access that might alias it, i.e. within the step that
// issued it.  The kernel waits for its loads itself (vmcnt) before the
// barrier that publishes them.  M0 is used by no other instruction of the
// kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 in the clobbers (see above)
__device__ __forceinline__ void dma16(const void *src, const void *lds_dst) {
    const unsigned a = (unsigned)(uintptr_t)(LDS_AS const void *)lds_dst;
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(a)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

__global__ __launch_bounds__(64 * kDmaWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prompt_dma_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) int8_t kbuf[2][kDmaBuf];
    __shared__ __attribute__((aligned(1024))) int8_t vbuf[2][kDmaBuf];
    __shared__ __attribute__((aligned(16))) float ks_s[4][kTile];
    __shared__ __attribute__((aligned(16))) float vs_s[4][kTile];
    __shared__ float vw_s[4];
    __shared__ __attribute__((aligned(16))) float bias_s[4][kTile];
    // shared scores of the split groups: [tile parity][group 4 or 5][block][lane]
    __shared__ __attribute__((aligned(16))) v4f xs[2][2][4][64];
    __shared__ __attribute__((aligned(16))) int pt_s[kPtLdsPages];
    // physical cell (or -1) of tile cell c at [slot][16 (c % 4) + c / 4]: the
    // four cells one lane loads in a wave's four blocks are adjacent
    __shared__ __attribute__((aligned(16))) int phys_s[4][kTile];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int i = blockIdx.x;
    const int R = p.n_rows;
    const int row0 = blockIdx.y * kDmaRows;
    const int64_t pos0 = p.pos0[i];
    const int last_row = min(row0 + kDmaRows, R) - 1;
    const int nlp = p.n_logical_pages;  // at most kPtLdsPages (the launch checks)
    const int j_end = (int)max((int64_t)0, min(pos0 + last_row / p.n_qheads + 1, (int64_t)nlp * kPage));
    const int n_tiles = (j_end + kTile - 1) / kTile;

    // the page-table row, and scale slots that are read before their first
    // write holding finite values
    const int32_t *pt = p.page_table + (int64_t)i * p.pt_stride;
    for (int e = threadIdx.x; e < nlp; e += 64 * kDmaWaves) pt_s[e] = pt[e];
    for (int e = threadIdx.x; e < 4 * kTile; e += 64 * kDmaWaves) {
        (&ks_s[0][0])[e] = 0.f;
        (&vs_s[0][0])[e] = 0.f;
        (&bias_s[0][0])[e] = -INFINITY;
        if (e < 4) vw_s[e] = 0.f;
    }
    __syncthreads();

    // physical cell of tile cell c of tile t, or -1 (past the cells, or an
    // unmapped page)
    auto phys_of = [&](int t, int c) {
        const int j = t * kTile + c;
        if (j >= j_end) return -1;
        const int pte = pt_s[j >> 4];
        return (pte >= 0 && (int64_t)pte < p.n_phys_pages) ? ((pte << 4) | (j & 15)) : -1;
    };
    // blocks 4w .. 4w + 3 (cells 16w .. 16w + 15) of tile t's K or V rows:
    // lane L writes slot L % 16 of cell 4b + L / 16, which holds the row's
    // granule (L % 16) ^ (L / 16); masked cells read cell 0 (weight 0)
    auto dma_blocks = [&](const int8_t *codes, int8_t *buf, int w, bool is_v, int t) {
        const int r = lane >> 4, q = lane & 15;
        const v4i ph4 = *reinterpret_cast<const v4i *>(&phys_s[t & 3][16 * r + 4 * w]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = 4 * w + k;
            const int8_t *src = codes + (int64_t)(ph4[k] < 0 ? 0 : ph4[k]) * kDim + 16 * (q ^ r);
            dma16(src, buf + kDmaBlock * b + 64 * (is_v ? dma_sigma_v(b) : dma_sigma_k(b)));
        }
    };
    // step t's staging: K rows of tile t + 2 (waves 0-3), V rows of tile t + 1
    // (waves 4-7); wave 4 also maps tile t + 3's cells and loads its scales
    // (written to LDS by scales_done once they arrive)
    unsigned kh = 0, vh = 0;
    int ph_s = -1;
    auto stage = [&](int t) {
        if (wave < 4) {
            if (t + 2 >= 0 && t + 2 < n_tiles) dma_blocks(p.k_codes, kbuf[(t + 2) & 1], wave, false, t + 2);
        } else {
            // (the scale loads first: their use at the end of the step then
            // waits for nothing issued after them)
            if (wave == 4 && t + 3 < n_tiles) {
                ph_s = phys_of(t + 3, lane);
                phys_s[(t + 3) & 3][16 * (lane & 3) + (lane >> 2)] = ph_s;
                const int64_t sc = (int64_t)(ph_s < 0 ? 0 : ph_s) * p.scale_stride;
                kh = p.k_scales[sc];
                vh = p.v_scales[sc];
            }
            if (t + 1 >= 0 && t + 1 < n_tiles) dma_blocks(p.v_codes, vbuf[(t + 1) & 1], wave - 4, true, t + 1);
        }
    };
    auto scales_done = [&](int t) {
        if (wave == 4 && t + 3 < n_tiles) {
            const int m2 = (t + 3) & 3;
            const bool ok = ph_s >= 0;
            const float ksf = ok ? half_bits_to_float((uint16_t)kh) : 0.f;
            const float vsf = ok ? half_bits_to_float((uint16_t)vh) : 0.f;
            ks_s[m2][lane] = ksf;
            put_v_scales(vs_s[m2], &vw_s[m2], vsf, lane);
            bias_s[m2][lane] = ok ? -kScoreOffset * ksf : -INFINITY;
        }
    };
    auto end_step = [&](int t) {
        __builtin_amdgcn_sched_barrier(0);  // the step's work first
        scales_done(t);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's LDS-DMA loads have landed
        __syncthreads();
    };

    // this wave's rows: group rg, dimensions [128 dh, 128 dh + 128) when split
    const bool whole = wave < 4;
    const int rg = whole ? wave : 4 + ((wave - 4) >> 1);
    const int dh = whole ? 0 : (wave - 4) & 1;
    const int row = 16 * rg + l16;
    const int64_t grow = (int64_t)i * R + row0 + row;
    const bool row_ok = row0 + row < R;
    const float *qrow = p.q + (row_ok ? grow : (int64_t)i * R + row0) * kDim;
    const int64_t lim_row = pos0 + (row0 + row) / p.n_qheads;
    // the mask limit of tile t + 1 (its first cell is 64 (t + 1))
    auto lim_next = [&](int t) {
        return (int)max((int64_t)-1, min(lim_row - (int64_t)(t + 1) * kTile, (int64_t)kTile));
    };

    if (whole) {
        RowBlock<16, true> rb;
        rb.init(qrow, row_ok, p.scale_log2, g, l16);
        stage(-3);
        end_step(-3);
        stage(-2);
        end_step(-2);
        stage(-1);
        if (n_tiles > 0) rb.template score<true>(rb.su, kbuf[0], ks_s[0], bias_s[0], lim_next(-1));
        end_step(-1);
        for (int t = 0; t < n_tiles - 1; ++t) {
            stage(t);
            rb.template step<true>(kbuf[(t + 1) & 1], ks_s[(t + 1) & 3], bias_s[(t + 1) & 3],
                                   vbuf[t & 1], vs_s[t & 3], &vw_s[t & 3], 0, lim_next(t));
            end_step(t);
        }
        if (n_tiles > 0) {
            const int t = n_tiles - 1;
            stage(t);
            rb.accumulate(rb.stats(), vbuf[t & 1], vs_s[t & 3], &vw_s[t & 3], 0);
            end_step(t);
        }
        // the row's output address formed only here, from an opaque copy of
        // the row index: hoisted above the tile loop it would hold two 64-bit
        // pointers across it
        int r_late = row;
        __asm__ volatile("" : "+v"(r_late));
        const int64_t g_late = (int64_t)i * R + row0 + r_late;
        rb.finish(row_ok ? p.out + g_late * kDim : nullptr, p.lse + g_late, g, 0);
    } else {
        RowBlock<8, true> rb;
        rb.init(qrow, row_ok, p.scale_log2, g, l16);
        // this wave's two cell blocks of tile t + 1, masked, into LDS
        auto score_half = [&](int t) {
            const int8_t *kb = kbuf[(t + 1) & 1];
            const float *ks_t = ks_s[(t + 1) & 3];
            const float *bias_t = bias_s[(t + 1) & 3];
            const int lim = lim_next(t);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int cb = 2 * dh + k;
                v4f sn = rb.score_block(cb, kb, ks_t, bias_t);
                if (__any(lim < kTile - 1)) {
                    const int mo = 16 * cb + 4 * g;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (mo + u > lim) sn[u] = -INFINITY;
                }
                xs[(t + 1) & 1][rg - 4][cb][lane] = sn;
            }
        };
        auto load_scores = [&](int t) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) rb.su[cb] = xs[t & 1][rg - 4][cb][lane];
        };
        stage(-3);
        end_step(-3);
        stage(-2);
        end_step(-2);
        stage(-1);
        if (n_tiles > 0) score_half(-1);
        end_step(-1);
        for (int t = 0; t < n_tiles - 1; ++t) {
            stage(t);
            load_scores(t);
            const auto d = rb.prepare(rb.stats(), vs_s[t & 3], &vw_s[t & 3]);
            __builtin_amdgcn_sched_barrier(0);
            score_half(t);
            rb.pv(d, vbuf[t & 1], dh);
            end_step(t);
        }
        if (n_tiles > 0) {
            const int t = n_tiles - 1;
            stage(t);
            load_scores(t);
            rb.accumulate(rb.stats(), vbuf[t & 1], vs_s[t & 3], &vw_s[t & 3], dh);
            end_step(t);
        }
        // the row's output address formed only here, from an opaque copy of
        // the row index: hoisted above the tile loop it would hold two 64-bit
        // pointers across it
        int r_late = row;
        __asm__ volatile("" : "+v"(r_late));
        const int64_t g_late = (int64_t)i * R + row0 + r_late;
        rb.finish(row_ok ? p.out + g_late * kDim : nullptr, p.lse + g_late, g, dh);
    }
}

template <int DS, bool kMulti>
void launch_rb(const Params &p, dim3 grid, int cpw, hipStream_t s) {
    switch ((p.n_rows + 15) / 16) {
        case 1: chunk_mfma_kernel<1, DS, false, 1, false, kMulti><<<grid, 64 * (DS + 1), 0, s>>>(p, cpw); break;
        case 2: chunk_mfma_kernel<2, DS, false, 1, false, kMulti><<<grid, 64 * (2 * DS + 1), 0, s>>>(p, cpw); break;
        case 3: chunk_mfma_kernel<3, 1, false, 1, false, kMulti><<<grid, 64 * 4, 0, s>>>(p, cpw); break;
        default: chunk_mfma_kernel<4, 1, false, 1, false, kMulti><<<grid, 64 * 5, 0, s>>>(p, cpw); break;
    }
}

}  // namespace

hipError_t launch_chunk(const Params &p, hipStream_t s) {
    const int64_t items = (int64_t)p.n_inst * p.n_chunks;
    // one-tile chunks in a grid of at most one workgroup per CU: stage the
    // tile at once.  While the grid still fits one workgroup per CU with a
    // workgroup per 16-row group, each row group gets its own (its V
    // accumulation split over two waves): the tile's compute then takes the
    // time of one group's, and the extra stagings of the tile are L2 hits
    // (the groups of a tile share an XCD).  Otherwise all groups share one
    // workgroup (a single group still splits its V accumulation; with more
    // groups that measured slower).
    if (p.chunk == kTile && items <= kLatencyWorkgroups) {
        const int groups = (p.n_rows + 15) / 16;
        if (groups > 1 && items * groups <= kLatencyWorkgroups) {
            const unsigned wgs = (unsigned)((items + 7) / 8) * 8u * (unsigned)groups;
            chunk_tile_kernel<1, 2, true><<<dim3(wgs), 64 * 3, 0, s>>>(p);
            return hipGetLastError();
        }
        const dim3 grid(p.n_inst, p.n_chunks);
        switch ((p.n_rows + 15) / 16) {
            case 1: chunk_tile_kernel<1, 2><<<grid, 64 * 3, 0, s>>>(p); break;
            case 2: chunk_tile_kernel<2, 1><<<grid, 64 * 3, 0, s>>>(p); break;
            case 3: chunk_tile_kernel<3, 1><<<grid, 64 * 4, 0, s>>>(p); break;
            default: chunk_tile_kernel<4, 1><<<grid, 64 * 5, 0, s>>>(p); break;
        }
        return hipGetLastError();
    }
    // Chunks per workgroup: enough that the grid stays at about two
    // workgroups per CU (256 CUs), so that no pipeline refills between the
    // chunks a workgroup would otherwise have left to a later wave of
    // workgroups; a small grid keeps one chunk per workgroup.
    int cpw = (int)(items / kResidentWorkgroups);
    cpw = cpw < 1 ? 1 : (cpw > p.n_chunks ? p.n_chunks : cpw);
    dim3 grid(p.n_inst, (p.n_chunks + cpw - 1) / cpw);
    // A grid of at most one workgroup per CU is latency-bound: split the V
    // accumulation of each 16-row group over two waves while that still
    // leaves about one compute wave per SIMD (up to 32 rows).
    // (a workgroup with several chunks emits partials inside its tile loop:
    // a form of its own, so that the one-chunk form keeps that code out of
    // the loop)
    if (items <= kLatencyWorkgroups && p.n_rows <= 32) {
        launch_rb<2, false>(p, grid, cpw, s);  // cpw is 1 here
    } else if (p.n_chunks > cpw && (p.n_rows + 15) / 16 == 2) {
        // two 16-row groups: two workgroups of three waves would share a CU,
        // and the second continues the first's cycle over the SIMDs, leaving
        // one SIMD two compute waves and another none; one workgroup of two
        // pipelines (each with cpw chunks) places its four compute waves on
        // four SIMDs
        const dim3 g2(p.n_inst, (grid.y + 1) / 2);
        if (cpw > 1)
            chunk_mfma_kernel<2, 1, false, 2, false, true><<<g2, 64 * 6, 0, s>>>(p, cpw);
        else
            chunk_mfma_kernel<2, 1, false, 2, false, false><<<g2, 64 * 6, 0, s>>>(p, 1);
    } else if (cpw > 1) {
        launch_rb<1, true>(p, grid, cpw, s);
    } else {
        launch_rb<1, false>(p, grid, cpw, s);
    }
    return hipGetLastError();
}

bool chunk_writes_output(const Params &p) {
    // multi-tile chunks only: one-tile chunks take the single-tile kernel
    if (p.n_chunks < 1 || p.n_chunks > 2 || p.chunk <= kTile) return false;
    // Two pipelines: 2 or 3 row groups (more do not fit two waves per SIMD).
    // With one row group the pair measured no faster than two workgroups and
    // the merge launch: the shared barrier makes each step wait for the
    // slower of two gathers, which costs about what the merge saves.
    return p.n_chunks == 1 || (p.n_rows > 16 && p.n_rows <= 48);
}

hipError_t launch_chunk_final(const Params &p, hipStream_t s) {
    const dim3 grid(p.n_inst, 1);
    const int rb = (p.n_rows + 15) / 16;
    if (p.n_chunks == 2) {
        // two pipelines of RB + 1 waves, one workgroup per CU (LDS)
        switch (rb) {
            case 2: chunk_mfma_kernel<2, 1, false, 2, true><<<grid, 64 * 6, 0, s>>>(p, 1); break;
            default: chunk_mfma_kernel<3, 1, false, 2, true><<<grid, 64 * 8, 0, s>>>(p, 1); break;
        }
    } else if (p.n_inst <= kLatencyWorkgroups && p.n_rows <= 32) {
        // the launch shapes of launch_chunk for the same grid
        switch (rb) {
            case 1: chunk_mfma_kernel<1, 2, false, 1, true><<<grid, 64 * 3, 0, s>>>(p, 1); break;
            default: chunk_mfma_kernel<2, 2, false, 1, true><<<grid, 64 * 5, 0, s>>>(p, 1); break;
        }
    } else {
        switch (rb) {
            case 1: chunk_mfma_kernel<1, 1, false, 1, true><<<grid, 64 * 2, 0, s>>>(p, 1); break;
            case 2: chunk_mfma_kernel<2, 1, false, 1, true><<<grid, 64 * 3, 0, s>>>(p, 1); break;
            case 3: chunk_mfma_kernel<3, 1, false, 1, true><<<grid, 64 * 4, 0, s>>>(p, 1); break;
            default: chunk_mfma_kernel<4, 1, false, 1, true><<<grid, 64 * 5, 0, s>>>(p, 1); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_prompt(const Params &p, hipStream_t s) {
    // A compute wave holds about 250 VGPRs, so a SIMD runs two: a workgroup
    // of four 16-row groups (five waves) runs alone on its CU, one of three
    // groups (four waves) runs beside a second one.  Per CU the two forms
    // have about the same throughput, so 64-row workgroups are used while
    // they fit one to a CU, 48-row ones when the grid is larger (two to a
    // CU), and fewer rows use fewer groups.
    int rb = (p.n_rows + 15) / 16;
    if (rb > 4 && p.n_logical_pages <= kPtLdsPages) {
        // more than four row groups: 96-row workgroups of eight compute waves,
        // one per CU, the vector and matrix work even over the SIMDs
        const dim3 grid(p.n_inst, (p.n_rows + kDmaRows - 1) / kDmaRows);
        prompt_dma_kernel<<<grid, 64 * kDmaWaves, 0, s>>>(p);
        return hipGetLastError();
    }
    if (rb > 4) rb = (int64_t)p.n_inst * ((p.n_rows + 63) / 64) <= kLatencyWorkgroups ? 4 : 3;
    const dim3 grid(p.n_inst, (p.n_rows + 16 * rb - 1) / (16 * rb));
    switch (rb) {
        case 1: chunk_mfma_kernel<1, 1, true><<<grid, 64 * 2, 0, s>>>(p, 1); break;
        case 2: chunk_mfma_kernel<2, 1, true><<<grid, 64 * 3, 0, s>>>(p, 1); break;
        case 3: chunk_mfma_kernel<3, 1, true><<<grid, 64 * 4, 0, s>>>(p, 1); break;
        default: chunk_mfma_kernel<4, 1, true><<<grid, 64 * 5, 0, s>>>(p, 1); break;
    }
    return hipGetLastError();
}

}  // namespace sda
