// Internal declarations shared by the HIP translation units of libsda.so.
// Not part of the public ABI (include/sda.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sda {

constexpr int kPage = 16;
constexpr int kDim = 256;
constexpr int kMaxRows = 64;

// Everything one call needs on the device, already validated on the host.
struct Params {
    // pools (physical cell = page * 16 + slot)
    const int8_t *k_codes;
    const uint16_t *k_scales;
    const int8_t *v_codes;
    const uint16_t *v_scales;
    int64_t scale_stride;       // elements between the scales of consecutive cells
    int64_t n_phys_pages;
    // per-instance inputs
    const int32_t *page_table;
    int64_t pt_stride;
    int32_t n_logical_pages;
    const int32_t *sel;
    int64_t sel_stride;
    const int32_t *n_sel_dev;  // device counts (batch) or nullptr (step)
    int32_t n_sel_host;        // count used when n_sel_dev is nullptr
    int32_t max_sel;
    const float *q;            // [n_inst][n_rows][kDim]
    int32_t n_inst;
    int32_t n_rows;            // n_q * n_qheads
    float scale_log2;          // softmax_scale * log2(e): scores in base-2 units
    int32_t chunk;             // cells per chunk
    int32_t n_chunks;          // ceil(max_sel / chunk)
    // chunk partials (workspace)
    float *acc;                // [n_inst][n_chunks][n_rows][kDim]
    float *m;                  // [n_inst][n_chunks][n_rows], natural-log units
    float *l;                  // [n_inst][n_chunks][n_rows]
    // outputs
    int32_t *gather_out;       // nullable [n_inst][sel_stride]
    float *out;                // [n_inst][n_rows][kDim]
    float *lse;                // [n_inst][n_rows]
    // prompt attention: rows r = t * n_qheads + h sit at position pos0[i] + t
    const int32_t *pos0;       // device [n_inst]
    int32_t n_qheads;
};

// IEEE binary16 bit pattern -> float (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// The log-sum-exp merge of a row's chunk partials (m_c, l_c, acc_c), as every
// merge in the library runs it, chunk by chunk in chunk order:
//   M = max_c m_c (from -inf),  w_c = e^(m_c - M) (0 for an empty chunk;
//   computed as 2^((m_c - M) log2 e) with the hardware exp2: with the
//   roundings of the difference and the product, relative error below
//   (1 + |m_c - M|) 2^-23, and weights far below 1 where that grows),
//   L = fma(l_c, w_c, L),  o = fma(w_c, acc_c, o) element by element (from 0),
//   out = o * (1 / L),  lse = M + ln L  (L = 0: out = 0, lse = -inf).
// The explicit fmas fix the rounding, so the merge kernels and the chunk
// kernel's in-place merge give the same bits.
__device__ __forceinline__ float merge_weight(float mc, float M) {
    return mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mc - M) * 1.4426950408889634f);
}

// Maximum over the four lanes l, l^16, l^32, l^48 (one query row of an
// MFMA output), with the gfx950 lane swaps (VALU, no LDS round trip).
__device__ __forceinline__ float max4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Maximum over all 64 lanes: quad permutes, half-row and row mirrors (DPP),
// then the 16- and 32-lane swaps (no LDS round trip).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xb1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4e>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return max4(x);
}

typedef float merge_v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ merge_v4f merge_acc(merge_v4f o, float w, merge_v4f a) {
    return (merge_v4f){__builtin_fmaf(w, a[0], o[0]), __builtin_fmaf(w, a[1], o[1]),
                       __builtin_fmaf(w, a[2], o[2]), __builtin_fmaf(w, a[3], o[3])};
}

// Number of selected entries instance i actually uses.
__device__ __forceinline__ int count_of(const Params &p, int i) {
    int n = p.n_sel_dev ? p.n_sel_dev[i] : p.n_sel_host;
    n = n < 0 ? 0 : n;
    return n > p.max_sel ? p.max_sel : n;
}

// KV append: new rows [n_inst][n_new][kDim] into the pools (already validated).
struct AppendParams {
    int8_t *k_codes;
    uint16_t *k_scales;
    int8_t *v_codes;
    uint16_t *v_scales;
    int64_t scale_stride;
    int64_t n_phys_pages;
    const int32_t *page_table;  // [n_inst][pt_stride]
    int64_t pt_stride;
    int32_t n_logical_pages;
    const int32_t *pos0;        // device [n_inst]: position of new row 0
    const float *k_new;         // [n_inst][n_new][kDim]
    const float *v_new;
    int32_t n_inst;
    int32_t n_new;
};

// QSA block scoring and selection (already validated).
constexpr int kQsaMaxRows = 8;
constexpr int kQsaMaxHd = 1024;        // n_heads * idx_dim, a multiple of 64
constexpr int kQsaMaxBlocks = 16384;   // blocks per instance the selection holds in LDS
constexpr int kQsaMaxK = 4096;
struct QsaParams {
    const float *pooled;       // [n_inst][max_blocks][hd]
    const uint8_t *dead;       // [n_inst][max_blocks]
    const float *q_idx;        // [n_inst][n_rows][hd]
    const int32_t *n_visible;  // [n_inst][n_rows]
    float *scores;             // [n_inst][n_rows][max_blocks]
    int32_t *sel;              // [n_inst][sel_stride]
    int32_t *n_sel;            // [n_inst]
    int64_t sel_stride;
    int32_t n_inst, n_rows, hd, block_cells, max_blocks, k_blocks;
};
hipError_t launch_qsa_scores(const QsaParams &p, hipStream_t s);
hipError_t launch_qsa_select(const QsaParams &p, hipStream_t s);

hipError_t launch_chunk(const Params &p, hipStream_t s);
// Whether a call with both passes runs as one chunk-kernel launch that writes
// the head outputs (every instance has at most two multi-tile chunks), and
// that launch.  The workspace is not touched.
bool chunk_writes_output(const Params &p);
hipError_t launch_chunk_final(const Params &p, hipStream_t s);
hipError_t launch_kv_append(const AppendParams &p, hipStream_t s);
hipError_t launch_merge(const Params &p, hipStream_t s);
hipError_t launch_prompt(const Params &p, hipStream_t s);

}  // namespace sda
