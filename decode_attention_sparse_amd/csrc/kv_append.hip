// KV append: quantise new K and V rows to INT8 and write them into the paged
// pools, the step that produces what the attention reads.
//
// Source: the Strata PR #2220 page names the pools (INT8 K/V, one binary16
// scale per cell for each) and the Strata round-9 page lists the KV append
// among the steps that follow the K/V projection (section "R9-gpu-8: one
// exact launch for QSA K and V").  The quantiser itself is not on the pages;
// this is symmetric per-cell absmax quantisation with every step in float32:
//   amax = max_d |x[d]|,  s16 = binary16(min(amax / 127, 65504)) (nearest
//   even),  s = value of s16,  code[d] = clamp(rint(x[d] / s), -127, 127)
//   (ties to even; all 0 when s = 0).
// The divisions are IEEE float32 (correctly rounded), so each code is the
// same integer decision a float32 reference takes.
//
// One wave per new cell: lane l holds dims [4l, 4l + 4) of the K and the V
// row (one 16-byte load each), the maximum runs over the wave with DPP and
// lane swaps, and each lane stores its four codes as one 4-byte word (a
// 256-byte row per wave).  Workgroup = four consecutive new rows of one
// instance.  HBM-bound: per cell 2 KB read, 516 B written.
#include "sda_internal.h"

namespace sda {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// Quantises this lane's four values of one row; returns the packed codes and
// sets the scale's binary16 bits.
__device__ __forceinline__ uint32_t quantise4(v4f x, uint16_t *scale_bits) {
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    amax = wave_max(amax);  // over the row's 64 lanes
    const float s32 = fminf(amax / 127.0f, 65504.0f);
    const _Float16 s16 = (_Float16)s32;  // round to nearest even
    const float s = (float)s16;
    uint32_t packed = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float q = 0.f;
        if (s > 0.f) q = fminf(fmaxf(rintf(x[u] / s), -127.f), 127.f);
        packed |= ((uint32_t)(int32_t)q & 0xffu) << (8 * u);
    }
    *scale_bits = __builtin_bit_cast(uint16_t, s16);
    return packed;
}

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.y;                     // instance
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;  // new row
    if (t >= p.n_new) return;
    // the row's values: issued before the page lookup, which they do not need
    const int64_t src = ((int64_t)i * p.n_new + t) * kDim + 4 * lane;
    const v4f xk = *reinterpret_cast<const v4f *>(p.k_new + src);
    const v4f xv = *reinterpret_cast<const v4f *>(p.v_new + src);
    const int64_t c = (int64_t)p.pos0[i] + t;
    if (c < 0 || c >= (int64_t)p.n_logical_pages * kPage) return;
    const int pte = p.page_table[(int64_t)i * p.pt_stride + (c >> 4)];
    if (pte < 0 || (int64_t)pte >= p.n_phys_pages) return;  // masked page: nothing written
    const int64_t ph = (int64_t)pte * kPage + (c & 15);
    uint16_t sk, sv;
    const uint32_t ck = quantise4(xk, &sk);
    const uint32_t cv = quantise4(xv, &sv);
    *reinterpret_cast<uint32_t *>(p.k_codes + ph * kDim + 4 * lane) = ck;
    *reinterpret_cast<uint32_t *>(p.v_codes + ph * kDim + 4 * lane) = cv;
    if (lane == 0) {
        p.k_scales[ph * p.scale_stride] = sk;
        p.v_scales[ph * p.scale_stride] = sv;
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendParams &p, hipStream_t s) {
    const dim3 grid((unsigned)((p.n_new + 3) / 4), (unsigned)p.n_inst);
    kv_append_kernel<<<grid, dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace sda
