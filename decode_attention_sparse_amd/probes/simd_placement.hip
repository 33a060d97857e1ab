// Where the waves of a workgroup land: 512 workgroups of W waves (2 to 8),
// each holding L bytes of LDS (73,728 by default, so two share a CU as the
// chunk kernels' do; 147,968 keeps one per CU), stay resident for a while and
// record the hardware id of each wave (SIMD, CU, shader array, engine) and
// the XCD id.  Printed: how often each assignment of the W waves to SIMDs
// occurs, and per CU how the waves not named in the producer mask P (a bit
// per wave index; by default the last wave) spread over the four SIMDs.
// Usage: simd_placement [W [P [L]]].  Standalone program (no library code),
// built next to libsda.so.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            return 1;                                                              \
        }                                                                          \
    } while (0)

constexpr int kWorkgroups = 512;
constexpr int kMaxWaves = 8;

// out: [kWorkgroups][kMaxWaves] hardware ids, then the same for XCD ids
__global__ __launch_bounds__(512) void placement(unsigned *out, long spin) {
    extern __shared__ int lds[];
    lds[threadIdx.x] = threadIdx.x;
    __syncthreads();
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const long t0 = clock64();  // stay resident so that the grid is placed at once
    while (clock64() - t0 < spin) {
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        out[blockIdx.x * kMaxWaves + w] = hw;
        out[kWorkgroups * kMaxWaves + blockIdx.x * kMaxWaves + w] = xcc;
    }
    if (lds[threadIdx.x] == -1) out[0] = 0;
}

int main(int argc, char **argv) {
    const int waves = argc > 1 ? atoi(argv[1]) : 4;
    const unsigned pmask = argc > 2 ? (unsigned)strtoul(argv[2], nullptr, 0) : 1u << (waves - 1);
    const int lds = argc > 3 ? atoi(argv[3]) : 73728;
    if (waves < 2 || waves > kMaxWaves || lds < 64 * kMaxWaves * 4 || lds > 160 * 1024) {
        fprintf(stderr, "waves 2..8, LDS bytes 2048..163840\n");
        return 1;
    }
    CHECK(hipFuncSetAttribute((const void *)placement, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    unsigned *d;
    const size_t n = 2 * (size_t)kWorkgroups * kMaxWaves;
    CHECK(hipMalloc(&d, n * sizeof(unsigned)));
    CHECK(hipMemset(d, 0, n * sizeof(unsigned)));
    hipLaunchKernelGGL(placement, kWorkgroups, 64 * waves, lds, 0, d, 200000L);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<unsigned> h(n);
    CHECK(hipMemcpy(h.data(), d, n * sizeof(unsigned), hipMemcpyDeviceToHost));
    // HW_ID (gfx9 layout): SIMD in bits 5:4, CU in bits 11:8, shader array in
    // bit 12, engine in bits 15:13
    auto simd = [&](int w, int k) { return (int)((h[w * kMaxWaves + k] >> 4) & 3); };
    std::map<std::vector<int>, int> pattern;
    for (int w = 0; w < kWorkgroups; ++w) {
        std::vector<int> s;
        for (int k = 0; k < waves; ++k) s.push_back(simd(w, k));
        pattern[s]++;
    }
    for (auto &kv : pattern) {
        printf("{\"waves\": %d, \"lds\": %d, \"simd_of_each_wave\": [", waves, lds);
        for (int k = 0; k < waves; ++k) printf(k ? ", %d" : "%d", kv.first[k]);
        printf("], \"workgroups\": %d}\n", kv.second);
    }
    std::map<unsigned, std::vector<int>> cu;  // (XCD, engine, array, CU) -> its workgroups
    for (int w = 0; w < kWorkgroups; ++w)
        cu[((h[w * kMaxWaves] >> 8) & 0xFF) | ((h[kWorkgroups * kMaxWaves + w * kMaxWaves] & 0xF) << 8)].push_back(w);
    std::map<std::vector<int>, int> spread;
    for (auto &kv : cu) {
        std::vector<int> c(4, 0);
        for (int w : kv.second)
            for (int k = 0; k < waves; ++k)
                if (!(pmask >> k & 1)) c[simd(w, k)]++;
        std::sort(c.begin(), c.end());
        spread[c]++;
    }
    for (auto &kv : spread)
        printf("{\"waves\": %d, \"producer_mask\": %u, \"other_waves_per_simd_sorted\": [%d, %d, %d, %d], \"cus\": %d}\n",
               waves, pmask, kv.first[0], kv.first[1], kv.first[2], kv.first[3], kv.second);
    CHECK(hipFree(d));
    return 0;
}
