// csa_sort.hip -- orders every output row by (score desc, key index asc).
//
// The scoring kernel leaves each row's top-k in key order; the result is
// returned sorted by score, ties by the lower key index, padding (-1, -inf)
// last.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_bitonic.hpp"
#include "csa_kernels.hpp"
#include "csa_order_key.hpp"

namespace csa {

// ------------------------------------------------------------------ row sort

// Sorts each row of k (index, score) pairs by (score desc, index asc);
// padding (-1, -inf) sorts last.  pow2 = next power of two >= k entries of
// 64-bit keys live in dynamic LDS; NT threads share a row (256 for rows wider
// than a wave sorts, 1,024 when there are fewer rows than compute units).
template <int NT>
__global__ void __launch_bounds__(NT)
sort_rows_kernel(int32_t *out_idx, float *out_score, int64_t nrows, int k, int pow2)
{
    extern __shared__ unsigned long long s_key[];
    const int tid = threadIdx.x;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        int32_t *ri = out_idx + row * k;
        float *rs = out_score + row * k;
        for (int e = tid; e < pow2; e += NT) {
            unsigned long long key = ~0ull;
            if (e < k) {
                const uint32_t u = order_key(rs[e]);
                key = (static_cast<unsigned long long>(~u) << 32) | uint32_t(ri[e]);
            }
            s_key[e] = key;
        }
        __syncthreads();
        lds_bitonic_sort(s_key, pow2, tid, NT);
        for (int e = tid; e < k; e += NT) {
            const unsigned long long key = s_key[e];
            ri[e] = int32_t(uint32_t(key));
            rs[e] = key_to_float(~uint32_t(key >> 32));
        }
        __syncthreads();
    }
}

// One wave per row: next_pow2(k) = 64*E keys (score desc, index asc as the
// ascending 64-bit key ~orderkey(score) << 32 | index), padding as all-ones.
// Rows move between memory and the blocked register layout through a
// per-wave LDS buffer, one 32-bit half at a time: the global loads and
// stores then cover whole cache lines (consecutive lanes, consecutive
// elements), and the buffer's one-word pad per 32 keeps each lane's run of
// E words on distinct banks.
// Three waves per SIMD: at E = 32 that costs a few spilled registers but
// beats two waves per SIMD without spills by 12% (the network is latency-
// bound: 64-bit compares, lane permutes, swizzles); the smaller E fit anyway.
template <int E>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
sort_rows_wave_kernel(int32_t *out_idx, float *out_score, int64_t nrows, int k)
{
    constexpr int N = 64 * E;
    constexpr int NPAD = N + N / 32;
    __shared__ uint32_t s_buf[4][NPAD];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint32_t *sb = s_buf[w];
    const int64_t wave = int64_t(blockIdx.x) * 4 + w;
    const int64_t nwaves = int64_t(gridDim.x) * 4;
    auto pad = [](int i) { return i + (i >> 5); };
    auto lds_sync = [] {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    };
    for (int64_t row = wave; row < nrows; row += nwaves) {
        int32_t *ri = out_idx + row * k;
        float *rs = out_score + row * k;
        unsigned long long key[E];
        // high halves: ~orderkey(score), all-ones past k
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const int i = j * 64 + lane;
            sb[pad(i)] = i < k ? ~order_key(rs[i]) : 0xFFFFFFFFu;
        }
        lds_sync();
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] = static_cast<unsigned long long>(sb[pad(lane * E + e)]) << 32;
        lds_sync();
        // low halves: the key index
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const int i = j * 64 + lane;
            sb[pad(i)] = i < k ? uint32_t(ri[i]) : 0xFFFFFFFFu;
        }
        lds_sync();
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] |= sb[pad(lane * E + e)];
        bitonic_sort<E, 2>(key, lane);
        lds_sync();
#pragma unroll
        for (int e = 0; e < E; ++e) sb[pad(lane * E + e)] = uint32_t(key[e]);
        lds_sync();
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const int i = j * 64 + lane;
            if (i < k) ri[i] = int32_t(sb[pad(i)]);
        }
        lds_sync();
#pragma unroll
        for (int e = 0; e < E; ++e) sb[pad(lane * E + e)] = uint32_t(key[e] >> 32);
        lds_sync();
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const int i = j * 64 + lane;
            if (i < k) rs[i] = key_to_float(~sb[pad(i)]);
        }
        lds_sync();
    }
}

template <int E>
static hipError_t launch_sort_wave(int64_t nrows, int k, int num_cus, int32_t *out_idx,
                                   float *out_score, hipStream_t s)
{
    const int64_t want = int64_t(num_cus) * 8;
    const int64_t blocks = (nrows + 3) / 4;
    const int grid = int(blocks < want ? blocks : want);
    hipLaunchKernelGGL(sort_rows_wave_kernel<E>, dim3(grid), dim3(256), 0, s, out_idx, out_score,
                       nrows, k);
    return hipGetLastError();
}

hipError_t launch_sort_rows(const Plan &p, int32_t *out_idx, float *out_score, int num_cus,
                            hipStream_t s)
{
    const int64_t nrows = p.B * p.S;
    if (nrows == 0) return hipSuccess;
    // fewer rows than compute units: one wave per row would leave each row's
    // long serial network alone on its CU; a workgroup per row is quicker
    const bool few = nrows < num_cus && p.sort_pow2 >= 256;
    switch (few ? 0 : p.sort_pow2 <= 64 ? 64 : p.sort_pow2) {
    case 64: return launch_sort_wave<1>(nrows, p.k, num_cus, out_idx, out_score, s);
    case 128: return launch_sort_wave<2>(nrows, p.k, num_cus, out_idx, out_score, s);
    case 256: return launch_sort_wave<4>(nrows, p.k, num_cus, out_idx, out_score, s);
    case 512: return launch_sort_wave<8>(nrows, p.k, num_cus, out_idx, out_score, s);
    case 1024: return launch_sort_wave<16>(nrows, p.k, num_cus, out_idx, out_score, s);
    case 2048: return launch_sort_wave<32>(nrows, p.k, num_cus, out_idx, out_score, s);
    default: break;
    }
    const int64_t want = int64_t(num_cus) * 8;
    const int grid = int(nrows < want ? nrows : want);
    const size_t lds = size_t(p.sort_pow2) * sizeof(unsigned long long);
    if (few) {
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(sort_rows_kernel<1024>),
                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(sort_rows_kernel<1024>, dim3(grid), dim3(1024), lds, s, out_idx,
                           out_score, nrows, p.k, p.sort_pow2);
        return hipGetLastError();
    }
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(sort_rows_kernel<256>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sort_rows_kernel<256>, dim3(grid), dim3(256), lds, s, out_idx, out_score,
                       nrows, p.k, p.sort_pow2);
    return hipGetLastError();
}

}  // namespace csa
