// csa_bitonic.hpp -- bitonic sort of 64*E 64-bit keys held by one wave in
// registers (E keys per lane), shared by the row sort and by the scoring
// kernel's final selection.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csa {

// Lane l holds slots l*E .. l*E+E-1 (blocked order) as 64-bit keys; the
// network runs its stages of stride < E inside each lane and the others
// across lanes with register permutes, with no workgroup barrier.
// The value of lane (lane ^ D) for D = 1, 2, ..., 32, by lane permutes
// that stay in registers: DPP quad permutes (1, 2), a bit-mask swizzle
// inside each half-wave (4), a DPP rotation by half a 16-lane row (8), and
// the row-pair and half-wave swaps (16, 32), which give every lane both the
// lower and the upper lane's value.  The DPP forms are full permutations
// with every row and bank enabled, so no lane keeps its old value: the moves
// take none (an `old` operand would cost a register initialisation each).
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane)
{
    if constexpr (D == 1) {
        return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    } else if constexpr (D == 2) {
        return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    } else if constexpr (D == 4) {
        return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), 0x101F));      // and 31, xor 4
    } else if constexpr (D == 8) {
        return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
    } else if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(D == 32, "partner lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

// One compare-exchange step of the bitonic network over N = 64*E keys held
// E per lane in blocked order (lane l holds positions l*E .. l*E+E-1):
// merging runs of SIZE, partners STRIDE positions apart.  Ascending order.
template <int E, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_step(unsigned long long (&key)[E], int lane)
{
    if constexpr (STRIDE < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int f = e ^ STRIDE;
            if (f > e) {
                const bool up = ((lane * E + e) & SIZE) == 0;
                const unsigned long long x = key[e], y = key[f];
                const bool sw = (x > y) == up;
                key[e] = sw ? y : x;
                key[f] = sw ? x : y;
            }
        }
    } else {
        constexpr int D = STRIDE / E;  // partner lane distance
        const bool lower = (lane & D) == 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const unsigned long long o =
                (static_cast<unsigned long long>(lane_xor<D>(uint32_t(key[e] >> 32), lane)) << 32) |
                lane_xor<D>(uint32_t(key[e]), lane);
            const bool up = ((lane * E + e) & SIZE) == 0;
            const bool keep_min = lower == up;
            // the partner's key replaces ours when it is the one to keep
            const bool take = (key[e] < o) != keep_min;
            key[e] = take ? o : key[e];
        }
    }
    if constexpr (STRIDE > 1) bitonic_step<E, SIZE, STRIDE / 2>(key, lane);
}

template <int E, int SIZE>
__device__ __forceinline__ void bitonic_sort(unsigned long long (&key)[E], int lane)
{
    bitonic_step<E, SIZE, SIZE / 2>(key, lane);
    if constexpr (SIZE < 64 * E) bitonic_sort<E, SIZE * 2>(key, lane);
}

// Sorts pow2 64-bit keys in LDS ascending with a bitonic network run by the
// nt threads of a workgroup (thread tid), one barrier per stage.  The
// caller has made the keys visible (barrier) before the call; they are
// visible to every thread on return.
__device__ __forceinline__ void lds_bitonic_sort(unsigned long long *s_key, int pow2, int tid,
                                                 int nt)
{
    for (int size = 2; size <= pow2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < pow2 / 2; i += nt) {
                const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const unsigned long long x = s_key[lo], y = s_key[hi];
                if ((x > y) == up) {
                    s_key[lo] = y;
                    s_key[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace csa
