// csa_kernels.hip -- the key-range merge kernel and the dispatch of the
// scoring kernel (csa_stream.hpp) to its per-type instantiations.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_stream.hpp"

namespace csa {

// ------------------------------------------------------------ key-range merge

constexpr int kMergeThreads = 256;

// Selects, for every query position, the k best entries by (score desc, key
// index asc) of its G partial lists (the exact top-k of each key range, the
// ranges in ascending key order, so that equal scores appear in ascending
// key order along the concatenated lists), and writes them to the output row
// in no particular order.  One workgroup per position: an MSB-first radix
// select (4 x 8 bits) on the order keys finds the k-th best key K and how
// many entries equal to K to take; a last pass writes every larger entry and
// the first such entries equal to K.  Padding entries (index -1, score -inf)
// order below every finite score and fill the row when fewer than k keys are
// visible.
__global__ void __launch_bounds__(kMergeThreads)
merge_splits_kernel(const int32_t *__restrict__ pidx, const float *__restrict__ pscore,
                    int64_t rows, int G, int k, int32_t *__restrict__ out_idx,
                    float *__restrict__ out_score)
{
    constexpr int NW = kMergeThreads / 64;
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_sel[2];
    __shared__ uint32_t s_wsum[NW];
    __shared__ int s_gt;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = G * k;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int32_t *ri = pidx + row * n;
        const float *rs = pscore + row * n;
        uint32_t prefix = 0u, pmask = 0u;
        int need = k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kMergeThreads) s_hist[i] = 0u;
            __syncthreads();
            for (int e = tid; e < n; e += kMergeThreads) {
                const uint32_t u = order_key(rs[e]);
                if ((u & pmask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l holds digits 255-4l .. 252-4l, so a prefix sum over
                // the lanes counts the entries at or above a lane's digits
                const uint32_t c0 = s_hist[255 - 4 * lane], c1 = s_hist[254 - 4 * lane];
                const uint32_t c2 = s_hist[253 - 4 * lane], c3 = s_hist[252 - 4 * lane];
                const uint32_t cl = c0 + c1 + c2 + c3;
                const uint32_t pre = wave_prefix_sum(cl);
                const uint64_t bal = __ballot(pre >= uint32_t(need));
                const int L = __ffsll(static_cast<unsigned long long>(bal)) - 1;
                const uint32_t a0 = pre - cl;
                int d;
                uint32_t above;
                if (a0 + c0 >= uint32_t(need)) {
                    d = 255 - 4 * lane;
                    above = a0;
                } else if (a0 + c0 + c1 >= uint32_t(need)) {
                    d = 254 - 4 * lane;
                    above = a0 + c0;
                } else if (a0 + c0 + c1 + c2 >= uint32_t(need)) {
                    d = 253 - 4 * lane;
                    above = a0 + c0 + c1;
                } else {
                    d = 252 - 4 * lane;
                    above = a0 + c0 + c1 + c2;
                }
                d = __builtin_amdgcn_readlane(d, L);
                above = __builtin_amdgcn_readlane(above, L);
                if (lane == 0) {
                    s_sel[0] = uint32_t(d);
                    s_sel[1] = above;
                }
            }
            __syncthreads();
            prefix |= s_sel[0] << shift;
            pmask |= 0xFFu << shift;
            need -= int(s_sel[1]);
            __syncthreads();
        }
        // prefix is the k-th best key: the k - need larger entries and the
        // first `need` equal ones along the lists form the result
        const int n_gt = k - need;
        int32_t *oi = out_idx + row * k;
        float *os = out_score + row * k;
        if (tid == 0) s_gt = 0;
        __syncthreads();
        int eq_base = 0;
        for (int base = 0; base < n; base += kMergeThreads) {
            const int e = base + tid;
            float sc = 0.f;
            uint32_t u = 0u;
            if (e < n) {
                sc = rs[e];
                u = order_key(sc);
            }
            const bool gt = e < n && u > prefix;
            const bool eq = e < n && u == prefix;
            if (gt) {
                const int p = atomicAdd(&s_gt, 1);
                if (p < n_gt) {  // exactly n_gt entries are larger
                    oi[p] = ri[e];
                    os[p] = sc;
                }
            }
            const uint64_t me = __ballot(eq);
            if (lane == 0) s_wsum[wave] = uint32_t(__popcll(me));
            __syncthreads();
            int wbase = 0, tot = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const int c = int(s_wsum[v]);
                wbase += v < wave ? c : 0;
                tot += c;
            }
            const int rank = eq_base + wbase + lanes_below(me);
            if (eq && rank < need) {
                oi[n_gt + rank] = ri[e];
                os[n_gt + rank] = sc;
            }
            eq_base += tot;
            __syncthreads();
        }
    }
}

hipError_t launch_merge_splits(const Plan &p, const int32_t *part_idx, const float *part_score,
                               int32_t *out_idx, float *out_score, int num_cus, hipStream_t s)
{
    const int64_t rows = p.B * p.S;
    if (rows <= 0 || p.n_splits <= 1) return hipSuccess;
    const int64_t cap = int64_t(num_cus) * 8;
    const int grid = int(rows < cap ? rows : cap);
    hipLaunchKernelGGL(merge_splits_kernel, dim3(grid), dim3(kMergeThreads), 0, s, part_idx,
                       part_score, rows, p.n_splits, p.k, out_idx, out_score);
    return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch

hipError_t launch_stream_topk(const Plan &p, const StreamArgs &a, hipStream_t s)
{
    if (p.grid <= 0) return hipSuccess;
    if (!p.fp8) {
        switch (p.D) {
        case 32: return launch_stream_bf16_d32(p.H, a, p.grid, s);
        case 64: return launch_stream_bf16_d64(p.H, a, p.grid, s);
        case 128: return launch_stream_bf16_d128(p.H, a, p.grid, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.D) {
    case 64: return launch_stream_fp8_d64(p.H, a, p.grid, s);
    case 128: return launch_stream_fp8_d128(p.H, a, p.grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
