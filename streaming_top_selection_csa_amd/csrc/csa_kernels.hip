// csa_kernels.hip -- the key-range merge kernel and the dispatch of the
// scoring kernel (csa_stream.hpp) to its per-type instantiations.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_stream.hpp"

namespace csa {

// ------------------------------------------------------------ key-range merge

constexpr int kMergeThreads = 512;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeBins = 4096;  // top 12 bits of the order key
constexpr int kMergeCap = 6144;   // candidates of the k-th bin held in LDS
constexpr int kMergeEpt = 8;      // consecutive list entries per thread in the gather

struct MergeShared {
    uint32_t hist[kMergeBins];
    uint32_t cu[kMergeCap];
    int32_t ci[kMergeCap];
    uint32_t w[kMergeWaves];
    uint32_t w2[2][kMergeWaves];
    uint32_t sel[2];
    int first;
    int out;
};

// Rank of this thread's flag among the flagged threads of the workgroup, in
// thread order, and their number (two barriers).
__device__ __forceinline__ int block_rank(bool f, uint32_t *sw, int lane, int wave, int *total)
{
    const uint64_t m = __ballot(f);
    if (lane == 0) sw[wave] = uint32_t(__popcll(m));
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int v = 0; v < kMergeWaves; ++v) {
        const int c = int(sw[v]);
        base += v < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return base + lanes_below(m);
}

// In a 256-bin histogram h whose bin d counts the candidates with digit d,
// finds (by wave 0; the others wait at the barrier) the digit of the
// `need`-th best candidate and the number of candidates with larger digits.
__device__ __forceinline__ void digit_of_rank(const uint32_t *h, int need, uint32_t *sel, int lane,
                                              int wave)
{
    if (wave == 0) {
        const uint32_t c0 = h[255 - 4 * lane], c1 = h[254 - 4 * lane];
        const uint32_t c2 = h[253 - 4 * lane], c3 = h[252 - 4 * lane];
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
            sel[0] = uint32_t(d);
            sel[1] = above;
        }
    }
    __syncthreads();
}

// Selects, for every query position, the k best entries by (score desc, key
// index asc) of its G partial lists (the exact top-k of each key range, the
// ranges in ascending key order, so that equal scores appear in ascending
// key order along the concatenated lists), and writes them to the output row
// in no particular order.  One workgroup per position.  A histogram of the
// top 12 bits of the order keys names the bin holding the k-th best; one
// more pass writes every entry of a higher bin and gathers that bin's
// entries, in list order, into LDS, where a radix select on the low 20 bits
// finishes.  If the bin holds more than kMergeCap entries, an MSB-first
// 4 x 8-bit radix select over the lists takes its place.  Equal keys are
// taken in list order.  Padding entries (index -1, score -inf) order below
// every finite score and fill the row when fewer than k keys are visible.
__global__ void __launch_bounds__(kMergeThreads)
merge_splits_kernel(const int32_t *__restrict__ pidx, const float *__restrict__ pscore,
                    int64_t rows, int G, int k, int32_t *__restrict__ out_idx,
                    float *__restrict__ out_score)
{
    __shared__ MergeShared sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = G * k;
    constexpr int PER = kMergeBins / kMergeThreads;  // histogram bins per thread
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int32_t *ri = pidx + row * n;
        const float *rs = pscore + row * n;
        int32_t *oi = out_idx + row * k;
        float *os = out_score + row * k;

        // ---- histogram of the top 12 bits
#pragma unroll
        for (int j = 0; j < PER; ++j) sh.hist[tid * PER + j] = 0u;
        if (tid == 0) {
            sh.first = kMergeThreads;
            sh.out = 0;
        }
        __syncthreads();
        for (int base = 0; base < n; base += 4 * kMergeThreads) {
            uint32_t bin[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = base + j * kMergeThreads + tid;
                bin[j] = e < n ? order_key(rs[e]) >> 20 : uint32_t(kMergeBins);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (bin[j] < uint32_t(kMergeBins)) atomicAdd(&sh.hist[bin[j]], 1u);
        }
        __syncthreads();

        // ---- the bin of the k-th best: thread t owns the PER bins just below
        // kMergeBins - t*PER, so a prefix sum over threads counts the entries
        // at or above each thread's bins
        uint32_t c[PER];
        uint32_t cl = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            c[j] = sh.hist[kMergeBins - 1 - (tid * PER + j)];
            cl += c[j];
        }
        const uint32_t pw = wave_prefix_sum(cl);
        if (lane == 63) sh.w[wave] = pw;
        __syncthreads();
        uint32_t pre = pw;
#pragma unroll
        for (int v = 0; v < kMergeWaves; ++v) pre += v < wave ? sh.w[v] : 0u;
        const uint64_t bal = __ballot(pre >= uint32_t(k));
        if (lane == 0 && bal)
            atomicMin(&sh.first, wave * 64 + __ffsll(static_cast<unsigned long long>(bal)) - 1);
        __syncthreads();
        if (tid == sh.first) {
            uint32_t acc = pre - cl, ab = acc;
            int below = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const bool under = acc + c[j] < uint32_t(k);
                below += under ? 1 : 0;
                ab += under ? c[j] : 0u;
                acc += c[j];
            }
            sh.sel[0] = uint32_t(kMergeBins - 1 - (tid * PER + below));
            sh.sel[1] = ab;
        }
        __syncthreads();
        const uint32_t bstar = sh.sel[0];
        const int n_above = int(sh.sel[1]);     // entries in higher bins
        const int in_bin = int(sh.hist[bstar]);
        __syncthreads();

        uint32_t prefix, pmask;
        int need = k - n_above;                  // still to take, >= 1
        const bool fast = in_bin <= kMergeCap;
        if (fast) {
            // ---- higher bins to the row, the k-th bin into LDS in list order:
            // thread t takes entries [base + t*EPT, base + (t+1)*EPT), so a
            // scan of the per-thread candidate counts places them in order
            int cpos = 0;
            int step = 0;
            for (int base = 0; base < n; base += kMergeThreads * kMergeEpt, ++step) {
                const int e0 = base + tid * kMergeEpt;
                float sc[kMergeEpt];
                uint32_t u[kMergeEpt];
                int nc = 0;
#pragma unroll
                for (int j = 0; j < kMergeEpt; ++j) {
                    const bool valid = e0 + j < n;
                    sc[j] = valid ? rs[e0 + j] : 0.f;
                    u[j] = valid ? order_key(sc[j]) : 0u;
                }
#pragma unroll
                for (int j = 0; j < kMergeEpt; ++j) {
                    const bool valid = e0 + j < n;
                    const uint32_t bin = u[j] >> 20;
                    if (valid && bin > bstar) {
                        const int p = atomicAdd(&sh.out, 1);
                        if (p < n_above) {
                            oi[p] = ri[e0 + j];
                            os[p] = sc[j];
                        }
                    }
                    nc += (valid && bin == bstar) ? 1 : 0;
                }
                const uint32_t incl = wave_prefix_sum(uint32_t(nc));
                uint32_t *w2 = sh.w2[step & 1];  // alternate: one barrier per step
                if (lane == 63) w2[wave] = incl;
                __syncthreads();
                int wbase = 0, tot = 0;
#pragma unroll
                for (int v = 0; v < kMergeWaves; ++v) {
                    const int c2 = int(w2[v]);
                    wbase += v < wave ? c2 : 0;
                    tot += c2;
                }
                int pos = cpos + wbase + int(incl) - nc;
#pragma unroll
                for (int j = 0; j < kMergeEpt; ++j) {
                    if (e0 + j < n && (u[j] >> 20) == bstar) {
                        sh.cu[pos] = u[j];
                        sh.ci[pos] = ri[e0 + j];
                        ++pos;
                    }
                }
                cpos += tot;
            }
            __syncthreads();
            // ---- radix select among the in_bin candidates: bits 19..12, 11..4, 3..0
            prefix = bstar << 20;
            pmask = 0xFFF00000u;
            uint32_t *h = sh.hist;  // reused as a 256-bin histogram
            for (int pass = 0; pass < 3; ++pass) {
                const int shift = pass == 0 ? 12 : (pass == 1 ? 4 : 0);
                const uint32_t dm = pass == 2 ? 0xFu : 0xFFu;
                for (int i = tid; i < 256; i += kMergeThreads) h[i] = 0u;
                __syncthreads();
                for (int i = tid; i < in_bin; i += kMergeThreads) {
                    const uint32_t u = sh.cu[i];
                    if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & dm], 1u);
                }
                __syncthreads();
                digit_of_rank(h, need, sh.sel, lane, wave);
                prefix |= sh.sel[0] << shift;
                pmask |= dm << shift;
                need -= int(sh.sel[1]);
                __syncthreads();
            }
            // ---- larger keys of the bin, then the first `need` equal ones
            const int n_gt = k - need;
            int eq_base = 0;
            for (int base = 0; base < in_bin; base += kMergeThreads) {
                const int i = base + tid;
                const uint32_t u = i < in_bin ? sh.cu[i] : 0u;
                const bool gt = i < in_bin && u > prefix;
                const bool eq = i < in_bin && u == prefix;
                if (gt) {
                    const int p = atomicAdd(&sh.out, 1);
                    if (p < n_gt) {
                        oi[p] = sh.ci[i];
                        os[p] = key_to_float(u);
                    }
                }
                int tot;
                const int r = eq_base + block_rank(eq, sh.w, lane, wave, &tot);
                if (eq && r < need) {
                    oi[n_gt + r] = sh.ci[i];
                    os[n_gt + r] = key_to_float(u);
                }
                eq_base += tot;
            }
        } else {
            // ---- MSB-first radix select over the lists
            prefix = 0u;
            pmask = 0u;
            need = k;
            uint32_t *h = sh.hist;
            for (int shift = 24; shift >= 0; shift -= 8) {
                for (int i = tid; i < 256; i += kMergeThreads) h[i] = 0u;
                __syncthreads();
                for (int e = tid; e < n; e += kMergeThreads) {
                    const uint32_t u = order_key(rs[e]);
                    if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1u);
                }
                __syncthreads();
                digit_of_rank(h, need, sh.sel, lane, wave);
                prefix |= sh.sel[0] << shift;
                pmask |= 0xFFu << shift;
                need -= int(sh.sel[1]);
                __syncthreads();
            }
            const int n_gt = k - need;
            if (tid == 0) sh.out = 0;
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
                    const int p = atomicAdd(&sh.out, 1);
                    if (p < n_gt) {
                        oi[p] = ri[e];
                        os[p] = sc;
                    }
                }
                int tot;
                const int r = eq_base + block_rank(eq, sh.w, lane, wave, &tot);
                if (eq && r < need) {
                    oi[n_gt + r] = ri[e];
                    os[n_gt + r] = sc;
                }
                eq_base += tot;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_merge_splits(const Plan &p, const int32_t *part_idx, const float *part_score,
                               int32_t *out_idx, float *out_score, int num_cus, hipStream_t s)
{
    const int64_t rows = p.B * p.S;
    if (rows <= 0 || p.n_splits <= 1) return hipSuccess;
    const int64_t cap = int64_t(num_cus) * 4;
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
