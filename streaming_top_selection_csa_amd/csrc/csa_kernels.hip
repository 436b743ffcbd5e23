// csa_kernels.hip -- the key-range merge kernel and the dispatch of the
// scoring kernel (csa_stream.hpp) to its per-type instantiations.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_bitonic.hpp"
#include "csa_stream.hpp"

namespace csa {

// ------------------------------------------------------------ key-range merge

// Threads per row: 1,024 where rows are few and sorted here (short query
// blocks: more loads in flight per step and more hands in the LDS sort),
// 512 for the unsorted merge of many rows (measured faster there).
template <bool SORTED> constexpr int kMergeThreads = SORTED ? 1024 : 512;
constexpr int kMergeMaxWaves = 1024 / 64;
constexpr int kMergeBins = 4096;  // 16-bit order-key prefixes in a window (see below)
constexpr int kMergeCap = 6144;   // candidates of the k-th bin held in LDS
constexpr int kMergeEpt = 8;      // consecutive list entries per thread in the gather
// With 16-byte loads (k a multiple of 4, lists 16-byte aligned) each thread
// takes more entries per step, so that a row's passes need fewer dependent
// round trips to memory: the lists of short query blocks come from other
// XCDs and miss L2.
constexpr int kMergeHistV = 16;   // entries per thread per histogram step
constexpr int kMergeEptV = 16;    // entries per thread per gather step

struct MergeShared {
    uint32_t hist[kMergeBins];
    uint32_t cu[kMergeCap];
    int32_t ci[kMergeCap];
    uint32_t w[kMergeMaxWaves];
    uint32_t w2[2][kMergeMaxWaves];
    uint32_t sel[2];
    int first;
    int out;
    int anchor;
};

// Rank of this thread's flag among the flagged threads of the workgroup, in
// thread order, and their number (two barriers).
template <int NW>
__device__ __forceinline__ int block_rank(bool f, uint32_t *sw, int lane, int wave, int *total)
{
    const uint64_t m = __ballot(f);
    if (lane == 0) sw[wave] = uint32_t(__popcll(m));
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
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
// 16-bit prefixes of the order keys (a window of kMergeBins prefixes around
// the lists' leading entries) names the bin holding the k-th best; one more
// pass writes every entry of a higher bin and gathers that bin's entries, in
// list order, into LDS, where a radix select on the low 16 bits finishes.
// If the bin holds more than kMergeCap entries or is an end bin of the
// window (keys outside it are clamped there), an MSB-first 4 x 8-bit radix
// select over the lists takes its place.  Equal keys are
// taken in list order.  Padding entries (index -1, score -inf) order below
// every finite score and fill the row when fewer than k keys are visible.
// SORTED (rows of next_pow2(k) = pow2 <= kMaxFusedSort slots): the chosen
// entries go to LDS instead, as ascending 64-bit keys ~orderkey << 32 |
// index, and the row leaves sorted by (score desc, key index asc); out_score
// may then be null.
template <bool SORTED, bool VEC>
__global__ void __launch_bounds__(kMergeThreads<SORTED>)
merge_splits_kernel(const int32_t *__restrict__ pidx, const float *__restrict__ pscore,
                    int64_t rows, int G, int k, int pow2, int32_t *__restrict__ out_idx,
                    float *__restrict__ out_score)
{
    __shared__ MergeShared sh;
    __shared__ unsigned long long s_row[SORTED ? kMaxFusedSort : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = G * k;
    constexpr int NT = kMergeThreads<SORTED>;
    constexpr int NW = NT / 64;
    constexpr int PER = kMergeBins / NT;  // histogram bins per thread
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int32_t *ri = pidx + row * n;
        const float *rs = pscore + row * n;
        int32_t *oi = out_idx + row * k;
        float *os = out_score ? out_score + row * k : nullptr;
        // output slot p of the row: (index, score) with order key u
        auto put = [&](int p, uint32_t u, int32_t idx, float sc) {
            if constexpr (SORTED) {
                s_row[p] = (static_cast<unsigned long long>(~u) << 32) | uint32_t(idx);
            } else {
                oi[p] = idx;
                os[p] = sc;
            }
        };

        // ---- histogram of 16-bit order-key prefixes (128 bins per binade of
        // |score|) in a window of kMergeBins around an anchor: the largest
        // prefix among the G lists' first entries.  Keys outside the window
        // are clamped into its end bins (the bins stay in key order); a k-th
        // best in an end bin takes the exact fallback below.  Bins this fine
        // spread the LDS atomics, which on a window of whole binades pile
        // onto a few counters.
#pragma unroll
        for (int j = 0; j < PER; ++j) sh.hist[tid * PER + j] = 0u;
        if (tid == 0) {
            sh.first = NT;
            sh.out = 0;
        }
        if (wave == 0) {
            int a = 0;
            for (int r = lane; r < G; r += 64) a = max(a, int(order_key(rs[int64_t(r) * k]) >> 16));
            a = wave_max(a);
            if (lane == 0) sh.anchor = a;
        }
        __syncthreads();
        const int lo16 = sh.anchor - kMergeBins / 2;  // prefix of bin 0
        auto bin_of = [&](uint32_t u) -> uint32_t {
            const int b = int(u >> 16) - lo16;
            return uint32_t(b < 0 ? 0 : (b > kMergeBins - 1 ? kMergeBins - 1 : b));
        };
        constexpr int HB = VEC ? kMergeHistV : 4;  // entries per thread per step
        for (int base = 0; base < n; base += HB * NT) {
            uint32_t bin[HB];
            if constexpr (VEC) {
                // thread t reads entries [base + t*HB, base + (t+1)*HB); n is
                // a multiple of 4, so a group of 4 lies wholly inside or out
#pragma unroll
                for (int q = 0; q < HB / 4; ++q) {
                    const int e = base + tid * HB + 4 * q;
                    if (e < n) {
                        const float4 v = *reinterpret_cast<const float4 *>(rs + e);
                        bin[4 * q] = bin_of(order_key(v.x));
                        bin[4 * q + 1] = bin_of(order_key(v.y));
                        bin[4 * q + 2] = bin_of(order_key(v.z));
                        bin[4 * q + 3] = bin_of(order_key(v.w));
                    } else {
                        bin[4 * q] = bin[4 * q + 1] = bin[4 * q + 2] = bin[4 * q + 3] =
                            uint32_t(kMergeBins);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < HB; ++j) {
                    const int e = base + j * NT + tid;
                    bin[j] = e < n ? bin_of(order_key(rs[e])) : uint32_t(kMergeBins);
                }
            }
#pragma unroll
            for (int j = 0; j < HB; ++j)
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
        for (int v = 0; v < NW; ++v) pre += v < wave ? sh.w[v] : 0u;
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
        // (a clamped end bin holds keys of different prefixes)
        const bool fast = in_bin <= kMergeCap && bstar > 0u && bstar < uint32_t(kMergeBins - 1);
        if (fast) {
            // ---- higher bins to the row, the k-th bin into LDS in list order:
            // thread t takes entries [base + t*EPT, base + (t+1)*EPT), so a
            // scan of the per-thread candidate counts places them in order
            // (with 16-byte loads the key indices are read together with the
            // scores rather than after them: one round trip per step)
            constexpr int EPT = VEC ? kMergeEptV : kMergeEpt;
            int cpos = 0;
            int step = 0;
            for (int base = 0; base < n; base += NT * EPT, ++step) {
                const int e0 = base + tid * EPT;
                float sc[EPT];
                uint32_t u[EPT];
                int32_t id[VEC ? EPT : 1];
                int nc = 0;
                if constexpr (VEC) {
#pragma unroll
                    for (int q = 0; q < EPT / 4; ++q) {
                        const int e = e0 + 4 * q;
                        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                        int4 x = make_int4(0, 0, 0, 0);
                        if (e < n) {
                            v = *reinterpret_cast<const float4 *>(rs + e);
                            x = *reinterpret_cast<const int4 *>(ri + e);
                        }
                        sc[4 * q] = v.x, sc[4 * q + 1] = v.y, sc[4 * q + 2] = v.z, sc[4 * q + 3] = v.w;
                        id[4 * q] = x.x, id[4 * q + 1] = x.y, id[4 * q + 2] = x.z, id[4 * q + 3] = x.w;
                    }
#pragma unroll
                    for (int j = 0; j < EPT; ++j) u[j] = e0 + j < n ? order_key(sc[j]) : 0u;
                } else {
#pragma unroll
                    for (int j = 0; j < EPT; ++j) {
                        const bool valid = e0 + j < n;
                        sc[j] = valid ? rs[e0 + j] : 0.f;
                        u[j] = valid ? order_key(sc[j]) : 0u;
                    }
                }
                auto index_of = [&](int j) {
                    if constexpr (VEC) return id[j];
                    else return ri[e0 + j];
                };
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    const bool valid = e0 + j < n;
                    const uint32_t bin = bin_of(u[j]);
                    if (valid && bin > bstar) {
                        const int p = atomicAdd(&sh.out, 1);
                        if (p < n_above) put(p, u[j], index_of(j), sc[j]);
                    }
                    nc += (valid && bin == bstar) ? 1 : 0;
                }
                const uint32_t incl = wave_prefix_sum(uint32_t(nc));
                uint32_t *w2 = sh.w2[step & 1];  // alternate: one barrier per step
                if (lane == 63) w2[wave] = incl;
                __syncthreads();
                int wbase = 0, tot = 0;
#pragma unroll
                for (int v = 0; v < NW; ++v) {
                    const int c2 = int(w2[v]);
                    wbase += v < wave ? c2 : 0;
                    tot += c2;
                }
                int pos = cpos + wbase + int(incl) - nc;
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    if (e0 + j < n && bin_of(u[j]) == bstar) {
                        sh.cu[pos] = u[j];
                        sh.ci[pos] = index_of(j);
                        ++pos;
                    }
                }
                cpos += tot;
            }
            __syncthreads();
            // ---- radix select among the in_bin candidates (one 16-bit
            // prefix): bits 15..8, then 7..0
            prefix = uint32_t(lo16 + int(bstar)) << 16;
            pmask = 0xFFFF0000u;
            uint32_t *h = sh.hist;  // reused as a 256-bin histogram
            for (int pass = 0; pass < 2; ++pass) {
                const int shift = pass == 0 ? 8 : 0;
                const uint32_t dm = 0xFFu;
                for (int i = tid; i < 256; i += NT) h[i] = 0u;
                __syncthreads();
                for (int i = tid; i < in_bin; i += NT) {
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
            for (int base = 0; base < in_bin; base += NT) {
                const int i = base + tid;
                const uint32_t u = i < in_bin ? sh.cu[i] : 0u;
                const bool gt = i < in_bin && u > prefix;
                const bool eq = i < in_bin && u == prefix;
                if (gt) {
                    const int p = atomicAdd(&sh.out, 1);
                    if (p < n_gt) put(p, u, sh.ci[i], key_to_float(u));
                }
                int tot;
                const int r = eq_base + block_rank<NW>(eq, sh.w, lane, wave, &tot);
                if (eq && r < need) put(n_gt + r, u, sh.ci[i], key_to_float(u));
                eq_base += tot;
            }
        } else {
            // ---- MSB-first radix select over the lists
            prefix = 0u;
            pmask = 0u;
            need = k;
            uint32_t *h = sh.hist;
            for (int shift = 24; shift >= 0; shift -= 8) {
                for (int i = tid; i < 256; i += NT) h[i] = 0u;
                __syncthreads();
                for (int e = tid; e < n; e += NT) {
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
            for (int base = 0; base < n; base += NT) {
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
                    if (p < n_gt) put(p, u, ri[e], sc);
                }
                int tot;
                const int r = eq_base + block_rank<NW>(eq, sh.w, lane, wave, &tot);
                if (eq && r < need) put(n_gt + r, u, ri[e], sc);
                eq_base += tot;
            }
        }
        __syncthreads();
        if constexpr (SORTED) {
            // the k chosen entries, padding slots after them, sorted in LDS
            for (int e = k + tid; e < pow2; e += NT) s_row[e] = ~0ull;
            __syncthreads();
            lds_bitonic_sort(s_row, pow2, tid, NT);
            for (int e = tid; e < k; e += NT) {
                const unsigned long long key = s_row[e];
                oi[e] = int32_t(uint32_t(key));
                if (os) os[e] = key_to_float(~uint32_t(key >> 32));
            }
            __syncthreads();
        }
    }
}

hipError_t launch_merge_splits(const Plan &p, const int32_t *part_idx, const float *part_score,
                               int32_t *out_idx, float *out_score, int num_cus, hipStream_t s)
{
    const int64_t rows = p.B * p.S;
    if (rows <= 0 || p.n_splits <= 1) return hipSuccess;
    const int64_t cap = int64_t(num_cus) * 4;
    const int grid = int(rows < cap ? rows : cap);
    // 16-byte loads when every row's lists start 16-byte aligned
    const bool vec = p.k % 4 == 0 && (reinterpret_cast<uintptr_t>(part_idx) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(part_score) & 15) == 0;
#define CSA_MERGE_LAUNCH(SORTED, VEC)                                                          \
    hipLaunchKernelGGL((merge_splits_kernel<SORTED, VEC>), dim3(grid), dim3(kMergeThreads<SORTED>), 0, \
                       s, part_idx, part_score, rows, p.n_splits, p.k, p.sort_pow2, out_idx,    \
                       out_score)
    if (p.merge_sorts) {
        if (vec) CSA_MERGE_LAUNCH(true, true);
        else CSA_MERGE_LAUNCH(true, false);
    } else {
        if (vec) CSA_MERGE_LAUNCH(false, true);
        else CSA_MERGE_LAUNCH(false, false);
    }
#undef CSA_MERGE_LAUNCH
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
