// csa_stream.hpp -- the gfx950 scoring kernel of the CSA lightning-indexer
// top-k and its device helpers (included by the csa_stream_*.hip files, one
// per operand type and head dimension, and by csa_kernels.hip).
//
// StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
// Top-k (Abstract): each query position rates the compressed keys with the
// lightning indexer and keeps its k best, folding the keys in chunk by chunk
// so that no [B,S,H_I,T] tensor is ever formed.
// Here that is one persistent kernel:
//
//   stream_topk_kernel  Each wave owns 64 (position, head) rows of q, held in
//       VGPRs as MFMA A-operands.  The workgroup stages tiles of KT keys of
//       k_cmp in LDS (64 or 128 keys; a ring of three, two tiles ahead, or
//       of two).  Per 64 keys a wave runs the [64 rows x D] x [D x 64 keys]
//       contraction on the matrix cores (bf16 32x32x16 or fp8 32x32x64),
//       then in registers applies ReLU, the per-head weights and the head
//       sum, and the causal cut.  A score
//       survives only if it beats the position's running threshold, which a
//       per-position histogram of the candidates raises to just below the
//       k-th best so far; survivors are appended, in key order, to the
//       position's candidate log.  A full log (k + chunk entries) is
//       compacted to the entries above the threshold (the merge step, with an
//       exact radix select as the fallback).  At the end the histogram and
//       one pass over the log give the exact top-min(k, n_vis) set, which is
//       sorted in registers and written to the output row.
//
// With key ranges (SPLIT) a unit is one (query block, key range) pair and
// the kernel leaves the exact top-k of the range in a partial list; the merge
// kernel of csa_kernels.hip combines the ranges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_bitonic.hpp"
#include "csa_dma.hpp"
#include "csa_kernels.hpp"
#include "csa_order_key.hpp"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

// max(x, 0) for finite x as one signed-integer max on the bit pattern:
// negative floats (and -0) have the sign bit set, i.e. are negative ints.
__device__ __forceinline__ float relu(float x)
{
    const int b = __float_as_int(x);
    return __int_as_float(b > 0 ? b : 0);
}

// The smallest score whose order key exceeds tau, so that for a finite
// score x, order_key(x) > tau <=> x >= score_floor(tau).  Keys below that of
// -inf (tau + 1 has no float) give -inf: every finite score passes.  Should
// the compare flush denormals, it can only let extra scores pass.
__device__ __forceinline__ float score_floor(uint32_t tau)
{
    return tau < 0x007FFFFFu ? -__builtin_huge_valf() : key_to_float(tau + 1u);
}

// Number of set bits of `m` in lanes below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

__device__ __forceinline__ int64_t n_visible(int64_t t, int64_t T, int m)
{
    const int64_t n = (t + 1) / m;
    return n < T ? n : T;
}

// LDS traffic of one wave is ordered; this keeps the compiler from moving
// shared-memory accesses across the point and waits for them to finish
// (lgkmcnt only: a fence would also wait for every global store and key-tile
// load in flight).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// *p += v on an LDS word, without returning the old value.  Inline assembly
// because the compiler makes an LDS atomic wait for all outstanding vector
// memory operations (the key-tile loads into LDS and the candidate-log
// stores) when it cannot prove the addresses disjoint; the counters updated
// here never share memory with a key tile.  One wave's LDS operations run in
// issue order, so its later reads of the word see the sum.
__device__ __forceinline__ void lds_add(uint32_t *p, uint32_t v)
{
    const uint32_t a = uint32_t(uintptr_t((__attribute__((address_space(3))) uint32_t *)p));
    __asm__ volatile("ds_add_u32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// Makes global stores of every lane of the wave visible to global loads of
// the other lanes: waits until this wave's stores are done, then a fence at
// workgroup scope (all lanes run on one CU, whose vector L1 is written
// through).  An agent-scope fence would also write back and invalidate the
// XCD's whole L2 each time, evicting the key tiles that the other
// workgroups of the XCD are streaming.
__device__ __forceinline__ void wave_global_sync()
{
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), on DPP row shifts
// and row broadcasts (no LDS round trips).
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// For lane l < 32 returns x[l] + x[l+32]; for lane l >= 32 returns
// y[l-32] + y[l] (one v_permlane32_swap exchanges the crossing halves).
__device__ __forceinline__ float cross_half_sum(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA operand traits: bf16 32x32x16 (8 bf16 per lane) or fp8 e4m3
// 32x32x64 (32 codes per lane, unit E8M0 block scales).  Lane l supplies row
// (or column) l % 32 and the K-slice half = l / 32 of each K step; A and B
// use the same slicing, so any slicing the hardware applies pairs them up.
template <bool FP8>
struct Op;

template <>
struct Op<false> {
    using T = bf16x8_t;
    static constexpr int KSTEP = 16;       // K per instruction
    static constexpr int ESZ = 2;          // bytes per element
    static constexpr int LANE_BYTES = 16;  // operand bytes per lane
    static __device__ __forceinline__ T load(const unsigned char *p)
    {
        return __builtin_bit_cast(T, *reinterpret_cast<const u32x4_t *>(p));
    }
    static __device__ __forceinline__ T zero() { return __builtin_bit_cast(T, u32x4_t{0, 0, 0, 0}); }
    // operand chunk c of an LDS key row stored with chunk swizzle `swz`
    static __device__ __forceinline__ T load_swz(const unsigned char *row, int c, int swz)
    {
        return load(row + ((c ^ swz) << 4));
    }
    static __device__ __forceinline__ f32x16_t mma(T a, T b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Op<true> {
    using T = i32x8_t;
    static constexpr int KSTEP = 64;
    static constexpr int ESZ = 1;
    static constexpr int LANE_BYTES = 32;
    static __device__ __forceinline__ T load(const unsigned char *p)
    {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(p);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(p + 16);
        return T{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    }
    static __device__ __forceinline__ T zero() { return T{0, 0, 0, 0, 0, 0, 0, 0}; }
    static __device__ __forceinline__ T load_swz(const unsigned char *row, int c, int swz)
    {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(row + ((c ^ swz) << 4));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(row + (((c + 1) ^ swz) << 4));
        return T{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    }
    static __device__ __forceinline__ f32x16_t mma(T a, T b, f32x16_t c)
    {
        // formats 0/0 = E4M3 for A and B; scale exponent 127 = 2^0
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

// ------------------------------------------------------- candidate merging

constexpr int kBatch = 8;  // log entries per lane in flight in the log passes
// Consecutive log entries one lane reads in the final staging pass; the
// planner keeps every log's capacity a multiple of it.
constexpr int kLogGroup = kLogCapMultiple;

// The log lu/li[0..n) holds candidates of one position in ascending key
// order, n > k.  Finds the k-th best under (score desc, key asc) with a
// 4 x 8-bit radix select on the order keys, compacts the log in place to
// exactly the k best (still in key order) and returns the k-th best key.
// rhist: 256 words of LDS private to the wave.
static __device__ __noinline__ uint32_t merge_log(uint32_t *lu, int32_t *li, int n, int k,
                                           uint32_t *rhist, int lane)
{
    wave_global_sync();
    uint32_t prefix = 0u, pmask = 0u;
    int kk = k;  // rank, from the top, of the wanted key among prefix matches
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = lane; i < 256; i += 64) rhist[i] = 0u;
        wave_lds_sync();
#pragma unroll 1
        for (int base = 0; base < n; base += 64 * kBatch) {
            uint32_t u[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int e = base + 64 * j + lane;
                u[j] = e < n ? lu[e] : 0u;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int e = base + 64 * j + lane;
                if (e < n && (u[j] & pmask) == prefix) atomicAdd(&rhist[(u[j] >> shift) & 255u], 1u);
            }
        }
        wave_lds_sync();
        const uint32_t c0 = rhist[4 * lane], c1 = rhist[4 * lane + 1];
        const uint32_t c2 = rhist[4 * lane + 2], c3 = rhist[4 * lane + 3];
        const uint32_t cl = c0 + c1 + c2 + c3;
        uint32_t sfx = cl;  // count in digits >= 4*lane
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_down(sfx, off);
            if (lane + off < 64) sfx += o;
        }
        const uint32_t want = uint32_t(kk);
        const uint64_t bal = __ballot(sfx >= want);
        const int L = 63 - __clzll(bal);
        const uint32_t above = sfx - cl;  // count in digits > 4*lane+3
        int d;
        uint32_t ab;
        if (above + c3 >= want) {
            d = 4 * lane + 3;
            ab = above;
        } else if (above + c3 + c2 >= want) {
            d = 4 * lane + 2;
            ab = above + c3;
        } else if (above + c3 + c2 + c1 >= want) {
            d = 4 * lane + 1;
            ab = above + c3 + c2;
        } else {
            d = 4 * lane;
            ab = above + c3 + c2 + c1;
        }
        d = __builtin_amdgcn_readlane(d, L);
        ab = __builtin_amdgcn_readlane(ab, L);
        kk -= int(ab);
        prefix |= uint32_t(d) << shift;
        pmask |= 0xFFu << shift;
        wave_lds_sync();
    }
    // prefix is the k-th best key; keep every larger key and the first kk
    // equal ones (the lowest key indices, since the log is in key order).
    int wpos = 0, eq_seen = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += 64 * kBatch) {
        uint32_t u[kBatch];
        int32_t id[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int e = base + 64 * j + lane;
            u[j] = e < n ? lu[e] : 0u;
            id[j] = e < n ? li[e] : 0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const bool valid = base + 64 * j + lane < n;
            const bool gt = valid && u[j] > prefix;
            const bool eq = valid && u[j] == prefix;
            const uint64_t meq = __ballot(eq);
            const bool keep = gt || (eq && eq_seen + lanes_below(meq) < kk);
            const uint64_t mk = __ballot(keep);
            if (keep) {
                const int p = wpos + lanes_below(mk);
                lu[p] = u[j];
                li[p] = id[j];
            }
            wpos += __popcll(mk);
            eq_seen += __popcll(meq);
        }
    }
    wave_global_sync();
    return prefix;
}

// Drops, in place and in order, every log entry whose key is below tau
// (such an entry is beaten by at least k earlier ones); returns the count.
static __device__ __noinline__ int compact_log(uint32_t *lu, int32_t *li, int n, uint32_t tau, int lane)
{
    wave_global_sync();
    int wpos = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += 64 * kBatch) {
        uint32_t u[kBatch];
        int32_t id[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int e = base + 64 * j + lane;
            u[j] = e < n ? lu[e] : 0u;
            id[j] = e < n ? li[e] : 0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const bool keep = base + 64 * j + lane < n && u[j] >= tau;
            const uint64_t mk = __ballot(keep);
            if (keep) {
                const int p = wpos + lanes_below(mk);
                lu[p] = u[j];
                li[p] = id[j];
            }
            wpos += __popcll(mk);
        }
    }
    wave_global_sync();
    return wpos;
}

// ---------------------------------------------------- threshold histogram
//
// Each position keeps, in LDS, counts of its live candidates over NB bins
// of the order key u: bin = (u >> 16) - base, i.e. 128 bins per binade of
// |score| (sign, 8 exponent bits, 7 mantissa bits), clamped to bin 0 below
// the window.  If the bins at and above b hold at least k candidates, every
// later key whose u is below the lower edge of bin b is beaten by k earlier
// ones, so the filter threshold may rise to that edge minus one without
// reading the log; bins below b are then dead and are cleared.

template <int NB>
struct Hist {
    static constexpr int PER = NB >= 64 ? NB / 64 : 1;  // bins per lane

    static __device__ __forceinline__ void clear(uint32_t *h, int lane)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (lane * PER + j < NB) h[lane * PER + j] = 0u;
    }

    // Highest bin b with at least `need` counts in bins >= b, or -1.
    // Lane l owns the PER bins just below NB - l*PER (lane 0 the top ones),
    // so a prefix sum over lanes counts everything at or above a lane's bins.
    static __device__ __forceinline__ int top_bin(const uint32_t *h, int need, int lane)
    {
        uint32_t c[PER];
        uint32_t cl = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = NB - 1 - (lane * PER + j);
            c[j] = b >= 0 ? h[b] : 0u;
            cl += c[j];
        }
        const uint32_t pre = wave_prefix_sum(cl);
        const uint64_t bal = __ballot(pre >= uint32_t(need));
        if (bal == 0) return -1;
        const int L = __ffsll(static_cast<unsigned long long>(bal)) - 1;
        // in lane L the running count reaches `need` at its first bin j
        // whose inclusive count does; the counts before it are the j below
        uint32_t acc = pre - cl;
        int below = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            acc += c[j];
            below += acc < uint32_t(need) ? 1 : 0;
        }
        return __builtin_amdgcn_readlane(NB - 1 - (lane * PER + below), L);
    }

    // As top_bin; *above receives the count in the bins above the result.
    static __device__ __forceinline__ int top_bin_above(const uint32_t *h, int need, int lane,
                                                        uint32_t *above)
    {
        uint32_t c[PER];
        uint32_t cl = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = NB - 1 - (lane * PER + j);
            c[j] = b >= 0 ? h[b] : 0u;
            cl += c[j];
        }
        const uint32_t pre = wave_prefix_sum(cl);
        const uint64_t bal = __ballot(pre >= uint32_t(need));
        if (bal == 0) return -1;
        const int L = __ffsll(static_cast<unsigned long long>(bal)) - 1;
        uint32_t acc = pre - cl, ab = acc;
        int below = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const bool under = acc + c[j] < uint32_t(need);
            below += under ? 1 : 0;
            acc += c[j];
            ab += under ? c[j] : 0u;
        }
        *above = __builtin_amdgcn_readlane(ab, L);
        return __builtin_amdgcn_readlane(NB - 1 - (lane * PER + below), L);
    }

    static __device__ __forceinline__ void zero_below(uint32_t *h, int b, int lane)
    {
        const int lim = (b < NB ? b : NB) - lane * PER;  // bins j < lim of this lane
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (j < lim) h[lane * PER + j] = 0u;
    }

    // Moves the window up by delta > 0 bins; counts falling below it are
    // clamped into bin 0.
    static __device__ __forceinline__ void shift(uint32_t *h, int delta, int lane)
    {
        uint32_t c[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) c[j] = lane * PER + j < NB ? h[lane * PER + j] : 0u;
        wave_lds_sync();
        clear(h, lane);
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int nb = lane * PER + j - delta;
            if (c[j]) lds_add(&h[nb > 0 ? nb : 0], c[j]);
        }
        wave_lds_sync();
    }
};

// Maximum over the 64 lanes, wave-uniform: a running maximum on DPP row
// shifts and row broadcasts leaves the total in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_max_step(int v)
{
    const int o = __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
    return o > v ? o : v;
}

__device__ __forceinline__ int wave_max(int v)
{
    v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
    v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15
    v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

// Re-counts the k log entries left by an exact merge (window unchanged).
template <int NB>
__device__ __noinline__ void hist_recount(uint32_t *h, int hbase, const uint32_t *lu, int n, int lane)
{
    wave_global_sync();
    Hist<NB>::clear(h, lane);
    wave_lds_sync();
#pragma unroll 1
    for (int base = 0; base < n; base += 64 * kBatch) {
        uint32_t u[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int e = base + 64 * j + lane;
            u[j] = e < n ? lu[e] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (base + 64 * j + lane < n) {
                const int lb = int(u[j] >> 16) - hbase;
                atomicAdd(&h[lb > 0 ? (lb < NB ? lb : NB - 1) : 0], 1u);
            }
        }
    }
    wave_lds_sync();
}

// Radix digit pick over the 256 counts in rhist: the digit d at which the
// count from the top digit down first reaches `want` (>= 1), and in *above
// the count in the digits above d.  Wave-uniform results.
__device__ __forceinline__ int pick_digit(const uint32_t *rhist, uint32_t want, int lane,
                                          uint32_t *above)
{
    // lane 0 owns the top digits: prefix sum over reversed digit order
    const uint32_t r0 = rhist[255 - 4 * lane], r1 = rhist[254 - 4 * lane];
    const uint32_t r2 = rhist[253 - 4 * lane], r3 = rhist[252 - 4 * lane];
    const uint32_t rl = r0 + r1 + r2 + r3;
    const uint32_t pre = wave_prefix_sum(rl);
    const uint64_t bal = __ballot(pre >= want);
    const int L = __ffsll(static_cast<unsigned long long>(bal)) - 1;
    const uint32_t acc = pre - rl;
    int d = 252 - 4 * lane;
    uint32_t ab = acc;
    if (acc + r0 >= want) {
        d = 255 - 4 * lane;
    } else if (acc + r0 + r1 >= want) {
        d = 254 - 4 * lane;
        ab = acc + r0;
    } else if (acc + r0 + r1 + r2 >= want) {
        d = 253 - 4 * lane;
        ab = acc + r0 + r1;
    } else {
        ab = acc + r0 + r1 + r2;
    }
    *above = __builtin_amdgcn_readlane(ab, L);
    return __builtin_amdgcn_readlane(d, L);
}

// Radix select, in LDS, of the `need` best of n candidates (cu, ci) whose
// order keys all lie in [lo, lo + 2^shift) (shift in {0, 8, 16}); hands
// each chosen one to put(rank, key, index), ranks 0..need-1, candidates
// kept in their LDS order (ascending key index among ties).
template <typename Put>
__device__ __forceinline__ void select_candidates(const uint32_t *cu, const int32_t *ci, int n,
                                                  int need, uint32_t lo, int shift,
                                                  uint32_t *rhist, int lane, Put put)
{
    uint32_t prefix = lo, pmask = shift >= 32 ? 0u : ~((1u << shift) - 1u);
    int kk = need;
#pragma unroll 1
    for (int sh = shift - 8; sh >= 0; sh -= 8) {
        for (int i = lane; i < 256; i += 64) rhist[i] = 0u;
        wave_lds_sync();
        for (int e = lane; e < n; e += 64) {
            const uint32_t u = cu[e];
            if ((u & pmask) == prefix) atomicAdd(&rhist[(u >> sh) & 255u], 1u);
        }
        wave_lds_sync();
        uint32_t ab = 0u;
        const int d = pick_digit(rhist, uint32_t(kk), lane, &ab);
        kk -= int(ab);
        prefix |= uint32_t(d) << sh;
        pmask |= 0xFFu << sh;
        wave_lds_sync();
    }
    int wpos = 0, eq_seen = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += 64) {
        const int e = base + lane;
        const bool valid = e < n;
        const uint32_t u = valid ? cu[e] : 0u;
        const bool gt = valid && u > prefix;
        const bool eq = valid && u == prefix;
        const uint64_t meq = __ballot(eq);
        const bool keep = gt || (eq && eq_seen + lanes_below(meq) < kk);
        const uint64_t mk = __ballot(keep);
        if (keep) put(wpos + lanes_below(mk), u, ci[e]);
        wpos += __popcll(mk);
        eq_seen += __popcll(meq);
    }
}

// Writes the min(k, cnt) best entries of a position's log (in any order)
// and the padding to its output row.  The threshold histogram names the
// bin holding the k-th best and counts what lies above it, so one pass
// over the log writes every entry above that bin and gathers the bin's
// entries into LDS (cu/ci, cap entries), where a short radix select picks
// the rest.  Falls back to the exact merge of the whole log when the bin
// is the clamped bottom bin, holds more than cap entries, or the counts
// disagree.
template <int NB>
__device__ __noinline__ void final_select(uint32_t *lu, int32_t *li, int cnt, int k,
                                          const uint32_t *h, int hbase, uint32_t *cu,
                                          int32_t *ci, int cap, uint32_t *rhist,
                                          int32_t *oi, float *os, int lane)
{
    wave_global_sync();
    wave_lds_sync();
    int wpos = 0;
    bool done = false;
    if (cnt <= k) {
        // every log entry is a result (see the filter rule)
#pragma unroll 1
        for (int e = lane; e < cnt; e += 64) {
            oi[e] = li[e];
            os[e] = key_to_float(lu[e]);
        }
        wpos = cnt;
        done = true;
    } else {
        uint32_t above = 0u;
        const int b = Hist<NB>::top_bin_above(h, k, lane, &above);
        const int g = hbase + b;
        const uint32_t nb = b >= 0 ? h[b] : 0u;
        if (b > 0 && g > 0 && g < 65535 && nb <= uint32_t(cap) && int(above) < k) {
            wpos = 0;
            const uint32_t lo = uint32_t(g) << 16, hi = uint32_t(g + 1) << 16;
            int cpos = 0;
#pragma unroll 1
            for (int base = 0; base < cnt; base += 64 * kBatch) {
                uint32_t u[kBatch];
                int32_t id[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int e = base + 64 * j + lane;
                    u[j] = e < cnt ? lu[e] : 0u;
                    id[j] = e < cnt ? li[e] : 0;
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const bool valid = base + 64 * j + lane < cnt;
                    const bool sel = valid && u[j] >= hi;
                    const bool cand = valid && u[j] >= lo && u[j] < hi;
                    const uint64_t ms = __ballot(sel);
                    const uint64_t mc = __ballot(cand);
                    const int ps = wpos + lanes_below(ms);
                    const int pc = cpos + lanes_below(mc);
                    if (sel && ps < k) {
                        oi[ps] = id[j];
                        os[ps] = key_to_float(u[j]);
                    }
                    if (cand && pc < cap) {
                        cu[pc] = u[j];
                        ci[pc] = id[j];
                    }
                    wpos += __popcll(ms);
                    cpos += __popcll(mc);
                }
            }
            wave_lds_sync();
            // the counts of this pass decide: with wpos < k <= wpos + cpos
            // the result is every entry above the bin plus the best k - wpos
            // of the bin (ties in log order, i.e. by ascending key)
            if (wpos < k && wpos + cpos >= k && cpos <= cap) {
                int32_t *const oo = oi + wpos;
                float *const so = os + wpos;
                select_candidates(cu, ci, cpos, k - wpos, uint32_t(g) << 16, 16, rhist, lane,
                                  [&](int p, uint32_t u, int32_t id) {
                                      oo[p] = id;
                                      so[p] = key_to_float(u);
                                  });
                wpos = k;
                done = true;
            }
        }
    }
    if (!done) {
        merge_log(lu, li, cnt, k, rhist, lane);
#pragma unroll 1
        for (int e = lane; e < k; e += 64) {
            oi[e] = li[e];
            os[e] = key_to_float(lu[e]);
        }
        wpos = k;
    }
#pragma unroll 1
    for (int e = wpos + lane; e < k; e += 64) {
        oi[e] = -1;
        os[e] = -__builtin_inff();
    }
}

// ------------------------------------------------- final selection + sort
//
// The wave's staging area holds up to kStageSlots (order key, key index)
// pairs in two LDS arrays; slot p lives at word stage_word(p), an XOR
// swizzle that keeps both the blocked (lane l: slots l*E .. l*E+E-1) and the
// striped (slot j*64 + lane) accesses of the sort on distinct banks.

constexpr int kStageSlots = 2048;  // largest next_pow2(k) sorted in the scoring kernel

__device__ __forceinline__ int stage_word(int p) { return p ^ ((p >> 5) & 31); }

// Leaves the min(k, cnt) best entries of a position's log, in no particular
// order, in staging slots [0, n) and returns n.  The threshold histogram
// names the bin holding the k-th best and counts what lies above it.  While
// that bin holds more entries than the candidate buffer, one counting pass
// over the log narrows it by the next 8 bits of the order key.  One pass
// then stages every entry above the range and gathers the range's entries
// into the candidate buffer (the position's histogram words, free by then),
// where a short radix select picks the rest; a range narrowed to a single
// order key instead stages its first entries in log order (the lowest key
// indices).  Falls back to the exact merge of the whole log when the bin is
// the clamped bottom bin or the counts disagree.
template <int NB>
__device__ __forceinline__ int stage_select(uint32_t *lu, int32_t *li, int cnt, int k, uint32_t *h,
                                         int hbase, uint32_t *su, uint32_t *si, uint32_t *rhist,
                                         int lane)
{
    constexpr int CAP = NB / 2;  // candidate entries that fit the histogram words
    wave_global_sync();
    wave_lds_sync();
    if (cnt <= k) {
        // every log entry is a result (see the filter rule)
#pragma unroll 1
        for (int e = lane; e < cnt; e += 64) {
            su[stage_word(e)] = lu[e];
            si[stage_word(e)] = uint32_t(li[e]);
        }
        return cnt;
    }
    uint32_t above = 0u;
    const int b = Hist<NB>::top_bin_above(h, k, lane, &above);
    const int g = hbase + b;
    uint32_t nb = b >= 0 ? h[b] : 0u;
    if (b > 0 && g > 0 && g < 65535 && int(above) < k) {
        uint32_t lo = uint32_t(g) << 16;
        int shift = 16;  // the k-th best lies in [lo, lo + 2^shift)
#pragma unroll 1
        while (nb > uint32_t(CAP) && shift > 0) {
            const uint32_t hi = lo + (1u << shift);
            shift -= 8;
            for (int i = lane; i < 256; i += 64) rhist[i] = 0u;
            wave_lds_sync();
#pragma unroll 1
            for (int base = 0; base < cnt; base += 64 * kBatch) {
                uint32_t u[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int e = base + 64 * j + lane;
                    u[j] = e < cnt ? lu[e] : 0u;
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    if (u[j] >= lo && u[j] < hi) atomicAdd(&rhist[(u[j] >> shift) & 255u], 1u);
            }
            wave_lds_sync();
            uint32_t ab = 0u;
            const int d = pick_digit(rhist, uint32_t(k) - above, lane, &ab);
            above += ab;
            nb = rhist[d];
            lo += uint32_t(d) << shift;
            wave_lds_sync();
        }
        const uint32_t hi = lo + (1u << shift);
        const bool direct = nb > uint32_t(CAP);  // one order key left: take the first ones
        const int need = k - int(above);
        uint32_t *const cu = h;
        int32_t *const ci = reinterpret_cast<int32_t *>(h + CAP);
        int wpos = 0, cpos = 0;
        // Each lane takes kLogGroup consecutive entries with two 16-byte
        // loads per array (the log's capacity is a multiple of kLogGroup, so
        // a group that starts below cnt lies inside it).  Ranks come from
        // the lanes' counts and one prefix sum per kind, so the entries
        // keep their log order.
#pragma unroll 1
        for (int base = 0; base < cnt; base += 64 * kLogGroup) {
            const int e0 = base + lane * kLogGroup;
            uint32_t u[kLogGroup];
            int32_t id[kLogGroup];
            if (e0 < cnt) {
                const uint4 *pu = reinterpret_cast<const uint4 *>(lu + e0);
                const int4 *pi = reinterpret_cast<const int4 *>(li + e0);
#pragma unroll
                for (int v = 0; v < kLogGroup / 4; ++v) {
                    const uint4 x = pu[v];
                    const int4 y = pi[v];
                    u[4 * v] = x.x, u[4 * v + 1] = x.y, u[4 * v + 2] = x.z, u[4 * v + 3] = x.w;
                    id[4 * v] = y.x, id[4 * v + 1] = y.y, id[4 * v + 2] = y.z, id[4 * v + 3] = y.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < kLogGroup; ++j) u[j] = 0u, id[j] = 0;
            }
            bool sel[kLogGroup], cand[kLogGroup];
            uint32_t ns = 0u, nc = 0u;
#pragma unroll
            for (int j = 0; j < kLogGroup; ++j) {
                const bool valid = e0 + j < cnt;
                sel[j] = valid && u[j] >= hi;
                cand[j] = valid && u[j] >= lo && u[j] < hi;
                ns += sel[j] ? 1u : 0u;
                nc += cand[j] ? 1u : 0u;
            }
            const uint32_t is = wave_prefix_sum(ns);
            const uint32_t ic = wave_prefix_sum(nc);
            int ps = wpos + int(is - ns);
            int pc = cpos + int(ic - nc);
#pragma unroll
            for (int j = 0; j < kLogGroup; ++j) {
                if (sel[j]) {
                    if (ps < k) {
                        su[stage_word(ps)] = u[j];
                        si[stage_word(ps)] = uint32_t(id[j]);
                    }
                    ++ps;
                }
                if (cand[j]) {
                    if (direct) {
                        if (pc < need) {
                            su[stage_word(int(above) + pc)] = u[j];
                            si[stage_word(int(above) + pc)] = uint32_t(id[j]);
                        }
                    } else if (pc < CAP) {
                        cu[pc] = u[j];
                        ci[pc] = id[j];
                    }
                    ++pc;
                }
            }
            wpos += int(__builtin_amdgcn_readlane(is, 63));
            cpos += int(__builtin_amdgcn_readlane(ic, 63));
        }
        wave_lds_sync();
        if (wpos == int(above) && cpos == int(nb)) {
            if (!direct)
                select_candidates(cu, ci, cpos, need, lo, shift, rhist, lane,
                                  [&](int p, uint32_t u, int32_t id) {
                                      su[stage_word(wpos + p)] = u;
                                      si[stage_word(wpos + p)] = uint32_t(id);
                                  });
            wave_lds_sync();
            return k;
        }
    }
    merge_log(lu, li, cnt, k, rhist, lane);
#pragma unroll 1
    for (int e = lane; e < k; e += 64) {
        su[stage_word(e)] = lu[e];
        si[stage_word(e)] = uint32_t(li[e]);
    }
    wave_lds_sync();
    return k;
}

// Staging slots [base, base + 64*E) to registers (blocked order) as ascending
// 64-bit keys ~orderkey << 32 | index; slots at or past n hold padding, which
// sorts after every finite score: ~orderkey(-inf) << 32 | 0xFFFFFFFF.
template <int E>
__device__ __forceinline__ void load_keys(const uint32_t *su, const uint32_t *si, int base, int n,
                                          unsigned long long (&key)[E], int lane)
{
    constexpr unsigned long long PAD = 0xFF800000FFFFFFFFull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int p = base + lane * E + e;
        const int w = stage_word(p);
        key[e] = p < n ? (static_cast<unsigned long long>(~su[w]) << 32) | si[w] : PAD;
    }
}

template <int E>
__device__ __forceinline__ void store_keys(uint32_t *su, uint32_t *si, int base,
                                           const unsigned long long (&key)[E], int lane)
{
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int w = stage_word(base + lane * E + e);
        si[w] = uint32_t(key[e]);
        su[w] = ~uint32_t(key[e] >> 32);
    }
}

// Writes sorted slots [base, base + 64*E) that lie below k to the output row
// through the staging words (whole cache lines per store); os may be null.
template <int E>
__device__ __forceinline__ void write_row(uint32_t *su, uint32_t *si, int base, int k,
                                          const unsigned long long (&key)[E], int32_t *oi,
                                          float *os, int lane)
{
    wave_lds_sync();
    store_keys<E>(su, si, base, key, lane);
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const int i = base + j * 64 + lane;
        if (i < k) {
            const int w = stage_word(i);
            oi[i] = int32_t(si[w]);
            if (os) os[i] = key_to_float(su[w]);
        }
    }
}

// Sorts staging slots [0, n) by (score desc, key index asc) and writes the
// first k to the output row, padding (-1, -inf) after the n entries.
// 64*E >= k slots; E <= 16 sorts in registers at once.  E = 32 sorts each
// half of 1,024 slots in registers, joins the halves with the first step
// of a bitonic merge on the staging words (slot i against slot 2047 - i,
// both halves ascending), and finishes each half in registers.
template <int E>
__device__ __forceinline__ void sort_store(uint32_t *su, uint32_t *si, int n, int k, int32_t *oi,
                                           float *os, int lane)
{
    if constexpr (E <= 16) {
        unsigned long long key[E];
        load_keys<E>(su, si, 0, n, key, lane);
        bitonic_sort<E, 2>(key, lane);
        write_row<E>(su, si, 0, k, key, oi, os, lane);
    } else {
        static_assert(E == 32, "one or two register passes");
        constexpr int HE = 16, HALF = 64 * HE;
        unsigned long long key[HE];
#pragma unroll 1
        for (int hf = 0; hf < 2; ++hf) {
            load_keys<HE>(su, si, hf * HALF, n, key, lane);
            bitonic_sort<HE, 2>(key, lane);
            wave_lds_sync();
            store_keys<HE>(su, si, hf * HALF, key, lane);
            wave_lds_sync();
        }
#pragma unroll
        for (int e = 0; e < HE; ++e) {
            const int i = lane * HE + e;
            const int wa = stage_word(i), wb = stage_word(2 * HALF - 1 - i);
            const unsigned long long x = (static_cast<unsigned long long>(~su[wa]) << 32) | si[wa];
            const unsigned long long y = (static_cast<unsigned long long>(~su[wb]) << 32) | si[wb];
            if (y < x) {
                su[wa] = ~uint32_t(y >> 32);
                si[wa] = uint32_t(y);
                su[wb] = ~uint32_t(x >> 32);
                si[wb] = uint32_t(x);
            }
        }
#pragma unroll 1
        for (int hf = 0; hf < 2 && hf * HALF < k; ++hf) {
            wave_lds_sync();
            load_keys<HE>(su, si, hf * HALF, 2 * HALF, key, lane);
            bitonic_step<HE, 2 * HALF, HALF / 2>(key, lane);
            write_row<HE>(su, si, hf * HALF, k, key, oi, os, lane);
        }
    }
}

// The final selection of one position's log and the sort of its row: rows
// of up to 64*e keys, e = 1, 8 or 32 (one call site in the kernel).
template <int NB>
__device__ __noinline__ void final_sorted(uint32_t *lu, int32_t *li, int cnt, int k, uint32_t *h,
                                          int hbase, uint32_t *su, uint32_t *si, uint32_t *rhist,
                                          int32_t *oi, float *os, int e, int lane)
{
    const int n = stage_select<NB>(lu, li, cnt, k, h, hbase, su, si, rhist, lane);
    if (e == 1)
        sort_store<1>(su, si, n, k, oi, os, lane);
    else if (e == 8)
        sort_store<8>(su, si, n, k, oi, os, lane);
    else
        sort_store<32>(su, si, n, k, oi, os, lane);
}

// ------------------------------------------------------------ score epilogue

// After the MFMAs of one 32-key half of a tile, acc[hb][i] is the dot
// product of q row R = hb*32 + 8*(i/4) + 4*half + i%4 (of the wave's 64
// (position, head) rows) with key lane%32 of that half, and wr[hb][i] is the
// head weight of row R.  partial() folds ReLU, the weights and the part of
// the head sum a lane can do alone; combine() joins the two halves of the
// tile so that sc[qi] holds, in lane l, the score of the wave's position qi
// against key l of the tile.
template <int H>
struct Epi {
    static constexpr int QW = 64 / H;
    // H >= 8: one partial per position; H <= 4: one per (hb, 8-row group,
    // position inside a 4-row quad) slot, each slot holding a lower-half and
    // an upper-half position.
    static constexpr int NP = H >= 8 ? QW : 32 / H;

    static __device__ __forceinline__ void partial(const f32x16_t (&acc)[2], const float (&wr)[2][16],
                                                   float (&p)[NP])
    {
#pragma unroll
        for (int x = 0; x < NP; ++x) p[x] = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int x = H >= 8 ? (hb * 32 + 8 * (i >> 2)) / H
                                     : (hb * 4 + (i >> 2)) * (4 / H) + (i & 3) / H;
                p[x] += wr[hb][i] * relu(acc[hb][i]);
            }
    }

    static __device__ __forceinline__ void combine(const float (&p0)[NP], const float (&p1)[NP],
                                                   float (&sc)[QW])
    {
        if constexpr (H >= 8) {
            // the other half-wave holds the remaining heads of the same keys
#pragma unroll
            for (int qi = 0; qi < QW; ++qi) sc[qi] = cross_half_sum(p0[qi], p1[qi]);
        } else {
            // lower lanes hold position qlo, upper lanes qhi, for the keys of
            // their half-tile; one swap gives each lane both positions at
            // key l of the tile
#pragma unroll
            for (int x = 0; x < NP; ++x) {
                const int hb = x / (4 * (4 / H));
                const int g = (x / (4 / H)) % 4;
                const int rho = x % (4 / H);
                const int qlo = (hb * 32 + 8 * g + H * rho) / H;
                const int qhi = (hb * 32 + 8 * g + 4 + H * rho) / H;
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0[x]),
                                                                __float_as_uint(p1[x]), false, false);
                sc[qlo] = __uint_as_float(r[0]);
                sc[qhi] = __uint_as_float(r[1]);
            }
        }
    }
};

// ------------------------------------------------------------ scoring kernel

// SPLIT: units are (query block, key range) pairs, a.n_splits ranges of
// a.split_keys keys (one range of all keys when n_splits = 1), and each unit
// leaves the top-k of its range unsorted in a list (a partial list, or the
// output row itself with one range) for the merge and sort passes.
// Otherwise units are query blocks and each row leaves the kernel sorted
// (next_pow2(k) <= kStageSlots).
// Kernel modes.  kPlain: q row i is position row_offset + i.  kPooled: q row
// i stands for position row_offset + i * pos_mul (the grouped entry point's
// pooled queries, one per group of pos_mul positions).  kList: the keys of
// a query block are not a prefix of k_cmp but a list of key indices in
// ascending order (a.klist), shared by a.list_rows consecutive query rows;
// a row still only accepts keys below its visible count (the grouped
// entry point's re-rank of shared candidates).
enum { kPlain = 0, kPooled = 1, kList = 2 };

template <int H, int D, bool FP8, bool SPLIT, int KT = kKeysPerTile, int MODE = kPlain>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
stream_topk_kernel(StreamArgs a)
{
    using O = Op<FP8>;
    using OpT = typename O::T;
    using E = Epi<H>;
    constexpr int QW = 64 / H;                       // positions per wave (64 rows)
    constexpr int QB = kWaves * QW;                  // positions per block
    // KT keys are staged per LDS tile (one workgroup barrier each); the
    // waves score and filter them CT = 64 at a time (one key per lane), in
    // two 32-key halves.  KT = 32 stages one half at a time.
    constexpr int CT = 64;
    static_assert(KT == 32 || KT % CT == 0, "key tile: 32 or a multiple of 64 keys");
    static_assert(!FP8 || KT >= CT, "fp8 key scales are staged 64 at a time");
    constexpr bool LIST = MODE == kList;
    static_assert(!LIST || (!FP8 && !SPLIT && KT >= CT), "key lists: bf16 sorted rows");
    // position of q row i
    auto position = [&](int64_t i) { return MODE == kPooled ? a.row_offset + i * a.pos_mul
                                                            : a.row_offset + i; };
    constexpr int NSUB = KT >= CT ? KT / CT : 1;     // compute tiles per staged tile
    constexpr bool HALF_TILES = KT < CT;             // a staged tile is one half
    constexpr int NDS = D / O::KSTEP;                // K steps per half tile
    constexpr int ROWB = D * O::ESZ;                 // LDS key row (swizzled, unpadded)
    constexpr int NC = ROWB / 16;                    // 16-byte chunks per key row
    constexpr int RPL = ROWB >= 256 ? 1 : 256 / ROWB;  // key rows per 256-byte LDS line
    auto swz = [](int r) { return (r / RPL) % NC; };
    constexpr int TILEB = KT * ROWB;
    constexpr int NDMA = TILEB / 1024;               // 1 KB wave DMA loads per tile
    constexpr int NDMA_W = (NDMA + kWaves - 1) / kWaves;
    // LDS ring of staged tiles: three (two ahead) while they fit beside the
    // staging area, else two
    constexpr int NBUF = 3 * TILEB <= kWaves * 2 * kStageSlots * 4 ? 3 : 2;
    constexpr int PD = NBUF - 1;                     // tiles loaded ahead
    constexpr int NB = 512 / QW;                     // threshold bins per position
    constexpr int HEAD = NB / 8 > 1 ? NB / 8 : 1;    // headroom above the max seen
    // appends between threshold refreshes: a refresh costs two LDS round
    // trips and a wave scan, a looser threshold only some extra appends
    constexpr int UPD = 512;

    // the key ring, and after a block's last tile each wave's staging area
    // for the final selection and sort (two arrays of kStageSlots words)
    constexpr int STAGEB = 2 * kStageSlots * 4;
    constexpr int UNIONB = NBUF * TILEB > kWaves * STAGEB ? NBUF * TILEB : kWaves * STAGEB;
    // One LDS block, laid out by hand: the small arrays the filter and the
    // selection hit on every tile first (lowest addresses), then the ring.
    constexpr int THB = kWaves * QW * NB * 4;       // threshold histograms
    constexpr int RHB = kWaves * 256 * 4;           // radix select scratch
    constexpr int KSB = (NBUF * KT * 4 + 15) / 16 * 16;  // fp8 key scales of the ring
    constexpr int UOFF = THB + RHB + KSB;
    __shared__ __attribute__((aligned(16))) unsigned char s_lds[UOFF + UNIONB];
    uint32_t (*const s_th)[QW * NB] = reinterpret_cast<uint32_t (*)[QW * NB]>(s_lds);
    uint32_t (*const s_rhist)[256] = reinterpret_cast<uint32_t (*)[256]>(s_lds + THB);
    float (*const s_ks)[KT] = reinterpret_cast<float (*)[KT]>(s_lds + THB + RHB);
    unsigned char *const s_union = s_lds + UOFF;
    unsigned char (*const s_k)[TILEB] = reinterpret_cast<unsigned char (*)[TILEB]>(s_union);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int half = lane >> 5;
    const int col = lane & 31;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int64_t slot = int64_t(g) * kWaves + wave;
    uint32_t *const log_u = a.ws + slot * (2 * int64_t(QW) * a.log_cap);
    int32_t *const log_i = reinterpret_cast<int32_t *>(log_u + int64_t(QW) * a.log_cap);
    uint32_t *const rhist = s_rhist[wave];

    // Heaviest blocks first (late positions see the most keys), snake order
    // over the persistent grid to even out the per-workgroup totals.  With
    // a multiple of 8 workgroups, workgroup g runs on XCD g % 8; the blocks
    // of one round are then dealt so that each XCD's workgroups hold
    // consecutive blocks, which stream the same key tiles through that
    // XCD's L2 at about the same time.
    const int xcd = g & 7, in_xcd = g >> 3, per_xcd = G >> 3;
    for (int64_t rnd = 0;; ++rnd) {
        const int64_t j = (G & 7) ? rnd * G + ((rnd & 1) ? (G - 1 - g) : g)
                                  : (rnd * 8 + ((rnd & 1) ? 7 - xcd : xcd)) * per_xcd + in_xcd;
        if (j >= a.n_units) break;
        // unit j: key range js of query block jq
        const int64_t jq = SPLIT ? j / a.n_splits : j;
        const int js = SPLIT ? int(j - jq * a.n_splits) : 0;
        const int64_t b = jq % a.B;
        const int64_t blk = a.blocks_per_batch - 1 - jq / a.B;
        const int64_t p0 = blk * QB;
        const int64_t p_last = (p0 + QB < a.S ? p0 + QB : a.S) - 1;
        // keys [klo, n_hi) of this unit: all visible keys, or one key range
        const int klo = SPLIT ? js * a.split_keys : 0;
        int n_hi = int(n_visible(position(p_last), a.T, a.m));
        if (SPLIT && klo + a.split_keys < n_hi) n_hi = klo + a.split_keys;
        // with key lists, the tiles cover list positions [0, length)
        const int32_t *const klist = LIST ? a.klist + (b * a.n_lists + p0 / a.list_rows) * a.list_cap
                                          : nullptr;
        if constexpr (LIST) n_hi = a.klen[b * a.n_lists + p0 / a.list_rows];
        const int64_t wp0 = p0 + int64_t(wave) * QW;

        // ---- the wave's 64 (position, head) rows of q and their weights
        OpT qa[2][NDS];
        float wr[2][16];
        const int64_t frow0 = (b * a.S + wp0) * H;
        const int64_t frow_end = (b * a.S + a.S) * H;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int64_t fr = frow0 + hb * 32 + col;
            const unsigned char *src = a.q + fr * (D * O::ESZ) + half * O::LANE_BYTES;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds)
                qa[hb][ds] = fr < frow_end ? O::load(src + ds * O::KSTEP * O::ESZ) : O::zero();
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t fw = frow0 + hb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                float wv = 0.f;
                if (fw < frow_end) {
                    wv = a.w[fw];
                    if constexpr (FP8) wv *= a.q_scale[fw];
                }
                wr[hb][i] = wv;
            }
        }
        int nv[QW];
        uint32_t tau[QW];   // a later key at or below tau is beaten by k earlier keys
        // fp8 takes the same test on the score, order key > tau <=> score >=
        // tauf, and orders only the scores of tiles where some lane passes
        // (measured faster with fp8's 256-key tiles; slower for bf16)
        constexpr bool SCORE_TEST = FP8;
        float tauf[QW];
        int cnt[QW];        // log entries
        int pend[QW];       // appends since the last threshold refresh
        int hbase[QW];      // global bin of threshold-histogram bin 0
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) {
            const int64_t pos = wp0 + qi;
            nv[qi] = pos < a.S ? int(n_visible(position(pos), a.T, a.m)) : 0;
            if (SPLIT && nv[qi] > n_hi) nv[qi] = n_hi;  // the end of the key range
            tau[qi] = 0u;  // below the key of any finite score: accept all
            if constexpr (SCORE_TEST) tauf[qi] = score_floor(0u);
            cnt[qi] = 0;
            pend[qi] = 0;
            hbase[qi] = 0;
            Hist<NB>::clear(&s_th[wave][qi * NB], lane);
        }
        wave_lds_sync();

        // Filter the wave's scores against key tile `it` and append the
        // survivors to the candidate logs (see the threshold histogram).
        auto consume = [&](const float (&sc)[QW], int it, int list_key) {
            const int kt = klo + it * CT;
            const int key = LIST ? list_key : kt + lane;
#pragma unroll
            for (int qi = 0; qi < QW; ++qi) {
                const int r = qi;
                if (!LIST && kt >= nv[qi]) continue;  // wave-uniform
                uint32_t u = SCORE_TEST ? 0u : order_key(sc[r]);
                const bool pass = key < nv[qi] && (SCORE_TEST ? sc[r] >= tauf[qi] : u > tau[qi]);
                const uint64_t mk = __ballot(pass);
                if (mk == 0) continue;
                if constexpr (SCORE_TEST) u = order_key(sc[r]);
                uint32_t *h = &s_th[wave][qi * NB];
                const int gb = int(u >> 16);
                if (cnt[qi] == 0) {
                    hbase[qi] = wave_max(pass ? gb : -1) + HEAD - (NB - 1);
                } else if (__ballot(pass && gb > hbase[qi] + NB - 1)) {
                    const int gmax = wave_max(pass ? gb : -1);
                    const int delta = gmax + HEAD - (hbase[qi] + NB - 1);
                    Hist<NB>::shift(h, delta, lane);
                    hbase[qi] += delta;
                }
                uint32_t *lu = log_u + qi * a.log_cap;
                int32_t *li = log_i + qi * a.log_cap;
                // LDS work first, the log stores last: an LDS write after a
                // global store waits for that store to complete
                if (pass) {
                    const int lb = gb - hbase[qi];
                    lds_add(&h[lb > 0 ? lb : 0], 1u);
                }
                const int p = cnt[qi] + lanes_below(mk);
                const int added = __popcll(mk);
                cnt[qi] += added;
                pend[qi] += added;
                const bool full = cnt[qi] > a.log_cap - CT;
                if (cnt[qi] >= a.topk && (pend[qi] >= UPD || full)) {
                    // raise tau to the lower edge of the highest bin that
                    // still has k candidates at or above it, minus one
                    wave_lds_sync();
                    const int bstar = Hist<NB>::top_bin(h, a.topk, lane);
                    const int gstar = hbase[qi] + bstar;
                    if (bstar > 0 && gstar > 0) {
                        const uint32_t t2 = (uint32_t(gstar) << 16) - 1u;
                        if (t2 > tau[qi]) {
                            tau[qi] = t2;
                            if constexpr (SCORE_TEST) tauf[qi] = score_floor(t2);
                        }
                        Hist<NB>::zero_below(h, bstar, lane);
                    }
                    pend[qi] = 0;
                }
                if (pass) {
                    lu[p] = u;
                    li[p] = key;
                }
                if (full) {
                    cnt[qi] = __builtin_amdgcn_readfirstlane(compact_log(lu, li, cnt[qi], tau[qi], lane));
                    const int room = a.topk + (a.log_cap - a.topk) / 2;
                    if (cnt[qi] > (room < a.log_cap - CT ? room : a.log_cap - CT)) {
                        // the bins could not separate enough: exact merge
                        tau[qi] = __builtin_amdgcn_readfirstlane(merge_log(lu, li, cnt[qi], a.topk, rhist, lane));
                        if constexpr (SCORE_TEST) tauf[qi] = score_floor(tau[qi]);
                        cnt[qi] = a.topk;
                        hist_recount<NB>(h, hbase[qi], lu, cnt[qi], lane);
                    }
                }
            }
        };

        // ---- key tiles: direct global -> LDS loads into a ring of NBUF
        // buffers, NBUF-1 tiles ahead.  Row r of a tile keeps its 16-byte
        // chunk c at chunk c ^ swz(r), swz(r) = (r / RPL) % NC with RPL rows
        // per 256-byte line of the 64 LDS banks: the 16 lanes of a read
        // cycle, one chunk of 16 consecutive rows, then fall on 16 distinct
        // 16-byte bank groups.  The swizzle is applied through each lane's
        // source address.
        const unsigned char *kbase = a.k + b * a.T * (D * O::ESZ);
        const float *ksbase = FP8 ? a.k_scale + b * a.T : nullptr;
        // DMA loads this wave issues per tile (the vmcnt it waits on); with
        // fp8 (key scales) or key lists (key indices), waves 0 .. NSUB-1 also
        // load 64 words each
        const int my_dma = (NDMA > wave ? (NDMA - wave + kWaves - 1) / kWaves : 0) +
                           (((FP8 || LIST) && wave < NSUB) ? 1 : 0);
        // key lists: the key index of each row this lane stages, fetched one
        // staged tile ahead of its DMA (list entries past the end hold
        // INT32_MAX and stage row T-1)
        int32_t lrow[NDMA_W];
        auto fetch_rows = [&](int st) {
#pragma unroll
            for (int v = 0; v < NDMA_W; ++v) {
                const int j = wave + v * kWaves;
                const int r = (j * 1024 + lane * 16) / ROWB;
                lrow[v] = (j < NDMA && st * KT < a.list_cap) ? klist[st * KT + r] : 0;
            }
        };
        auto dma_tile = [&](int st, int buf) {
            const int64_t row0 = int64_t(klo) + int64_t(st) * KT;
            const unsigned char *tb = kbase + (LIST ? 0 : row0 * ROWB);  // first key row of the tile
            // rows past T are never used: they repeat row T-1
            const int rmax = a.T - row0 - 1 < KT - 1 ? int(a.T - row0 - 1) : KT - 1;
#pragma unroll
            for (int v = 0; v < NDMA_W; ++v) {
                const int j = wave + v * kWaves;          // 1 KB block of the tile
                if (j < NDMA) {
                    const int off = j * 1024 + lane * 16;  // LDS byte of this lane
                    const int r = off / ROWB;
                    const int c = ((off % ROWB) / 16) ^ swz(r);
                    const unsigned char *src;
                    if constexpr (LIST) {
                        // a listed key row anywhere in k_cmp: 64-bit offset
                        const int64_t row = lrow[v] < a.T ? lrow[v] : a.T - 1;
                        src = tb + row * ROWB + c * 16;
                    } else {
                        // a row of this tile: 32-bit offset from the tile's first row
                        src = tb + (uint32_t(r < rmax ? r : rmax) * ROWB + uint32_t(c * 16));
                    }
                    if constexpr (FP8)
                        dma16(src, &s_k[buf][j * 1024]);
                    else
                        __builtin_amdgcn_global_load_lds(
                            src, (__attribute__((address_space(3))) void *)&s_k[buf][j * 1024],
                            16, 0, 0);
                }
            }
            if constexpr (LIST) {
                // the tile's key indices, for the filter
                if (wave < NSUB)
                    __builtin_amdgcn_global_load_lds(
                        klist + row0 + wave * CT + lane,
                        (__attribute__((address_space(3))) void *)&s_ks[buf][wave * CT], 4, 0, 0);
                // the next staged tile's rows
                fetch_rows(st + 1);
            }
            if constexpr (FP8) {
                if (wave < NSUB) {
                    int64_t key = row0 + wave * CT + lane;
                    key = key < a.T ? key : a.T - 1;
                    dma4(ksbase + key, &s_ks[buf][wave * CT]);
                }
            }
        };
        // Waits until at most `outstanding` of this wave's loads are in flight
        // (the most recent ones) and its LDS accesses are done, then joins
        // the workgroup barrier.
        auto sync_tiles = [&](int outstanding) {
            // s_waitcnt: vmcnt = outstanding (0..15), lgkmcnt = 0, expcnt = 7
            switch (outstanding) {
            case 0: __builtin_amdgcn_s_waitcnt(0x0070); break;
            case 1: __builtin_amdgcn_s_waitcnt(0x0071); break;
            case 2: __builtin_amdgcn_s_waitcnt(0x0072); break;
            case 3: __builtin_amdgcn_s_waitcnt(0x0073); break;
            case 4: __builtin_amdgcn_s_waitcnt(0x0074); break;
            case 5: __builtin_amdgcn_s_waitcnt(0x0075); break;
            case 6: __builtin_amdgcn_s_waitcnt(0x0076); break;
            case 7: __builtin_amdgcn_s_waitcnt(0x0077); break;
            case 8: __builtin_amdgcn_s_waitcnt(0x0078); break;
            default: __builtin_amdgcn_s_waitcnt(0x0079); break;
            }
            __builtin_amdgcn_s_barrier();
        };
        // loads this wave issued after those of staged tile t+1, once the
        // tiles up to min(t + PD, nst - 1) are staged
        auto later_loads = [&](int t, int nst) {
            const int last = t + PD < nst - 1 ? t + PD : nst - 1;
            return last > t + 1 ? my_dma * (last - t - 1) : 0;
        };
        // the 2*NDS MFMAs of the wave's rows against the 32 keys at row r0 of
        // staged tile buf
        f32x16_t acc[2];
        auto mma_half = [&](int buf, int r0) {
            const int r = r0 + col;
            const unsigned char *kb = &s_k[buf][r * ROWB];
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                const int c0 = (ds * O::KSTEP * O::ESZ + half * O::LANE_BYTES) / 16;
                const OpT bk = O::load_swz(kb, c0, swz(r));
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    acc[hb] = O::mma(qa[hb][ds], bk, ds == 0 ? f32x16_t{} : acc[hb]);
            }
            // operand reads two K steps ahead of their MFMAs
            constexpr int RD = FP8 ? 2 : 1;  // LDS reads per K step
            __builtin_amdgcn_sched_group_barrier(0x100, 3 * RD, 0);
#pragma unroll
            for (int st = 0; st < NDS - 3; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        };
        // fp8: the operands of a half's first two K steps are read earlier
        // (mma_pre), before the vector work that precedes the half, so that
        // its first MFMAs do not wait on LDS (bf16: no gain, more spills)
        constexpr bool PF = FP8;
        OpT bpf[2];
        auto mma_pre = [&](int buf, int r0) {
            if constexpr (PF) {
                const int r = r0 + col;
                const unsigned char *kb = &s_k[buf][r * ROWB];
#pragma unroll
                for (int ds = 0; ds < 2; ++ds)
                    bpf[ds] = O::load_swz(kb, (ds * O::KSTEP * O::ESZ + half * O::LANE_BYTES) / 16, swz(r));
            }
        };
        auto mma_half_pf = [&](int buf, int r0) {
            if constexpr (!PF) {
                mma_half(buf, r0);
            } else {
                const int r = r0 + col;
                const unsigned char *kb = &s_k[buf][r * ROWB];
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    const int c0 = (ds * O::KSTEP * O::ESZ + half * O::LANE_BYTES) / 16;
                    const OpT bk = ds < 2 ? bpf[ds] : O::load_swz(kb, c0, swz(r));
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
                        acc[hb] = O::mma(qa[hb][ds], bk, ds == 0 ? f32x16_t{} : acc[hb]);
                }
                constexpr int RD = 2;  // LDS reads per K step
                __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
                for (int st = 0; st < NDS - 3; ++st) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
            }
        };
        // scores of compute tile it from the two half partials; filter and append
        auto finish = [&](const float (&ha)[E::NP], const float (&hb)[E::NP], int it, float ksv) {
            float sc[QW];
            E::combine(ha, hb, sc);
            if constexpr (FP8)
#pragma unroll
                for (int qi = 0; qi < QW; ++qi) sc[qi] *= ksv;
            // with key lists, ksv carries the lane's key index
            consume(sc, it, LIST ? __float_as_int(ksv) : 0);
        };

        // Waves 0-3 run, per compute tile i: MFMA(half 0), its epilogue,
        // MFMA(half 1), its epilogue, the filter.  Waves 4-7 (the second wave
        // of each SIMD) run the same steps half a tile later: they open tile i
        // with the epilogue and filter of tile i-1 and close it with MFMA(half
        // 1), whose accumulators they carry over the barrier.  The two waves
        // of a SIMD thus alternate between matrix-core and VALU work.
        const bool lagging = wave >= kWaves / 2;
        const int ntiles = n_hi > klo ? (n_hi - klo + CT - 1) / CT : 0;  // compute tiles
        const int nst = n_hi > klo ? (n_hi - klo + KT - 1) / KT : 0;     // staged tiles
        // every wave is past its last read of the ring (previous block)
        __syncthreads();
        if constexpr (LIST) fetch_rows(0);
        for (int t = 0; t < PD && t < nst; ++t) dma_tile(t, t);
        sync_tiles(later_loads(-1, nst));
        float ksv_prev = 1.f;
        float h0[E::NP], h1[E::NP];
#pragma unroll 1
        for (int it = 0; it < ntiles; ++it) {
            // staged tile and row of half 0 (half 1: the next 32 rows, or with
            // half-tile staging row 0 of the next staged tile)
            const int st = HALF_TILES ? 2 * it : it / NSUB;
            const int buf = st % NBUF;
            const int r0 = HALF_TILES ? 0 : (it % NSUB) * CT;
            float ksv = 1.f;
            if constexpr (FP8 || LIST) ksv = s_ks[buf][r0 + lane];
            // Each wave stages its share of tile st+PD (over tile st-1, which
            // every wave has finished) after its own filter step, so that the
            // leading and the lagging waves issue their loads half a tile
            // apart.
            const bool stage = (HALF_TILES || it % NSUB == 0) && st + PD < nst;
            const bool last = HALF_TILES || it % NSUB == NSUB - 1 || it == ntiles - 1;
            // The epilogue of one half tile is issued before the next half's
            // MFMAs (a scheduling barrier), so both halves share one set of
            // accumulator registers: the other wave of the SIMD keeps the
            // matrix core busy meanwhile.
            if constexpr (HALF_TILES) {
                const int buf1 = (st + 1) % NBUF;
                const bool stage1 = st + 1 + PD < nst;
                if (!lagging) {
                    mma_half(buf, 0);
                    E::partial(acc, wr, h0);
                    if (stage) dma_tile(st + PD, (st + PD) % NBUF);
                    sync_tiles(later_loads(st, nst));
                    mma_half(buf1, 0);
                    E::partial(acc, wr, h1);
                    finish(h0, h1, it, ksv);
                    if (stage1) dma_tile(st + 1 + PD, (st + 1 + PD) % NBUF);
                } else {
                    if (it > 0) {
                        E::partial(acc, wr, h1);
                        __builtin_amdgcn_sched_barrier(0);
                        finish(h0, h1, it - 1, ksv_prev);
                    }
                    if (stage) dma_tile(st + PD, (st + PD) % NBUF);
                    mma_half(buf, 0);
                    E::partial(acc, wr, h0);
                    sync_tiles(later_loads(st, nst));
                    if (stage1) dma_tile(st + 1 + PD, (st + 1 + PD) % NBUF);
                    mma_half(buf1, 0);
                }
                ksv_prev = ksv;
                sync_tiles(later_loads(st + 1, nst));
            } else {
                if (!lagging) {
                    mma_half(buf, r0);
                    mma_pre(buf, r0 + 32);
                    E::partial(acc, wr, h0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_half_pf(buf, r0 + 32);
                    E::partial(acc, wr, h1);
                    finish(h0, h1, it, ksv);
                    if (stage) dma_tile(st + PD, (st + PD) % NBUF);
                } else {
                    mma_pre(buf, r0);
                    if (it > 0) {
                        E::partial(acc, wr, h1);
                        __builtin_amdgcn_sched_barrier(0);
                        finish(h0, h1, it - 1, ksv_prev);
                    }
                    if (stage) dma_tile(st + PD, (st + PD) % NBUF);
                    mma_half_pf(buf, r0);
                    mma_pre(buf, r0 + 32);
                    E::partial(acc, wr, h0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_half_pf(buf, r0 + 32);
                }
                ksv_prev = ksv;
                if (last) sync_tiles(later_loads(st, nst));
            }
        }
        if (lagging && ntiles > 0) {
            E::partial(acc, wr, h1);
            finish(h0, h1, ntiles - 1, ksv_prev);
        }

        // ---- final selection.  The key ring is idle until the next block's
        // first barrier: it serves as each wave's staging area (sorted rows)
        // or candidate buffer (unsorted rows, sorted by a later pass).
        if constexpr (!SPLIT) {
            uint32_t *const su = reinterpret_cast<uint32_t *>(s_union + wave * STAGEB);
            uint32_t *const si = su + kStageSlots;
#pragma unroll 1
            for (int qi = 0; qi < QW; ++qi) {
                const int64_t pos = wp0 + qi;
                if (pos >= a.S) break;
                const int64_t row = (b * a.S + pos) * a.topk;
                int32_t *const oi = a.out_idx + row;
                float *const os = a.out_score ? a.out_score + row : nullptr;
                final_sorted<NB>(log_u + qi * a.log_cap, log_i + qi * a.log_cap, cnt[qi], a.topk,
                                 &s_th[wave][qi * NB], hbase[qi], su, si, rhist, oi, os, a.sort_e,
                                 lane);
            }
            continue;
        }
        constexpr int CAP = NBUF * TILEB / kWaves / 8;
        uint32_t *const cu = reinterpret_cast<uint32_t *>(s_union + wave * (NBUF * TILEB / kWaves));
        int32_t *const ci = reinterpret_cast<int32_t *>(cu + CAP);
#pragma unroll 1
        for (int qi = 0; qi < QW; ++qi) {
            const int64_t pos = wp0 + qi;
            if (pos >= a.S) break;
            // one key range: its top-k goes to the partial list (js) of the row
            const int64_t row = SPLIT ? ((b * a.S + pos) * a.n_splits + js) * a.topk
                                      : (b * a.S + pos) * a.topk;
            int32_t *oi = SPLIT ? a.part_idx : a.out_idx;
            float *os = SPLIT ? a.part_score : a.out_score;
            final_select<NB>(log_u + qi * a.log_cap, log_i + qi * a.log_cap, cnt[qi], a.topk,
                             &s_th[wave][qi * NB], hbase[qi], cu, ci, CAP, rhist,
                             oi + row, os + row, lane);
        }
    }
}

template <int H, int D, bool FP8>
static hipError_t launch_one(const StreamArgs &a, int grid, hipStream_t s)
{
    if (a.sort_e == 0) {
        if constexpr (H == 64 && D == 128 && !FP8) {
            if (a.key_tile == 128) {
                hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, true, 128>), dim3(grid),
                                   dim3(kThreads), 0, s, a);
                return hipGetLastError();
            }
        }
        if (a.key_tile != kKeysPerTile) return hipErrorInvalidValue;
        hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, true>), dim3(grid), dim3(kThreads), 0,
                           s, a);
        return hipGetLastError();
    }
    if constexpr (H == 64 && D == 128 && FP8) {
        if (a.key_tile == 128) {
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 128>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
        if (a.key_tile == 256) {
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 256>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
    }
    if constexpr (H == 64 && D == 128 && !FP8) {
        // the other staged key tiles (a speed knob) of this one shape
        switch (a.key_tile) {
        case 32:
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 32>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        case 128:
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 128>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        case 192:
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 192>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        case 256:
            hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false, 256>), dim3(grid),
                               dim3(kThreads), 0, s, a);
            return hipGetLastError();
        default: break;
        }
    }
    if (a.key_tile != kKeysPerTile) return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8, false>), dim3(grid), dim3(kThreads), 0, s,
                       a);
    return hipGetLastError();
}

// Launches stream_topk_kernel<H, D, FP8, *> for a runtime H.
template <int D, bool FP8>
static hipError_t launch_h(int H, const StreamArgs &a, int grid, hipStream_t s)
{
    switch (H) {
    case 1: return launch_one<1, D, FP8>(a, grid, s);
    case 2: return launch_one<2, D, FP8>(a, grid, s);
    case 4: return launch_one<4, D, FP8>(a, grid, s);
    case 8: return launch_one<8, D, FP8>(a, grid, s);
    case 16: return launch_one<16, D, FP8>(a, grid, s);
    case 32: return launch_one<32, D, FP8>(a, grid, s);
    case 64: return launch_one<64, D, FP8>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
