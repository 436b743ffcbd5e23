// csa_kernels.hip -- gfx950 kernels of the CSA lightning-indexer top-k.
//
// StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
// Top-k (Abstract) computes, per query position, lightning-indexer scores
// over the compressed keys and keeps the top-k, with a chunked
// partition-merge driver that never materialises the [B,S,H_I,T] tensor.
// Here that is one persistent scoring kernel plus a row sort:
//
//   stream_topk_kernel  Each wave owns 64 (position, head) rows of q, held in
//       VGPRs as MFMA A-operands.  The workgroup stages 64-key tiles of k_cmp
//       in LDS (double buffered).  Per tile a wave runs the [64 rows x D] x
//       [D x 64 keys] contraction on the matrix cores (bf16 32x32x16 or fp8
//       32x32x64), then in registers applies ReLU, the per-head weights and
//       the head sum, and the causal cut.  A score survives only if it beats
//       the position's running threshold (the k-th best so far); survivors
//       are appended, in key order, to the position's candidate log.  When
//       the log holds k + chunk entries a wave-level radix select finds the
//       k-th best (score desc, index asc), compacts the log to exactly the
//       running top-k in key order (the merge step), and raises the
//       threshold.  At the end the log is the exact top-min(k, n_vis) set.
//   sort_rows_kernel  Orders every output row by (score desc, index asc)
//       with a bitonic sort in LDS and leaves padding (-1, -inf) last.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_kernels.hpp"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

// Monotone map float -> uint32 (larger float -> larger key), -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
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
// shared-memory accesses across the point and waits for them to finish.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// Makes global stores of every lane of the wave visible to global loads of
// the other lanes (write completion + L1 invalidation).
__device__ __forceinline__ void wave_global_sync()
{
    __threadfence();
    __builtin_amdgcn_wave_barrier();
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
    static __device__ __forceinline__ f32x16_t mma(T a, T b, f32x16_t c)
    {
        // formats 0/0 = E4M3 for A and B; scale exponent 127 = 2^0
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

// ------------------------------------------------------- candidate merging

// The log lu/li[0..n) holds candidates of one position in ascending key
// order, n > k.  Finds the k-th best under (score desc, key asc) with a
// 4 x 8-bit radix select on the order keys, compacts the log in place to
// exactly the k best (still in key order) and returns the k-th best key.
__device__ __noinline__ uint32_t merge_log(uint32_t *lu, int32_t *li, int n, int k,
                                           uint32_t *hist, int lane)
{
    wave_global_sync();
    uint32_t prefix = 0u, pmask = 0u;
    int kk = k;  // rank, from the top, of the wanted key among prefix matches
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = lane; i < 256; i += 64) hist[i] = 0u;
        wave_lds_sync();
        for (int e = lane; e < n; e += 64) {
            const uint32_t u = lu[e];
            if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        wave_lds_sync();
        const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
        const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
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
        d = __shfl(d, L);
        ab = __shfl(ab, L);
        kk -= int(ab);
        prefix |= uint32_t(d) << shift;
        pmask |= 0xFFu << shift;
        wave_lds_sync();
    }
    // prefix is the k-th best key; keep every larger key and the first kk
    // equal ones (the lowest key indices, since the log is in key order).
    int wpos = 0, eq_seen = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += 64) {
        const int e = base + lane;
        const bool valid = e < n;
        const uint32_t u = valid ? lu[e] : 0u;
        const int32_t id = valid ? li[e] : 0;
        const bool gt = valid && u > prefix;
        const bool eq = valid && u == prefix;
        const uint64_t meq = __ballot(eq);
        const bool keep = gt || (eq && eq_seen + lanes_below(meq) < kk);
        const uint64_t mk = __ballot(keep);
        if (keep) {
            const int p = wpos + lanes_below(mk);
            lu[p] = u;
            li[p] = id;
        }
        wpos += __popcll(mk);
        eq_seen += __popcll(meq);
    }
    wave_global_sync();
    return prefix;
}

// ------------------------------------------------------------ score epilogue

// acc[hb][ks][i] is the dot product of q row R = hb*32 + 8*(i/4) +
// 4*half + i%4 (of the wave's 64 (position, head) rows) with key
// ks*32 + lane%32 of the tile.  wr[hb][i] is the head weight of row R.
// On return sc[qi] holds, in lane l, the score of the wave's position qi
// against key l of the tile: sum over the position's heads of w*ReLU(dot).
template <int H>
__device__ __forceinline__ void head_reduce(const f32x16_t (&acc)[2][2], const float (&wr)[2][16],
                                            float (&sc)[64 / H], int half)
{
    constexpr int QW = 64 / H;
    if constexpr (H >= 8) {
        // a lane's rows of one 8-row group belong to one position; the other
        // half-wave holds the remaining heads of the same key column.
        float s[QW][2];
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) s[qi][0] = s[qi][1] = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qi = (hb * 32 + 8 * (i >> 2)) / H;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    s[qi][ks] += wr[hb][i] * fmaxf(acc[hb][ks][i], 0.f);
            }
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) {
            const float give = half ? s[qi][0] : s[qi][1];
            const float got = __shfl_xor(give, 32);
            sc[qi] = (half ? s[qi][1] : s[qi][0]) + got;
        }
    } else {
        // H <= 4: each half-wave holds whole positions; pair a lower-half
        // position with an upper-half one and swap the key halves.
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int rho = 0; rho < 4 / H; ++rho) {
                    float val[2] = {0.f, 0.f};
#pragma unroll
                    for (int r = H * rho; r < H * rho + H; ++r)
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
                            val[ks] += wr[hb][4 * g + r] * fmaxf(acc[hb][ks][4 * g + r], 0.f);
                    const float give = half ? val[0] : val[1];
                    const float got = __shfl_xor(give, 32);
                    const int qlo = (hb * 32 + 8 * g + H * rho) / H;
                    const int qhi = (hb * 32 + 8 * g + 4 + H * rho) / H;
                    sc[qlo] = half ? got : val[0];
                    sc[qhi] = half ? val[1] : got;
                }
    }
}

// ------------------------------------------------------------ scoring kernel

template <int H, int D, bool FP8>
__global__ void __launch_bounds__(kThreads)
stream_topk_kernel(StreamArgs a)
{
    using O = Op<FP8>;
    using OpT = typename O::T;
    constexpr int QW = kRowsPerWave / H;             // positions per wave
    constexpr int QB = kWaves * QW;                  // positions per block
    constexpr int KT = kKeysPerTile;
    constexpr int NDS = D / O::KSTEP;                // K steps per tile
    constexpr int ROWB = D * O::ESZ + 16;            // padded LDS key row
    constexpr int TILEB = KT * ROWB;
    constexpr int RV = D * O::ESZ / 16;              // 16-byte vectors per key row
    constexpr int NV = KT * RV;                      // vectors per tile
    constexpr int VPT = (NV + kThreads - 1) / kThreads;

    __shared__ __attribute__((aligned(16))) unsigned char s_k[2][TILEB];
    __shared__ float s_ks[2][KT];
    __shared__ uint32_t s_hist[kWaves][256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int64_t slot = int64_t(g) * kWaves + wave;
    uint32_t *const log_u = a.ws + slot * (2 * int64_t(QW) * a.log_cap);
    int32_t *const log_i = reinterpret_cast<int32_t *>(log_u + int64_t(QW) * a.log_cap);
    uint32_t *const hist = s_hist[wave];

    // heaviest blocks first (late positions see the most keys); snake order
    // over the persistent grid evens out the per-workgroup totals.
    for (int64_t rnd = 0;; ++rnd) {
        const int64_t j = rnd * G + ((rnd & 1) ? (G - 1 - g) : g);
        if (j >= a.n_blocks) break;
        const int64_t b = j % a.B;
        const int64_t blk = a.blocks_per_batch - 1 - j / a.B;
        const int64_t p0 = blk * QB;
        const int64_t p_last = (p0 + QB < a.S ? p0 + QB : a.S) - 1;
        const int n_hi = int(n_visible(a.row_offset + p_last, a.T, a.m));
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
        uint32_t tau[QW];
        int cnt[QW];
        int nv_max = 0;
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) {
            const int64_t pos = wp0 + qi;
            nv[qi] = pos < a.S ? int(n_visible(a.row_offset + pos, a.T, a.m)) : 0;
            tau[qi] = 0u;  // below the key of any finite score: accept all
            cnt[qi] = 0;
            nv_max = nv[qi] > nv_max ? nv[qi] : nv_max;
        }

        // ---- key tiles: global -> registers -> LDS, double buffered
        const unsigned char *kbase = a.k + b * a.T * (D * O::ESZ);
        const float *ksbase = FP8 ? a.k_scale + b * a.T : nullptr;
        u32x4_t pre[VPT];
        float pks = 0.f;
        auto load_tile = [&](int it) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int vi = tid + v * kThreads;
                pre[v] = u32x4_t{0, 0, 0, 0};
                if (vi < NV) {
                    const int64_t key = int64_t(it) * KT + vi / RV;
                    if (key < a.T)
                        pre[v] = *reinterpret_cast<const u32x4_t *>(
                            kbase + key * (D * O::ESZ) + (vi % RV) * 16);
                }
            }
            if constexpr (FP8) {
                const int64_t key = int64_t(it) * KT + tid;
                pks = (tid < KT && key < a.T) ? ksbase[key] : 0.f;
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int vi = tid + v * kThreads;
                if (vi < NV)
                    *reinterpret_cast<u32x4_t *>(&s_k[buf][(vi / RV) * ROWB + (vi % RV) * 16]) = pre[v];
            }
            if constexpr (FP8)
                if (tid < KT) s_ks[buf][tid] = pks;
        };

        const int ntiles = (n_hi + KT - 1) / KT;
        if (ntiles > 0) {
            load_tile(0);
            store_tile(0);
        }
        __syncthreads();
#pragma unroll 1
        for (int it = 0; it < ntiles; ++it) {
            const int buf = it & 1;
            const bool more = it + 1 < ntiles;
            if (more) load_tile(it + 1);
            const int kt = it * KT;
            if (kt < nv_max) {
                f32x16_t acc[2][2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[hb][ks][e] = 0.f;
                const unsigned char *kb = &s_k[buf][col * ROWB + half * O::LANE_BYTES];
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    const OpT b0 = O::load(kb + ds * O::KSTEP * O::ESZ);
                    const OpT b1 = O::load(kb + 32 * ROWB + ds * O::KSTEP * O::ESZ);
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb) {
                        acc[hb][0] = O::mma(qa[hb][ds], b0, acc[hb][0]);
                        acc[hb][1] = O::mma(qa[hb][ds], b1, acc[hb][1]);
                    }
                }
                float sc[QW];
                head_reduce<H>(acc, wr, sc, half);
                if constexpr (FP8) {
                    const float ksv = s_ks[buf][lane];
#pragma unroll
                    for (int qi = 0; qi < QW; ++qi) sc[qi] *= ksv;
                }
                const int key = kt + lane;
#pragma unroll
                for (int qi = 0; qi < QW; ++qi) {
                    if (kt >= nv[qi]) continue;  // wave-uniform
                    const uint32_t u = order_key(sc[qi]);
                    const bool pass = key < nv[qi] && u > tau[qi];
                    const uint64_t mk = __ballot(pass);
                    if (mk == 0) continue;
                    uint32_t *lu = log_u + qi * a.log_cap;
                    int32_t *li = log_i + qi * a.log_cap;
                    if (pass) {
                        const int p = cnt[qi] + lanes_below(mk);
                        lu[p] = u;
                        li[p] = key;
                    }
                    cnt[qi] += __popcll(mk);
                    if (cnt[qi] > a.log_cap - KT) {
                        tau[qi] = merge_log(lu, li, cnt[qi], a.topk, hist, lane);
                        cnt[qi] = a.topk;
                    }
                }
            }
            if (more) store_tile(buf ^ 1);
            __syncthreads();
        }

        // ---- final merge and (unsorted, key-ordered) output rows
#pragma unroll 1
        for (int qi = 0; qi < QW; ++qi) {
            const int64_t pos = wp0 + qi;
            if (pos >= a.S) break;
            uint32_t *lu = log_u + qi * a.log_cap;
            int32_t *li = log_i + qi * a.log_cap;
            int c = cnt[qi];
            if (c > a.topk) {
                merge_log(lu, li, c, a.topk, hist, lane);
                c = a.topk;
            } else {
                wave_global_sync();
            }
            const int64_t row = (b * a.S + pos) * a.topk;
            for (int e = lane; e < a.topk; e += 64) {
                if (e < c) {
                    a.out_idx[row + e] = li[e];
                    a.out_score[row + e] = key_to_float(lu[e]);
                } else {
                    a.out_idx[row + e] = -1;
                    a.out_score[row + e] = -__builtin_inff();
                }
            }
        }
    }
}

// ------------------------------------------------------------------ row sort

// Sorts each row of k (index, score) pairs by (score desc, index asc);
// padding (-1, -inf) sorts last.  pow2 = next power of two >= k entries of
// 64-bit keys live in dynamic LDS.
__global__ void __launch_bounds__(256)
sort_rows_kernel(int32_t *out_idx, float *out_score, int64_t nrows, int k, int pow2)
{
    extern __shared__ unsigned long long s_key[];
    const int tid = threadIdx.x;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        int32_t *ri = out_idx + row * k;
        float *rs = out_score + row * k;
        for (int e = tid; e < pow2; e += 256) {
            unsigned long long key = ~0ull;
            if (e < k) {
                const uint32_t u = order_key(rs[e]);
                key = (static_cast<unsigned long long>(~u) << 32) | uint32_t(ri[e]);
            }
            s_key[e] = key;
        }
        __syncthreads();
        for (int size = 2; size <= pow2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < pow2 / 2; i += 256) {
                    const int lo = 2 * stride * (i / stride) + (i % stride);
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
        for (int e = tid; e < k; e += 256) {
            const unsigned long long key = s_key[e];
            ri[e] = int32_t(uint32_t(key));
            rs[e] = key_to_float(~uint32_t(key >> 32));
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ dispatch

template <int H, int D, bool FP8>
static hipError_t launch_one(const StreamArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((stream_topk_kernel<H, D, FP8>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

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

hipError_t launch_stream_topk(const Plan &p, const StreamArgs &a, hipStream_t s)
{
    if (p.grid <= 0) return hipSuccess;
    if (!p.fp8) {
        switch (p.D) {
        case 32: return launch_h<32, false>(p.H, a, p.grid, s);
        case 64: return launch_h<64, false>(p.H, a, p.grid, s);
        case 128: return launch_h<128, false>(p.H, a, p.grid, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.D) {
    case 64: return launch_h<64, true>(p.H, a, p.grid, s);
    case 128: return launch_h<128, true>(p.H, a, p.grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sort_rows(const Plan &p, int32_t *out_idx, float *out_score, int num_cus,
                            hipStream_t s)
{
    const int64_t nrows = p.B * p.S;
    if (nrows == 0) return hipSuccess;
    const int64_t want = int64_t(num_cus) * 8;
    const int grid = int(nrows < want ? nrows : want);
    const size_t lds = size_t(p.sort_pow2) * sizeof(unsigned long long);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(sort_rows_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sort_rows_kernel, dim3(grid), dim3(256), lds, s, out_idx, out_score,
                       nrows, p.k, p.sort_pow2);
    return hipGetLastError();
}

}  // namespace csa
