// csa_attn.hip -- sparse attention over the compressed keys the indexer
// selected, for gfx950.
//
// StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
// Top-k (Abstract): after the lightning indexer has chosen each query's
// keys, the attention reads only those keys.  For query row r and head h:
// softmax over the valid entries e of the row's index list of
// scale * q[r,h,:] . k[idx[e],:], applied to v[idx[e],:]; every head shares
// the compressed key and value rows.
//
// One workgroup per query row, one wave per 32 heads.  The row's index list
// is taken 32 entries at a time (a tile); each lane loads one entry per
// tile, one tile early.  Every tile's 32 key rows and 32 value rows stream
// from global memory straight into LDS (global_load_lds, 16 bytes per lane)
// into a ring of two buffers, one tile ahead; at 32 KB of LDS the register
// budget (two waves per SIMD) is what bounds residency, four workgroups per
// CU (more resident workgroups beat deeper rings here).  Each row's 16-byte
// chunks are XOR-swizzled by row, so the operand reads below hit distinct
// LDS banks.  For every tile each wave
//   * computes the 32x32 block S^T = K_tile . Q^T of (key, head) scores with
//     v_mfma_f32_32x32x16_bf16: A = key rows from LDS, B = the wave's 32
//     query heads, held in registers for the whole row;
//   * runs the online softmax: in the MFMA output layout each lane holds one
//     head (lane % 32) and 16 of the tile's keys, so the running maximum and
//     the sum stay in the lane, and the two lanes of a head agree through one
//     v_permlane32_swap;
//   * accumulates O^T += V_tile^T . P^T with B = the bf16 weights straight
//     from the lane's score registers and A read from the row-major value
//     rows with gfx950's LDS transpose load (ds_read_b64_tr_b16), which
//     hands each lane one value column at the keys its weights belong to.
// Rows are mapped to workgroups so that consecutive rows share an XCD (and
// its L2), where queries close in position may pick the same keys.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_dma.hpp"
#include "csa_kernels.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef short s8_t __attribute__((ext_vector_type(8)));

constexpr int KT = 32;                 // selected entries per tile
constexpr int kXcds = 8;               // XCDs of an MI355X; workgroups go round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_op(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ bf16x8_t lds_op(const unsigned char *p)
{
    return as_op(*reinterpret_cast<const u32x4_t *>(p));
}

// The other lane of the pair (l, l ^ 32) for every lane: v_permlane32_swap
// returns {x[l], x[l ^ 32]} (in lane-half order), so min/max/sum over the
// pair come out bit-identical in both lanes.
__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt immediate: at most n vector-memory loads of this wave in flight,
// no LDS / scalar access outstanding (lgkmcnt 0), export count untouched.
constexpr int vm_wait_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }

// One unit is a query row (SPLIT = false) or one of the n_splits ranges of
// split_entries entries of a row's list (SPLIT = true: short query blocks,
// where rows alone cannot fill the device).  A range writes its unnormalised
// output, running maximum and weight sum to the partial buffers; the
// combine kernel merges the ranges of a row.
template <int H, int D, bool SPLIT>
__global__ void __launch_bounds__(64 * (H / 32))
sparse_attn_kernel(AttnArgs a, int64_t unit0, int64_t nunits)
{
    constexpr int W = H / 32;              // waves; wave w owns heads 32w .. 32w+31
    constexpr int ROWB = 2 * D;            // bytes of one key or value row
    constexpr int NC = ROWB / 16;          // 16-byte chunks per row
    constexpr int HALF = KT * ROWB;        // bytes of the tile's key (or value) rows
    constexpr int NBLK = 2 * HALF / 1024;  // 1 KB DMA blocks per tile
    constexpr int BPW = NBLK / W;          // DMA blocks (loads) per wave per tile
    constexpr int KS = D / 16;             // K steps of the score product
    constexpr int MB = D / 32;             // 32-row blocks of the output
    static_assert(NBLK % W == 0 && BPW <= 32, "DMA layout");

    // two tile buffers: the one being computed and the one being loaded
    __shared__ __attribute__((aligned(1024))) unsigned char s_ring[2][2 * HALF];

    // consecutive units on one XCD: workgroup i runs on XCD i % 8
    const int64_t per_xcd = (nunits + kXcds - 1) / kXcds;
    const int64_t slot = int64_t(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (slot >= nunits) return;  // whole workgroup, before any barrier
    const int64_t unit = unit0 + slot;
    const int64_t row = SPLIT ? unit / a.n_splits : unit;
    const int64_t b = row / a.S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5;              // lane half: K slice of MFMA operands
    const int col = lane & 31;
    const int head = 32 * wave + col;

    // B operand of the score product: q[row, head, 16s + 8hh .. +8]
    bf16x8_t qop[KS];
    {
        const unsigned char *qr = a.q + (row * H + head) * int64_t(ROWB) + 16 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = as_op(*reinterpret_cast<const u32x4_t *>(qr + 32 * s));
    }
    const unsigned char *kbase = a.k + b * a.T * int64_t(ROWB);
    const unsigned char *vbase = a.v + b * a.T * int64_t(ROWB);
    const int32_t *list = a.idx + row * int64_t(a.n_sel);
    const int64_t T = a.T;
    // this unit's entries [e0, e1) of the row's list
    const int e0 = SPLIT ? int(unit % a.n_splits) * a.split_entries : 0;
    const int e1 = SPLIT ? (a.n_sel - e0 < a.split_entries ? a.n_sel : e0 + a.split_entries)
                         : a.n_sel;
    const int ntiles = (T > 0 && e1 > e0) ? (e1 - e0 + KT - 1) / KT : 0;

    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
    float m_run = -INFINITY;  // running maximum of the head's scores, log2 units
    float l_run = 0.f;        // this lane's part of the running sum of weights
    const float c = a.scale * kLog2e;

    // Entry `col` of tile t (a key index in [0, T), or -1): every lane
    // loads one, so lanes r and r + 32 hold entry r of the tile.
    auto load_entry = [&](int t) -> int {
        const int pos = e0 + t * KT + col;
        if (t >= ntiles || pos >= e1) return -1;
        const int s = list[pos];
        return (s >= 0 && s < T) ? s : -1;
    };
    // One tile into buffer `buf`, given the lane's entry `ent` of it: this
    // wave's blocks j = wave + v*W; block j < NBLK/2 holds key rows, the
    // rest value rows; the lane's 16 bytes land at chunk p of row r and carry
    // the row's logical chunk p ^ swizzle(r): r % NC for key rows (32 rows
    // read at one chunk), 2r % NC for value rows (4 rows read at two adjacent
    // chunks).  Padding entries load row 0 (never used).
    auto dma_tile = [&](int ent, int buf) {
#pragma unroll
        for (int v = 0; v < BPW; ++v) {
            const int j = wave + v * W;
            const bool is_v = j >= NBLK / 2;
            const int off = (is_v ? j - NBLK / 2 : j) * 1024 + lane * 16;
            const int r = off / ROWB;
            const int p = (off % ROWB) / 16;
            const int s = __shfl(ent, r);
            const int swz = is_v ? (2 * r) % NC : r % NC;
            const unsigned char *src = (is_v ? vbase : kbase) +
                                       int64_t(s >= 0 ? s : 0) * ROWB + 16 * (p ^ swz);
            dma16(src, &s_ring[buf][j * 1024]);
        }
    };

    {
        int e_cur = load_entry(0);   // the lane's entry of the tile being computed
        int e_next = load_entry(1);  // ... of the next tile
        if (ntiles > 0) {
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            dma_tile(e_cur, 0);
        }
        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            // this wave's loads are done (tile t and the entries of tile
            // t + 1), then every wave's
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
            // every wave is past tile t-1: its buffer takes tile t+1
            if (t + 1 < ntiles) dma_tile(e_next, buf ^ 1);
            const int ent = e_cur;
            e_cur = e_next;
            e_next = load_entry(t + 2);  // lands before the next wait

            const uint32_t vmask = uint32_t(__builtin_amdgcn_ballot_w64(ent >= 0));  // bit = tile key
            if (vmask == 0) continue;
            const unsigned char *kt = &s_ring[buf][0];
            __attribute__((address_space(3))) unsigned char *vt_lds =
                (__attribute__((address_space(3))) unsigned char *)&s_ring[buf][HALF];
            const int swz = col % NC;
            // S^T[key][head] for the tile's 32 keys and the wave's 32 heads
            f32x16_t s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
#pragma unroll
            for (int s = 0; s < KS; s += 2) {
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    lds_op(kt + col * ROWB + 16 * ((2 * s + hh) ^ swz)), qop[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    lds_op(kt + col * ROWB + 16 * ((2 * s + 2 + hh) ^ swz)), qop[s + 1], s1, 0, 0,
                    0);
            }
            // lane holds head `col`, keys 8(i/4) + 4hh + i%4
            float sc[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
                sc[i] = ((vmask >> key) & 1u) ? (s0[i] + s1[i]) * c : -INFINITY;
                tmax = fmaxf(tmax, sc[i]);
            }
            tmax = pair_max(tmax);
            const float m_new = fmaxf(m_run, tmax);  // finite: the tile has a valid key
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            float psum = 0.f;
            bf16x8_t pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);
                psum += p;
                pb[i >> 3][i & 7] = __bf16(p);
            }
            l_run = l_run * alpha + psum;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
            }
            // O^T[dv][head] += V^T[dv][keys] . P^T[keys][head].  The A operand
            // (lane: column 32mb + col, keys 16j + 8rho + 4hh + 0..3 for
            // rho = 0, 1) comes from two LDS transpose reads: in each group of
            // 16 lanes, lane i receives element i % 4 of the 8 bytes addressed
            // by lane 4e + i / 4, for e = 0..3; so lane g*16 + s points at
            // key 16j + 8rho + 4hh + s/4, columns 32mb + 16(g%2) + 4(s%4) ..+3.
            const int g16 = (lane >> 4) & 1;
            const int s16 = lane & 15;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    s4_t part[2];
#pragma unroll
                    for (int rho = 0; rho < 2; ++rho) {
                        const int key = 16 * j + 8 * rho + 4 * hh + (s16 >> 2);
                        const int dv = 32 * mb + 16 * g16 + 4 * (s16 & 3);
                        const int off = key * ROWB + 16 * ((dv >> 3) ^ ((2 * key) % NC)) + 2 * (dv & 7);
                        part[rho] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s4_t *)(vt_lds + off));
                    }
                    const bf16x8_t va = __builtin_bit_cast(
                        bf16x8_t, s8_t{part[0][0], part[0][1], part[0][2], part[0][3],
                                       part[1][0], part[1][1], part[1][2], part[1][3]});
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[j], acc[mb], 0, 0, 0);
                }
        }
    }

    // epilogue: lane holds head `col`, rows dv = 32mb + 8(i/4) + 4hh + i%4
    const float l_tot = pair_sum(l_run);
    if constexpr (SPLIT) {
        float *po = a.part_o + (unit * H + head) * int64_t(D);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4_t *>(po + 32 * mb + 8 * g + 4 * hh) =
                    f32x4_t{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
        if (hh == 0) {
            a.part_ml[(unit * H + head) * 2] = m_run;  // -inf for a range without entries
            a.part_ml[(unit * H + head) * 2 + 1] = l_tot;
        }
        return;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char *orow = a.out + (row * H + head) * int64_t(ROWB);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __bf16(acc[mb][4 * g + e] * inv);
            *reinterpret_cast<u32x2_t *>(orow + 2 * (32 * mb + 8 * g + 4 * hh)) =
                __builtin_bit_cast(u32x2_t, o);
        }
    if (a.lse && hh == 0)
        a.lse[row * H + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

// Merges the n_splits ranges of each row: with M = max_g m_g (log2 units),
// out = sum_g 2^(m_g - M) O_g / sum_g 2^(m_g - M) l_g, in range order.
// 256 threads per row, four output columns each.
template <int H, int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a, int64_t row0, int64_t nrows)
{
    const int64_t row = row0 + blockIdx.x;
    if (blockIdx.x >= nrows) return;
    const int G = a.n_splits;
    for (int w = threadIdx.x; w < H * D / 4; w += 256) {
        const int h = (4 * w) / D;
        const int dv = (4 * w) % D;
        const float *ml = a.part_ml + (row * G * H + h) * 2;  // range g at + g * 2H
        float M = -INFINITY;
        for (int g = 0; g < G; ++g) M = fmaxf(M, ml[g * 2 * H]);
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
        if (M != -INFINITY) {
            for (int g = 0; g < G; ++g) {
                const float sc = __builtin_amdgcn_exp2f(ml[g * 2 * H] - M);
                L += sc * ml[g * 2 * H + 1];
                const f32x4_t og = *reinterpret_cast<const f32x4_t *>(
                    a.part_o + ((row * G + g) * H + h) * int64_t(D) + dv);
                o += sc * og;
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        bf16x4_t ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = __bf16(o[e] * inv);
        *reinterpret_cast<u32x2_t *>(a.out + ((row * H + h) * int64_t(D) + dv) * 2) =
            __builtin_bit_cast(u32x2_t, ob);
        if (a.lse && dv == 0) a.lse[row * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
}

template <int H, int D>
hipError_t launch_hd(const AttnArgs &a, hipStream_t stream)
{
    const int64_t rows = a.B * a.S;
    const bool split = a.n_splits > 1;
    const int64_t units = split ? rows * a.n_splits : rows;
    // at most 2^22 workgroups per launch keeps grid * block far below 2^32
    constexpr int64_t kMaxUnits = int64_t(1) << 22;
    for (int64_t u0 = 0; u0 < units; u0 += kMaxUnits) {
        const int64_t n = units - u0 < kMaxUnits ? units - u0 : kMaxUnits;
        const int64_t grid = kXcds * ((n + kXcds - 1) / kXcds);
        if (split)
            hipLaunchKernelGGL((sparse_attn_kernel<H, D, true>), dim3(unsigned(grid)),
                               dim3(64 * (H / 32)), 0, stream, a, u0, n);
        else
            hipLaunchKernelGGL((sparse_attn_kernel<H, D, false>), dim3(unsigned(grid)),
                               dim3(64 * (H / 32)), 0, stream, a, u0, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!split) return hipSuccess;
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxUnits) {
        const int64_t n = rows - r0 < kMaxUnits ? rows - r0 : kMaxUnits;
        hipLaunchKernelGGL((attn_combine_kernel<H, D>), dim3(unsigned(n)), dim3(256), 0, stream,
                           a, r0, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_sparse_attention(const AttnArgs &a, int H, int D, hipStream_t stream)
{
    if (D == 128) {
        if (H == 32) return launch_hd<32, 128>(a, stream);
        if (H == 64) return launch_hd<64, 128>(a, stream);
        if (H == 128) return launch_hd<128, 128>(a, stream);
    } else if (D == 64) {
        if (H == 32) return launch_hd<32, 64>(a, stream);
        if (H == 64) return launch_hd<64, 64>(a, stream);
        if (H == 128) return launch_hd<128, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa
