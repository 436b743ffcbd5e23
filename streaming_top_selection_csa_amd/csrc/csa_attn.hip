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
// One workgroup per query row, one wave per 32 heads.  The row's selected
// entries are taken 32 at a time: the workgroup gathers the 32 key rows and
// 32 value rows (each a contiguous D*2-byte row; 16 lanes per row, so every
// load is a full row segment) into LDS, then every wave
//   * computes the 32x32 block S^T = K_tile . Q^T of (key, head) scores with
//     v_mfma_f32_32x32x16_bf16: A = the key rows from LDS, B = the wave's 32
//     query heads, held in registers for the whole row;
//   * runs the online softmax: in the MFMA output layout each lane holds one
//     head (lane % 32) and 16 of the tile's keys, so the running maximum and
//     the sum stay in the lane, and the two lanes of a head agree through one
//     v_permlane32_swap;
//   * accumulates O^T += V_tile^T . P^T: B = the bf16 weights straight from
//     the lane's score registers, A = the value tile, stored transposed in
//     LDS with the tile's keys permuted so that each lane's eight keys of a
//     K step are the eight keys its weights belong to.
// The gather of the next tile is issued before the current tile's MFMA work
// and lands in registers, so the (mostly L2 / MALL) gather latency overlaps
// compute.  Rows are mapped to workgroups so that consecutive rows share an
// XCD (and its L2): queries close in position tend to pick the same keys.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_kernels.hpp"

namespace csa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

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

// Position of tile key `key` in a transposed value row.  The PV product's K
// step j pairs lane half hh, element e with key 16j + 8(e/4) + 4hh + e%4 (the
// keys that score-output element 8j + e of that lane half holds); swapping
// bits 2 and 3 of the key puts those eight keys at 16j + 8hh + e, one 16-byte
// read.
__device__ __forceinline__ int vt_pos(int key)
{
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int H, int D>
__global__ void __launch_bounds__(64 * (H / 32))
sparse_attn_kernel(AttnArgs a, int64_t row0, int64_t nrows)
{
    constexpr int W = H / 32;              // waves; wave w owns heads 32w .. 32w+31
    constexpr int NT = 64 * W;
    constexpr int CH = D / 8;              // 16-byte chunks per key or value row
    constexpr int PER_KEY = 2 * CH;        // chunks of one entry (key row + value row)
    constexpr int KPP = NT / PER_KEY;      // entries gathered per pass of the workgroup
    constexpr int NLD = KT / KPP;          // gather passes per tile
    constexpr int KS = D / 16;             // K steps of the score product
    constexpr int MB = D / 32;             // 32-row blocks of the output
    constexpr int KROW = 2 * D + 16;       // LDS bytes per key row (16-byte pad)
    constexpr int VROW = 2 * KT + 16;      // LDS bytes per transposed value row
    static_assert(NT % PER_KEY == 0 && KT % KPP == 0, "gather layout");

    __shared__ __attribute__((aligned(16))) unsigned char s_k[KT * KROW];
    __shared__ __attribute__((aligned(16))) unsigned char s_v[D * VROW];
    __shared__ int s_valid[KT];

    // consecutive rows on one XCD: workgroup i runs on XCD i % 8
    const int64_t per_xcd = (nrows + kXcds - 1) / kXcds;
    const int64_t slot = int64_t(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (slot >= nrows) return;  // whole workgroup, before any barrier
    const int64_t row = row0 + slot;
    const int64_t b = row / a.S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hh = lane >> 5;              // lane half: K slice of MFMA operands
    const int col = lane & 31;
    const int head = 32 * (tid >> 6) + col;

    // B operand of the score product: q[row, head, 16s + 8hh .. +8]
    bf16x8_t qop[KS];
    {
        const unsigned char *qr = a.q + (row * H + head) * int64_t(2 * D) + 16 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = as_op(*reinterpret_cast<const u32x4_t *>(qr + 32 * s));
    }

    // gather role: this thread moves 16-byte chunk `ch` of the key row (or of
    // the value row) of entries i*KPP + ent, i < NLD, of every tile
    const int part = tid % PER_KEY;
    const int ent = tid / PER_KEY;
    const bool is_v = part >= CH;
    const int ch = is_v ? part - CH : part;
    const unsigned char *src = (is_v ? a.v : a.k) + b * a.T * int64_t(2 * D) + 16 * ch;
    const int32_t *list = a.idx + row * int64_t(a.n_sel);
    const int n_sel = a.n_sel;
    const int64_t T = a.T;
    const int ntiles = (n_sel + KT - 1) / KT;

    int cur[NLD], nxt[NLD];
    u32x4_t stage[NLD];

    auto load_ids = [&](int tile, int *ids) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int pos = tile * KT + i * KPP + ent;
            int s = pos < n_sel ? list[pos] : -1;
            ids[i] = (s >= 0 && s < T) ? s : -1;
        }
    };
    auto gather = [&](const int *ids) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            stage[i] = ids[i] >= 0 ? *reinterpret_cast<const u32x4_t *>(src + int64_t(ids[i]) * (2 * D))
                                   : u32x4_t{0, 0, 0, 0};
    };
    auto to_lds = [&](const int *ids) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int key = i * KPP + ent;
            if (!is_v) {
                *reinterpret_cast<u32x4_t *>(s_k + key * KROW + 16 * ch) = stage[i];
                if (ch == 0) s_valid[key] = ids[i] >= 0;
            } else {
                unsigned char *dst = s_v + (8 * ch) * VROW + 2 * vt_pos(key);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned x = stage[i][e];
                    *reinterpret_cast<uint16_t *>(dst + (2 * e) * VROW) = uint16_t(x);
                    *reinterpret_cast<uint16_t *>(dst + (2 * e + 1) * VROW) = uint16_t(x >> 16);
                }
            }
        }
    };

    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
    float m_run = -INFINITY;  // running maximum of the head's scores, log2 units
    float l_run = 0.f;        // this lane's part of the running sum of weights
    const float c = a.scale * kLog2e;

    load_ids(0, cur);
    gather(cur);
    load_ids(1, nxt);
    to_lds(cur);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const bool more = it + 1 < ntiles;
        if (more) gather(nxt);  // in flight during this tile's work
        int later[NLD];
        load_ids(it + 2, later);

        const uint32_t vmask =
            uint32_t(__builtin_amdgcn_ballot_w64(s_valid[col] != 0));  // bit = tile key
        if (vmask != 0) {
            // S^T[key][head] for the tile's 32 keys and the wave's 32 heads
            f32x16_t sc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = 0.f;
            const unsigned char *krow = s_k + col * KROW + 16 * hh;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(krow + 32 * s), qop[s], sc, 0,
                                                             0, 0);
            // lane holds head `col`, keys 8(i/4) + 4hh + i%4
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
                sc[i] = ((vmask >> key) & 1u) ? sc[i] * c : -INFINITY;
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
            // O^T[dv][head] += V^T[dv][keys] . P^T[keys][head]
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        lds_op(s_v + (32 * mb + col) * VROW + 32 * j + 16 * hh), pb[j], acc[mb],
                        0, 0, 0);
        }
        __syncthreads();  // every wave is done with the tile
        if (more) to_lds(nxt);
#pragma unroll
        for (int i = 0; i < NLD; ++i) nxt[i] = later[i];
        __syncthreads();
    }

    // epilogue: lane holds head `col`, rows dv = 32mb + 8(i/4) + 4hh + i%4
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char *orow = a.out + (row * H + head) * int64_t(2 * D);
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

template <int H, int D>
hipError_t launch_hd(const AttnArgs &a, hipStream_t stream)
{
    const int64_t rows = a.B * a.S;
    // at most 2^22 rows per launch keeps grid * block far below 2^32
    constexpr int64_t kMaxRows = int64_t(1) << 22;
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxRows) {
        const int64_t n = rows - r0 < kMaxRows ? rows - r0 : kMaxRows;
        const int64_t grid = kXcds * ((n + kXcds - 1) / kXcds);
        hipLaunchKernelGGL((sparse_attn_kernel<H, D>), dim3(unsigned(grid)), dim3(64 * (H / 32)),
                           0, stream, a, r0, n);
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
