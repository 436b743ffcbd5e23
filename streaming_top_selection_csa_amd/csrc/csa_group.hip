// csa_group.hip -- the two helper kernels of the grouped (approximate)
// indexer, the query-group shared scan the PIVOT news item describes
// (themodelwire, "PIVOT reduces sparse attention indexing bottleneck"):
// nearby query positions share one scan of the keys they all see.
//
//   pool_queries_kernel  the pooled query of each group of g consecutive
//       positions: per head, the fp32 mean of the members' q rows (summed
//       in member order, divided by the member count) rounded to bf16
//       (nearest even), and the fp32 mean of their weights.
//   build_lists_kernel   each group's key list for the re-rank: the shared
//       scan's candidates in ascending key order, then the keys only some
//       members see (from the first member's visible count to the last
//       member's), padded with INT32_MAX to the list capacity.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa_group.hpp"

namespace csa {

typedef unsigned short bf16_bits;

__device__ __forceinline__ float bf16_to_f32(bf16_bits b)
{
    return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ bf16_bits f32_to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return bf16_bits(r >> 16);
}

// One thread per (group, head, dimension) element; one per (group, head)
// weight.  Rows [B, S, H, D] -> [B, Sg, H, D].
__global__ void __launch_bounds__(256)
pool_queries_kernel(const bf16_bits *__restrict__ q, const float *__restrict__ w,
                    bf16_bits *__restrict__ qp, float *__restrict__ wp, int64_t B, int64_t S,
                    int H, int D, int g)
{
    const int64_t Sg = (S + g - 1) / g;
    const int64_t nq = B * Sg * H * D;
    const int64_t nw = B * Sg * H;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < nq + nw;
         e += int64_t(gridDim.x) * blockDim.x) {
        if (e < nq) {
            const int64_t x = e % D, hh = (e / D) % H, r = (e / (int64_t(D) * H)) % Sg;
            const int64_t b = e / (int64_t(D) * H * Sg);
            const int64_t t0 = r * g;
            const int n = int(S - t0 < g ? S - t0 : g);
            float sum = 0.f;
            for (int i = 0; i < n; ++i)
                sum += bf16_to_f32(q[(((b * S) + t0 + i) * H + hh) * D + x]);
            qp[e] = f32_to_bf16(sum / float(n));
        } else {
            const int64_t f = e - nq;
            const int64_t hh = f % H, r = (f / H) % Sg, b = f / (int64_t(H) * Sg);
            const int64_t t0 = r * g;
            const int n = int(S - t0 < g ? S - t0 : g);
            float sum = 0.f;
            for (int i = 0; i < n; ++i) sum += w[((b * S) + t0 + i) * H + hh];
            wp[f] = sum / float(n);
        }
    }
}

// One 256-thread workgroup per group: the C candidates (-1 = none) sorted
// ascending in LDS (bitonic), then the extra keys, then padding.
__global__ void __launch_bounds__(256)
build_lists_kernel(const int32_t *__restrict__ cand, int32_t *__restrict__ lists,
                   int32_t *__restrict__ lens, int64_t B, int64_t S, int64_t T, int64_t row_offset,
                   int m, int g, int C, int cap)
{
    extern __shared__ int32_t s_c[];  // next_pow2(C) entries
    const int64_t Sg = (S + g - 1) / g;
    int pow2 = 1;
    while (pow2 < C) pow2 <<= 1;
    for (int64_t grp = blockIdx.x; grp < B * Sg; grp += gridDim.x) {
        const int64_t r = grp % Sg;
        const int64_t t_first = row_offset + r * g;
        const int64_t t_last = row_offset + (r * g + g < S ? r * g + g : S) - 1;
        const int64_t n_first = (t_first + 1) / m < T ? (t_first + 1) / m : T;
        const int64_t n_last = (t_last + 1) / m < T ? (t_last + 1) / m : T;
        for (int e = threadIdx.x; e < pow2; e += blockDim.x) {
            const int32_t v = e < C ? cand[grp * C + e] : -1;
            s_c[e] = v < 0 ? INT32_MAX : v;
        }
        __syncthreads();
        for (int size = 2; size <= pow2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = threadIdx.x; i < pow2 / 2; i += blockDim.x) {
                    const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool up = (lo & size) == 0;
                    const int32_t x = s_c[lo], y = s_c[hi];
                    if ((x > y) == up) {
                        s_c[lo] = y;
                        s_c[hi] = x;
                    }
                }
                __syncthreads();
            }
        }
        // valid candidates come first after the sort
        __shared__ int s_nc;
        if (threadIdx.x == 0) {
            int lo = 0, hi = C;  // first entry that is INT32_MAX
            while (lo < hi) {
                const int mid = (lo + hi) / 2;
                if (s_c[mid] == INT32_MAX) hi = mid; else lo = mid + 1;
            }
            s_nc = lo;
        }
        __syncthreads();
        const int nc = s_nc;
        const int nx = int(n_last - n_first);
        int32_t *out = lists + grp * cap;
        for (int e = threadIdx.x; e < cap; e += blockDim.x) {
            int32_t v = INT32_MAX;
            if (e < nc) v = s_c[e];
            else if (e < nc + nx) v = int32_t(n_first + (e - nc));
            out[e] = v;
        }
        if (threadIdx.x == 0) lens[grp] = nc + nx;
        __syncthreads();
    }
}

hipError_t launch_pool_queries(const void *q, const float *w, void *qp, float *wp, int64_t B,
                               int64_t S, int H, int D, int g, int num_cus, hipStream_t s)
{
    const int64_t Sg = (S + g - 1) / g;
    const int64_t n = B * Sg * H * (D + 1);
    if (n == 0) return hipSuccess;
    const int64_t want = int64_t(num_cus) * 16;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(pool_queries_kernel, dim3(int(blocks < want ? blocks : want)), dim3(256), 0,
                       s, static_cast<const bf16_bits *>(q), w, static_cast<bf16_bits *>(qp), wp,
                       B, S, H, D, g);
    return hipGetLastError();
}

hipError_t launch_build_lists(const int32_t *cand, int32_t *lists, int32_t *lens, int64_t B,
                              int64_t S, int64_t T, int64_t row_offset, int m, int g, int C,
                              int cap, int num_cus, hipStream_t s)
{
    const int64_t groups = B * ((S + g - 1) / g);
    if (groups == 0) return hipSuccess;
    int pow2 = 1;
    while (pow2 < C) pow2 <<= 1;
    const int64_t want = int64_t(num_cus) * 8;
    hipLaunchKernelGGL(build_lists_kernel, dim3(int(groups < want ? groups : want)), dim3(256),
                       size_t(pow2) * 4, s, cand, lists, lens, B, S, T, row_offset, m, g, C, cap);
    return hipGetLastError();
}

}  // namespace csa
