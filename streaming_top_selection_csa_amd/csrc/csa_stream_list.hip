// csa_stream_list.hip -- the grouped indexer's instantiations of the scoring
// kernel (bf16, H_I = 64, d_I = 128): over key lists (the re-rank; 128-key
// staged tiles, rows sorted in the kernel) and over pooled query rows (the
// shared scan; sorted rows, or unsorted lists for the row sort).
#include "csa_stream.hpp"

namespace csa {

hipError_t launch_stream_list(const StreamArgs &a, int grid, hipStream_t s)
{
    if (a.sort_e <= 0 || a.key_tile != 128 || !a.klist || !a.klen || a.list_rows <= 0 ||
        a.list_cap % 128 != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_topk_kernel<64, 128, false, false, 128, kList>), dim3(grid),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_stream_pooled(const StreamArgs &a, int grid, hipStream_t s)
{
    if (a.sort_e == 0) {
        hipLaunchKernelGGL((stream_topk_kernel<64, 128, false, true, kKeysPerTile, kPooled>),
                           dim3(grid), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    if (a.key_tile != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((stream_topk_kernel<64, 128, false, false, 128, kPooled>), dim3(grid),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace csa
