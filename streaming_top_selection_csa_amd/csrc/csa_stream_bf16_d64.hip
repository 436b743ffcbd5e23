// csa_stream_bf16_d64.hip -- scoring-kernel instantiations for bf16
// operands of head dimension 64, every head count, with and without key
// ranges (one file per type and dimension so that they compile in parallel).
#include "csa_stream.hpp"

namespace csa {

hipError_t launch_stream_bf16_d64(int H, const StreamArgs &a, int grid, hipStream_t s)
{
    return launch_h<64, false>(H, a, grid, s);
}

}  // namespace csa
