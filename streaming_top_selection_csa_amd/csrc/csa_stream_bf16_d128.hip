// csa_stream_bf16_d128.hip -- scoring-kernel instantiations for bf16
// operands of head dimension 128, every head count, with and without key
// ranges (one file per type and dimension so that they compile in parallel).
#include "csa_stream.hpp"

namespace csa {

hipError_t launch_stream_bf16_d128(int H, const StreamArgs &a, int grid, hipStream_t s)
{
    return launch_h<128, false>(H, a, grid, s);
}

}  // namespace csa
