// csa_stream_fp8_d64.hip -- scoring-kernel instantiations for e4m3fn
// operands of head dimension 64, every head count, with and without key
// ranges (one file per type and dimension so that they compile in parallel).
#include "csa_stream.hpp"

namespace csa {

hipError_t launch_stream_fp8_d64(int H, const StreamArgs &a, int grid, hipStream_t s)
{
    return launch_h<64, true>(H, a, grid, s);
}

}  // namespace csa
