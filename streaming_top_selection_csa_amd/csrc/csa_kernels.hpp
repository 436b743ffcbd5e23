// csa_kernels.hpp -- launch interface of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "csa_plan.hpp"

namespace csa {

// Arguments of the scoring kernel (device pointers; sizes from the plan).
struct StreamArgs {
    const unsigned char *q;     // [B, S, H, D] bf16 or e4m3fn
    const float *w;             // [B, S, H]
    const unsigned char *k;     // [B, T, D]
    const float *q_scale;       // [B, S, H] (fp8) or null
    const float *k_scale;       // [B, T] (fp8) or null
    int32_t *out_idx;           // [B, S, k]
    float *out_score;           // [B, S, k]
    uint32_t *ws;               // candidate logs: grid * 8 waves * QW * log_cap * 8 bytes
    int64_t B, S, T, row_offset;
    int m, topk, log_cap;
    int64_t blocks_per_batch, n_blocks;
};

hipError_t launch_stream_topk(const Plan &p, const StreamArgs &a, hipStream_t s);
hipError_t launch_sort_rows(const Plan &p, int32_t *out_idx, float *out_score, int num_cus,
                            hipStream_t s);

}  // namespace csa
