// csa_group.hpp -- launchers of the grouped indexer's helper kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace csa {

// Pooled queries: qp [B, Sg, H, D] bf16 and wp [B, Sg, H] fp32, Sg = ceil(S/g).
hipError_t launch_pool_queries(const void *q, const float *w, void *qp, float *wp, int64_t B,
                               int64_t S, int H, int D, int g, int num_cus, hipStream_t s);
// Key lists [B*Sg, cap] and their lengths from the candidates [B*Sg, C]
// (-1 = none); C <= 2048.
hipError_t launch_build_lists(const int32_t *cand, int32_t *lists, int32_t *lens, int64_t B,
                              int64_t S, int64_t T, int64_t row_offset, int m, int g, int C,
                              int cap, int num_cus, hipStream_t s);

}  // namespace csa
