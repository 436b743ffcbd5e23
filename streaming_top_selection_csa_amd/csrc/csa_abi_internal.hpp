// csa_abi_internal.hpp -- host pieces of the C ABI shared by its source files.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "csa_index.h"
#include "csa_plan.hpp"

namespace csa {

// Key lists of the grouped re-rank (see StreamArgs).
struct ListArgs {
    const int32_t *klist;
    const int32_t *klen;
    int64_t n_lists;
    int list_cap, list_rows;
};

// Compute units of the current device; CSA_OK or CSA_ERR_HIP.
int device_cus(int *out);
// Validates and plans a call (no device work when opt->num_cus > 0).
int plan_call(const csa_desc *desc, int32_t m, int32_t k, const csa_options *opt, Plan *p,
              int *cus, bool no_score, int64_t pos_mul);
// Enqueues a planned call on `stream`; ws holds p.ws_bytes bytes.
int run_index(const Plan &p, int cus, const void *q, const float *w, const void *k_cmp,
              const float *q_scale, const float *k_scale, int32_t *out_idx, float *out_score,
              void *ws, const hipEvent_t *timing, hipStream_t stream, const ListArgs *lists);
bool aligned(const void *p, uintptr_t a);

}  // namespace csa
