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
    float *out_score;           // [B, S, k]; may be null when the rows are sorted in the kernel
    uint32_t *ws;               // candidate logs: grid * 8 waves * QW * log_cap * 8 bytes
    int32_t *part_idx;          // [B, S, G, k] per-key-range top-k lists (G > 1)
    float *part_score;          // [B, S, G, k]
    int64_t B, S, T, row_offset;
    int m, topk, log_cap;
    int n_splits, split_keys;   // G key ranges of split_keys keys (G = 1: all keys)
    int64_t blocks_per_batch, n_units;
    int sort_e;                 // > 0: rows sorted in the kernel, sort_e keys per lane
    int key_tile;               // keys staged in LDS per workgroup step
    int64_t pos_mul;            // q row i is position row_offset + i * pos_mul (1: rows)
    // key lists (grouped re-rank): list l holds ascending key indices for
    // list_rows consecutive rows, list_cap entries (a multiple of the key
    // tile, INT32_MAX past its klen[l] valid ones)
    const int32_t *klist;       // [B, n_lists, list_cap] or null
    const int32_t *klen;        // [B, n_lists]
    int64_t n_lists;
    int list_cap, list_rows;
};

hipError_t launch_stream_topk(const Plan &p, const StreamArgs &a, hipStream_t s);
// The scoring kernel over key lists (bf16, H = 64, D = 128, sorted rows).
hipError_t launch_stream_list(const StreamArgs &a, int grid, hipStream_t s);
// The scoring kernel over pooled query rows (bf16, H = 64, D = 128).
hipError_t launch_stream_pooled(const StreamArgs &a, int grid, hipStream_t s);
// per operand type and head dimension (csa_stream_*.hip)
hipError_t launch_stream_bf16_d32(int H, const StreamArgs &a, int grid, hipStream_t s);
hipError_t launch_stream_bf16_d64(int H, const StreamArgs &a, int grid, hipStream_t s);
hipError_t launch_stream_bf16_d128(int H, const StreamArgs &a, int grid, hipStream_t s);
hipError_t launch_stream_fp8_d64(int H, const StreamArgs &a, int grid, hipStream_t s);
hipError_t launch_stream_fp8_d128(int H, const StreamArgs &a, int grid, hipStream_t s);
// Top-k of the G partial lists of every position into the (unsorted) rows.
hipError_t launch_merge_splits(const Plan &p, const int32_t *part_idx, const float *part_score,
                               int32_t *out_idx, float *out_score, int num_cus, hipStream_t s);
hipError_t launch_sort_rows(const Plan &p, int32_t *out_idx, float *out_score, int num_cus,
                            hipStream_t s);

// Arguments of the sparse-attention kernel (device pointers, row-major).
struct AttnArgs {
    const unsigned char *q;     // [B, S, H, D] bf16
    const unsigned char *k;     // [B, T, D] bf16
    const unsigned char *v;     // [B, T, D] bf16
    const int32_t *idx;         // [B, S, n_sel]; entries outside [0, T) are padding
    unsigned char *out;         // [B, S, H, D] bf16
    float *lse;                 // [B, S, H] or null
    int64_t B, S, T;
    int n_sel;
    float scale;                // multiplies q . k
    int n_splits;               // ranges per row (1: none)
    int split_entries;          // entries per range (a multiple of 32)
    float *part_o;              // [B*S*n_splits, H, D] unnormalised range outputs
    float *part_ml;             // [B*S*n_splits, H, 2] range maximum (log2 units), weight sum
};

// H in {32, 64, 128}, D in {64, 128}; anything else is hipErrorInvalidValue.
hipError_t launch_sparse_attention(const AttnArgs &a, int H, int D, hipStream_t s);

}  // namespace csa
