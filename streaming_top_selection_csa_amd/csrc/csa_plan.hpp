// csa_plan.hpp -- host-side validation and launch planning (no HIP calls).
//
// The plan splits the query positions of every batch entry into blocks of
// QB consecutive positions (one workgroup of 8 waves; each wave owns 64
// (position, head) rows of q = 64/H positions).  A persistent grid walks the
// blocks heaviest-first; each wave streams the visible compressed keys of its
// positions in ascending order, 64 keys per staged tile, and keeps a running
// top-k per position in a bounded candidate log of k + chunk entries
// (StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
// Top-k, Abstract: the keys are taken in chunks and each chunk's winners are
// merged into the running set, so the full score tensor is never formed).  The workspace therefore depends on the grid, k and
// the chunk size, never on S or T.
//
// When the query blocks are too few to fill the device (a short query block
// at the end of a long context, a decode step) the visible keys are also
// split into G ranges of split_keys keys: each (query block, key range) unit
// produces the exact top-k of its range, and a merge pass selects the top-k
// of the G partial lists per position.  Only then does the workspace grow,
// by B*S*G*k candidate entries.
#pragma once

#include <cstddef>
#include <cstdint>

#include "csa_index.h"

namespace csa {

constexpr int kWaves = 8;           // waves per workgroup (two per SIMD, one workgroup per CU)
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;    // (position, head) rows of q per wave
constexpr int kKeysPerTile = 64;    // compressed keys per compute tile (one key per lane)
constexpr int kMaxTopK = 16384;     // row sort holds next_pow2(k) keys in LDS
constexpr int kMaxFusedSort = 2048; // rows up to this next_pow2(k) are sorted by the scoring kernel
constexpr int kMaxChunk = 1 << 20;
constexpr int kLogCapMultiple = 8;  // candidate-log capacity granularity (entries)
constexpr int64_t kMaxKeys = int64_t(1) << 30;   // largest T
constexpr int kMinSplitKeys = 1024;              // smallest automatic key range
constexpr size_t kMaxSplitBytes = size_t(1) << 30;  // bound of the partial lists (automatic G)
constexpr size_t kMaxSplitBytesRequested = size_t(1) << 36;  // same, G set by the caller

struct Plan {
    int64_t B = 0, S = 0, T = 0, row_offset = 0;
    int H = 0, D = 0, fp8 = 0, m = 0, k = 0;
    int QW = 0;                 // positions per wave (64 / H)
    int QB = 0;                 // positions per block (8 * QW)
    int64_t blocks_per_batch = 0;
    int64_t n_blocks = 0;       // query blocks over all batch entries
    int n_splits = 1;           // key ranges per query block (G)
    int split_keys = 0;         // keys per range (multiple of 64) when G > 1
    int64_t n_units = 0;        // n_blocks * n_splits scoring units
    int grid = 0;               // scoring workgroups (persistent)
    int chunk = 0;              // candidates buffered beyond k before a merge
    int log_cap = 0;            // k + chunk
    int sort_pow2 = 0;          // next power of two >= k
    int sort_e = 0;             // > 0: the scoring kernel sorts the rows (sort_e keys per lane)
    bool merge_sorts = false;   // key ranges, few rows: the merge kernel sorts the rows
    int key_tile = kKeysPerTile;  // keys staged in LDS per workgroup step
    bool no_score = false;      // the caller passes no score output
    int64_t pos_mul = 1;        // q row i is position row_offset + i * pos_mul
    size_t part_offset = 0;     // byte offset of the partial lists (G > 1)
    size_t score_offset = 0;    // byte offset of the score rows a separate sort needs
    size_t ws_bytes = 0;        // 256-aligned
};

bool supported(int dtype, int H, int D);
// Staged key tiles other than kKeysPerTile are built for H = 64, D = 128
// only (bf16: 32, 128, 192, 256; fp8: 128); the default there is 128.
bool key_tile_supported(int key_tile, int dtype, int H, int D);
int default_key_tile(int H, int D, int dtype);

// Validates every argument and fills `plan`.  num_cus must be > 0.
// no_score: the call writes no scores (also implied by CSA_FLAG_NO_SCORE).
// Returns CSA_OK or a negative csa_status; never throws.
// pos_mul: q row i is position row_offset + i * pos_mul (the grouped scan's
// pooled rows stand for every pos_mul-th position).
int make_plan(const csa_desc *desc, int32_t m, int32_t k,
              const csa_options *opt, int num_cus, Plan *plan, bool no_score = false,
              int64_t pos_mul = 1);

}  // namespace csa
