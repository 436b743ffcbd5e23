// csa_plan.cpp -- argument validation and launch planning (host only).
#include "csa_plan.hpp"

#include <algorithm>

namespace csa {

bool supported(int dtype, int H, int D)
{
    const bool h_ok = H == 1 || H == 2 || H == 4 || H == 8 || H == 16 ||
                      H == 32 || H == 64;
    if (!h_ok) return false;
    if (dtype == CSA_BF16) return D == 32 || D == 64 || D == 128;
    if (dtype == CSA_FP8_E4M3FN) return D == 64 || D == 128;
    return false;
}

bool key_tile_supported(int key_tile, int dtype, int H, int D)
{
    if (key_tile == kKeysPerTile) return true;
    if (H != 64 || D != 128) return false;
    if (dtype == CSA_FP8_E4M3FN) return key_tile == 128 || key_tile == 256;
    return key_tile == 32 || key_tile == 128 || key_tile == 192 || key_tile == 256;
}

int default_key_tile(int H, int D, int dtype)
{
    // several 64-key compute tiles per staged tile cut the workgroup
    // barriers (measured faster at H_I = 64, d_I = 128: two for bf16, whose
    // larger tiles spill or leave room for only two buffers; four for fp8,
    // whose 128-byte rows still fit a ring of three)
    if (H != 64 || D != 128) return kKeysPerTile;
    return dtype == CSA_FP8_E4M3FN ? 256 : 128;
}

static int64_t next_pow2(int64_t x)
{
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

int make_plan(const csa_desc *desc, int32_t m, int32_t k,
              const csa_options *opt, int num_cus, Plan *plan, bool no_score, int64_t pos_mul)
{
    if (!desc || !plan || num_cus <= 0 || pos_mul < 1 || pos_mul > (int64_t(1) << 20))
        return CSA_ERR_INVALID_ARG;
    if (desc->B < 1 || desc->S < 0 || desc->T < 0) return CSA_ERR_INVALID_ARG;
    // key indices and the kernels' key arithmetic (tile ends, key ranges) are
    // 32-bit: T <= 2^30 keeps every such sum below 2^31
    if (desc->T > kMaxKeys) return CSA_ERR_INVALID_ARG;
    if (desc->reserved0 != 0) return CSA_ERR_INVALID_ARG;
    if (m < 1 || k < 1) return CSA_ERR_INVALID_ARG;
    if (desc->dtype != CSA_BF16 && desc->dtype != CSA_FP8_E4M3FN)
        return CSA_ERR_INVALID_ARG;
    const bool fp8 = desc->dtype == CSA_FP8_E4M3FN;
    if (fp8 && (!desc->q_scale || !desc->k_scale)) return CSA_ERR_INVALID_ARG;
    if (!fp8 && (desc->q_scale || desc->k_scale)) return CSA_ERR_INVALID_ARG;
    if (!supported(desc->dtype, desc->H, desc->D)) return CSA_ERR_UNSUPPORTED;
    if (k > kMaxTopK) return CSA_ERR_UNSUPPORTED;

    int64_t row_offset = 0;
    int chunk = 0;
    int splits_req = 0;
    int key_tile = 0;
    if (opt) {
        if (opt->reserved2 != 0 || opt->key_tile < 0) return CSA_ERR_INVALID_ARG;
        key_tile = opt->key_tile;
        if (opt->row_offset < 0 || opt->chunk_keys < 0 || opt->chunk_keys > kMaxChunk)
            return CSA_ERR_INVALID_ARG;
        if (opt->key_splits < 0 || (opt->flags & ~int32_t(CSA_FLAG_NO_SCORE)) != 0)
            return CSA_ERR_INVALID_ARG;
        if (opt->flags & CSA_FLAG_NO_SCORE) no_score = true;
        row_offset = opt->row_offset;
        chunk = opt->chunk_keys;
        splits_req = opt->key_splits;
    }
    // positions must stay representable: t + 1 fits comfortably in int64
    if (desc->S > (int64_t(1) << 40) || row_offset > (int64_t(1) << 40) ||
        desc->S * pos_mul > (int64_t(1) << 41))
        return CSA_ERR_INVALID_ARG;
    // element counts must fit the 64-bit offsets used by the kernels (checked
    // before multiplying: a signed overflow would already be undefined)
    if (desc->S > 0 && desc->B > INT64_MAX / desc->S) return CSA_ERR_INVALID_ARG;
    const int64_t rows = desc->B * desc->S;
    if (rows > (int64_t(1) << 46) / (int64_t(desc->H) * desc->D)) return CSA_ERR_INVALID_ARG;
    if (rows > (int64_t(1) << 46) / k) return CSA_ERR_INVALID_ARG;

    if (chunk == 0) {  // default partition: 4k, within [1024, 8192]
        const int64_t c = int64_t(4) * k;
        chunk = int(c < 1024 ? 1024 : (c > 8192 ? 8192 : c));
    }
    chunk = (chunk + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile;

    Plan p;
    p.B = desc->B;
    p.S = desc->S;
    p.T = desc->T;
    p.row_offset = row_offset;
    p.H = desc->H;
    p.D = desc->D;
    p.fp8 = fp8 ? 1 : 0;
    p.m = m;
    p.k = k;
    p.QW = kRowsPerWave / desc->H;
    p.QB = kWaves * p.QW;
    p.blocks_per_batch = (desc->S + p.QB - 1) / p.QB;
    p.n_blocks = p.blocks_per_batch * desc->B;
    const int64_t resident = int64_t(num_cus);  // one 8-wave workgroup per CU

    // key ranges: requested, or automatic when the query blocks leave CUs idle
    const int64_t last_pos = row_offset + (desc->S - 1) * pos_mul;  // position of the last row
    const int64_t n_max = desc->S > 0 ? std::min<int64_t>(desc->T, (last_pos + 1) / m) : 0;
    const int64_t tiles = (n_max + kKeysPerTile - 1) / kKeysPerTile;
    int64_t G = 1;
    if (splits_req > 0) {
        G = std::min<int64_t>(splits_req, tiles);
    } else if (p.n_blocks > 0 && p.n_blocks < resident) {
        // a range of at least 9k/8 keys: the merge reads G*k entries per
        // position, the scoring of a unit takes keys/G (measured on 64
        // decode positions over 65,536 keys and on 32 x 4 over 16,384: the
        // call is fastest with ranges of 1.1k to 1.4k keys)
        const int64_t min_keys = std::max<int64_t>(int64_t(k) + k / 8, kMinSplitKeys);
        G = std::min<int64_t>((resident + p.n_blocks - 1) / p.n_blocks, n_max / min_keys);
    }
    // the partial lists take rows*G*k*8 bytes: an automatic G keeps them
    // under 1 GiB, a requested one under 64 GiB
    const size_t list_cap = splits_req > 0 ? kMaxSplitBytesRequested : kMaxSplitBytes;
    const int64_t g_cap = int64_t(list_cap / (size_t(rows > 0 ? rows : 1) * size_t(k) * 8u));
    G = std::max<int64_t>(1, std::min(G, g_cap));
    if (G > 1) {
        const int64_t per = (n_max + G - 1) / G;
        p.split_keys = int((per + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile);
        G = (n_max + p.split_keys - 1) / p.split_keys;
    }
    p.n_splits = int(G);
    if (p.n_splits == 1) p.split_keys = 0;
    p.n_units = p.n_blocks * p.n_splits;
    p.grid = int(p.n_units < resident ? p.n_units : resident);
    p.chunk = chunk;
    // rounded up so that the final selection can read whole groups of
    // entries with 16-byte loads
    p.log_cap = int((int64_t(k) + chunk + kLogCapMultiple - 1) / kLogCapMultiple * kLogCapMultiple);
    p.sort_pow2 = int(next_pow2(k));
    // rows of up to kMaxFusedSort slots are sorted at the end of the scoring
    // kernel (no key ranges); the others by a separate pass, which needs the
    // scores, in the workspace when the caller wants none
    p.sort_e = (p.n_splits == 1 && p.sort_pow2 <= kMaxFusedSort)
                   ? (p.sort_pow2 <= 64 ? 1 : p.sort_pow2 <= 512 ? 8 : 32)
                   : 0;
    // with key ranges and fewer rows than compute units (short query blocks)
    // the merge kernel, one workgroup per row, also sorts the row
    p.merge_sorts = p.n_splits > 1 && p.sort_pow2 <= kMaxFusedSort && rows < resident;
    // the sorted-row kernel has several key tiles; the unsorted one (key
    // ranges, or rows sorted by a later pass) 64 everywhere and 128 at
    // bf16, H = 64, D = 128 (half the barriers: measured 2-3% faster on
    // decode calls)
    const bool wide = desc->dtype == CSA_BF16 && desc->H == 64 && desc->D == 128;
    if (key_tile == 0) key_tile = p.sort_e > 0 ? default_key_tile(desc->H, desc->D, desc->dtype)
                                               : (wide ? 128 : kKeysPerTile);
    if (key_tile != kKeysPerTile &&
        (p.sort_e > 0 ? !key_tile_supported(key_tile, desc->dtype, desc->H, desc->D)
                      : !(wide && key_tile == 128)))
        return CSA_ERR_UNSUPPORTED;
    p.key_tile = key_tile;
    p.no_score = no_score;
    p.pos_mul = pos_mul;
    const size_t per_wave = size_t(p.QW) * size_t(p.log_cap) * 8u;  // u32 key + i32 index
    const size_t logs = (size_t(p.grid) * kWaves * per_wave + 255) / 256 * 256;
    p.part_offset = logs;
    const size_t parts = p.n_splits > 1 ? size_t(rows) * size_t(p.n_splits) * size_t(k) * 8u : 0u;
    p.score_offset = logs + (parts + 255) / 256 * 256;
    const size_t scores =
        (no_score && p.sort_e == 0 && !p.merge_sorts) ? size_t(rows) * size_t(k) * 4u : 0u;
    p.ws_bytes = p.score_offset + (scores + 255) / 256 * 256;
    *plan = p;
    return CSA_OK;
}

}  // namespace csa
