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

static int64_t next_pow2(int64_t x)
{
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

int make_plan(const csa_desc *desc, int32_t m, int32_t k,
              const csa_options *opt, int num_cus, Plan *plan)
{
    if (!desc || !plan || num_cus <= 0) return CSA_ERR_INVALID_ARG;
    if (desc->B < 1 || desc->S < 0 || desc->T < 0) return CSA_ERR_INVALID_ARG;
    if (desc->T > INT32_MAX - 1) return CSA_ERR_INVALID_ARG;  // int32 key indices
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
    if (opt) {
        if (opt->row_offset < 0 || opt->chunk_keys < 0 || opt->chunk_keys > kMaxChunk)
            return CSA_ERR_INVALID_ARG;
        if (opt->key_splits < 0 || opt->reserved1 != 0) return CSA_ERR_INVALID_ARG;
        row_offset = opt->row_offset;
        chunk = opt->chunk_keys;
        splits_req = opt->key_splits;
    }
    // positions must stay representable: t + 1 fits comfortably in int64
    if (desc->S > (int64_t(1) << 40) || row_offset > (int64_t(1) << 40))
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
    const int64_t n_max = desc->S > 0 ? std::min<int64_t>(desc->T, (row_offset + desc->S) / m) : 0;
    const int64_t tiles = (n_max + kKeysPerTile - 1) / kKeysPerTile;
    int64_t G = 1;
    if (splits_req > 0) {
        G = std::min<int64_t>(splits_req, tiles);
    } else if (p.n_blocks > 0 && p.n_blocks < resident) {
        // a range of at least 2k keys: the merge reads G*k entries per
        // position, the scoring of a unit takes keys/G
        const int64_t min_keys = std::max<int64_t>(int64_t(2) * k, kMinSplitKeys);
        G = std::min<int64_t>((resident + p.n_blocks - 1) / p.n_blocks, n_max / min_keys);
    }
    const int64_t g_cap = int64_t(kMaxSplitBytes / (size_t(rows > 0 ? rows : 1) * size_t(k) * 8u));
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
    p.log_cap = k + chunk;
    p.sort_pow2 = int(next_pow2(k));
    const size_t per_wave = size_t(p.QW) * size_t(p.log_cap) * 8u;  // u32 key + i32 index
    const size_t logs = (size_t(p.grid) * kWaves * per_wave + 255) / 256 * 256;
    p.part_offset = logs;
    const size_t parts = p.n_splits > 1 ? size_t(rows) * size_t(p.n_splits) * size_t(k) * 8u : 0u;
    p.ws_bytes = logs + (parts + 255) / 256 * 256;
    *plan = p;
    return CSA_OK;
}

}  // namespace csa
