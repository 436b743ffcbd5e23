// csa_plan.cpp -- argument validation and launch planning (host only).
#include "csa_plan.hpp"

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
    if (opt) {
        if (opt->row_offset < 0 || opt->chunk_keys < 0 || opt->chunk_keys > kMaxChunk)
            return CSA_ERR_INVALID_ARG;
        row_offset = opt->row_offset;
        chunk = opt->chunk_keys;
    }
    // positions must stay representable: t + 1 fits comfortably in int64
    if (desc->S > (int64_t(1) << 40) || row_offset > (int64_t(1) << 40))
        return CSA_ERR_INVALID_ARG;
    // element counts must fit the 64-bit offsets used by the kernels
    const int64_t rows = desc->B * desc->S;
    if (desc->S > 0 && rows / desc->S != desc->B) return CSA_ERR_INVALID_ARG;
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
    p.grid = int(p.n_blocks < resident ? p.n_blocks : resident);
    p.chunk = chunk;
    p.log_cap = k + chunk;
    p.sort_pow2 = int(next_pow2(k));
    const size_t per_wave = size_t(p.QW) * size_t(p.log_cap) * 8u;  // u32 key + i32 index
    size_t ws = size_t(p.grid) * kWaves * per_wave;
    p.ws_bytes = (ws + 255) / 256 * 256;
    *plan = p;
    return CSA_OK;
}

}  // namespace csa
