// csa_abi.cpp -- the extern "C" entry points declared in csa_index.h.
//
// Every call validates and plans on the host first (nothing touches the
// device on an invalid call), then enqueues, on the caller's stream: the
// scoring kernel (scores + running top-k per query position, or per key
// range; rows of up to 2,048 keys leave it sorted), the merge of the key
// ranges' lists when there are several, and the row sort when the kernel
// did not sort.  No host synchronisation, no host<->device copies.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "csa_abi_internal.hpp"
#include "csa_index.h"
#include "csa_kernels.hpp"
#include "csa_plan.hpp"

namespace csa {

int device_cus(int *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CSA_ERR_HIP;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return CSA_ERR_HIP;
    if (n <= 0) return CSA_ERR_HIP;
    *out = n;
    return CSA_OK;
}

}  // namespace csa

namespace {

using csa::device_cus;

int plan_for(const csa_desc *desc, int32_t m, int32_t k, const csa_options *opt,
             csa::Plan *p, int *cus, bool no_score = false)
{
    return csa::plan_call(desc, m, k, opt, p, cus, no_score, 1);
}

}  // namespace

namespace csa {

int plan_call(const csa_desc *desc, int32_t m, int32_t k, const csa_options *opt, Plan *p,
              int *cus, bool no_score, int64_t pos_mul)
{
    int num_cus = (opt && opt->num_cus > 0) ? opt->num_cus : 0;
    if (opt && opt->num_cus < 0) return CSA_ERR_INVALID_ARG;
    const int pre = make_plan(desc, m, k, opt, num_cus > 0 ? num_cus : 1, p, no_score, pos_mul);
    if (pre != CSA_OK) return pre;
    if (num_cus == 0) {
        const int rc = device_cus(&num_cus);
        if (rc != CSA_OK) return rc;
    }
    *cus = num_cus;
    return make_plan(desc, m, k, opt, num_cus, p, no_score, pos_mul);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace csa

namespace {

using csa::aligned;

// CSA_LOG set to anything but "" or "0": each call prints its plan to stderr.
bool log_plans()
{
    static const bool on = [] {
        const char *e = std::getenv("CSA_LOG");
        return e && *e && !(e[0] == '0' && e[1] == 0);
    }();
    return on;
}

void print_plan(const csa::Plan &p, int cus, bool caller_ws)
{
    std::fprintf(stderr,
                 "csa_index: B=%lld S=%lld T=%lld H=%d D=%d %s m=%d k=%d row_offset=%lld | "
                 "grid=%d of %d CUs, %lld blocks of %d positions, key tile %d, chunk %d "
                 "(log %d), key ranges %d of %d keys, rows sorted %s, scores %s, "
                 "workspace %zu bytes (%s)\n",
                 (long long)p.B, (long long)p.S, (long long)p.T, p.H, p.D, p.fp8 ? "fp8" : "bf16",
                 p.m, p.k, (long long)p.row_offset, p.grid, cus, (long long)p.n_blocks, p.QB,
                 p.key_tile, p.chunk, p.log_cap, p.n_splits, p.split_keys,
                 p.sort_e > 0 ? "in the scoring kernel" : "by a separate pass",
                 p.no_score ? "not returned" : "returned", p.ws_bytes,
                 caller_ws ? "caller" : "stream-ordered allocation");
}

}  // namespace

extern "C" const char *csa_status_string(int status)
{
    switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported dtype / head count / head dimension / k";
    case CSA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case CSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

extern "C" int csa_plan_query(const csa_desc *desc, int32_t m, int32_t k,
                              const csa_options *opt, csa_plan_info *out)
{
    if (!out) return CSA_ERR_INVALID_ARG;
    csa::Plan p;
    int cus = 0;
    const int rc = plan_for(desc, m, k, opt, &p, &cus);
    if (rc != CSA_OK) return rc;
    out->queries_per_block = p.QB;
    out->keys_per_tile = p.key_tile;
    out->chunk_keys = p.chunk;
    out->log_capacity = p.log_cap;
    out->grid = p.grid;
    out->key_splits = p.n_splits;
    out->n_blocks = p.n_blocks;
    out->workspace_bytes = p.ws_bytes;
    out->keys_per_range = p.n_splits > 1 ? p.split_keys : 0;
    out->reserved = 0;
    return CSA_OK;
}

extern "C" size_t csa_workspace_bytes(const csa_desc *desc, int32_t m, int32_t k,
                                      const csa_options *opt)
{
    csa::Plan p;
    int cus = 0;
    if (plan_for(desc, m, k, opt, &p, &cus) != CSA_OK) return 0;
    return p.ws_bytes;
}

namespace csa {

// Enqueues a planned call: the scoring kernel, the merge of the key ranges'
// lists and the row sort, as the plan asks.  ws holds p.ws_bytes bytes.
int run_index(const Plan &p, int cus, const void *q, const float *w, const void *k_cmp,
              const float *q_scale, const float *k_scale, int32_t *out_idx, float *out_score,
              void *ws, const hipEvent_t *timing, hipStream_t stream, const ListArgs *lists)
{
    StreamArgs a;
    a.q = static_cast<const unsigned char *>(q);
    a.w = w;
    a.k = static_cast<const unsigned char *>(k_cmp);
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.out_idx = out_idx;
    // without a score output, a separate row sort keeps the scores in the workspace
    float *const scores = out_score ? out_score
        : (p.sort_e == 0 && !p.merge_sorts
               ? reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + p.score_offset)
               : nullptr);
    a.out_score = scores;
    a.ws = static_cast<uint32_t *>(ws);
    // unsorted lists: the ranges' partial lists, or with one range the output
    // rows themselves (sorted afterwards by the row sort)
    unsigned char *part = static_cast<unsigned char *>(ws) + p.part_offset;
    a.part_idx = p.n_splits > 1 ? reinterpret_cast<int32_t *>(part) : out_idx;
    a.part_score = p.n_splits > 1
        ? reinterpret_cast<float *>(part + size_t(p.B * p.S) * size_t(p.n_splits) * size_t(p.k) * 4u)
        : scores;
    a.B = p.B;
    a.S = p.S;
    a.T = p.T;
    a.row_offset = p.row_offset;
    a.m = p.m;
    a.topk = p.k;
    a.log_cap = p.log_cap;
    a.n_splits = p.n_splits;
    a.split_keys = p.n_splits > 1 ? p.split_keys : int(kMaxKeys);
    a.blocks_per_batch = p.blocks_per_batch;
    a.n_units = p.n_units;
    a.sort_e = p.sort_e;
    a.key_tile = p.key_tile;
    a.pos_mul = p.pos_mul;
    a.klist = lists ? lists->klist : nullptr;
    a.klen = lists ? lists->klen : nullptr;
    a.n_lists = lists ? lists->n_lists : 0;
    a.list_cap = lists ? lists->list_cap : 0;
    a.list_rows = lists ? lists->list_rows : 0;

    int rc = CSA_OK;
    if (timing && timing[0] && hipEventRecord(timing[0], stream) != hipSuccess) rc = CSA_ERR_HIP;
    hipError_t e = hipSuccess;
    if (p.grid <= 0)
        e = hipSuccess;
    else if (lists)
        e = launch_stream_list(a, p.grid, stream);
    else if (p.pos_mul != 1)
        e = (p.fp8 || p.H != 64 || p.D != 128) ? hipErrorInvalidValue
                                               : launch_stream_pooled(a, p.grid, stream);
    else
        e = launch_stream_topk(p, a, stream);
    if (rc == CSA_OK && e != hipSuccess) rc = CSA_ERR_HIP;
    if (rc == CSA_OK && timing && timing[1] && hipEventRecord(timing[1], stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    if (rc == CSA_OK &&
        launch_merge_splits(p, a.part_idx, a.part_score, out_idx, scores, cus, stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    if (rc == CSA_OK && p.sort_e == 0 && !p.merge_sorts &&
        launch_sort_rows(p, out_idx, scores, cus, stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    return rc;
}

}  // namespace csa

extern "C" int csa_index_ex(const void *q, const float *w, const void *k_cmp,
                            const csa_desc *desc, int32_t m, int32_t k,
                            int32_t *out_idx, float *out_score,
                            const csa_options *opt, hipStream_t stream)
{
    csa::Plan p;
    int cus = 0;
    int rc = plan_for(desc, m, k, opt, &p, &cus, out_score == nullptr);
    if (rc != CSA_OK) return rc;
    const bool rows = p.B * p.S > 0;
    if (rows && (!q || !w || !out_idx)) return CSA_ERR_INVALID_ARG;
    if (p.T > 0 && !k_cmp) return CSA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_cmp, 16) || !aligned(w, 4) || !aligned(out_idx, 4) ||
        !aligned(out_score, 4) || !aligned(desc->q_scale, 4) || !aligned(desc->k_scale, 4))
        return CSA_ERR_INVALID_ARG;
    if (!rows) return CSA_OK;

    void *ws = nullptr;
    bool owned = false;
    if (opt && opt->workspace) {
        if (opt->workspace_bytes < p.ws_bytes || !aligned(opt->workspace, 256))
            return CSA_ERR_WORKSPACE;
        ws = opt->workspace;
    }
    if (log_plans()) print_plan(p, cus, ws != nullptr);
    if (!ws && p.ws_bytes > 0) {
        if (hipMallocAsync(&ws, p.ws_bytes, stream) != hipSuccess) return CSA_ERR_HIP;
        owned = true;
    }
    rc = csa::run_index(p, cus, q, w, k_cmp, desc->q_scale, desc->k_scale, out_idx, out_score, ws,
                        opt ? opt->timing : nullptr, stream, nullptr);
    if (owned && hipFreeAsync(ws, stream) != hipSuccess && rc == CSA_OK) rc = CSA_ERR_HIP;
    return rc;
}

extern "C" int csa_index(const void *q, const float *w, const void *k_cmp,
                         const csa_desc *desc, int32_t m, int32_t k,
                         int32_t *out_idx, float *out_score, hipStream_t stream)
{
    return csa_index_ex(q, w, k_cmp, desc, m, k, out_idx, out_score, nullptr, stream);
}

namespace {

struct AttnPlan {
    int64_t rows = 0;
    int splits = 1;
    int split_entries = 0;
    size_t ws_bytes = 0;
};

constexpr int kAttnTile = 32;         // entries per tile of the attention kernel
constexpr int kAttnMinRangeTiles = 16; // automatic ranges hold at least 512 entries
constexpr int kAttnUnitsPerCu = 4;    // workgroups per compute unit the split aims for

int attn_plan(const csa_attn_desc *desc, const csa_attn_options *opt, AttnPlan *p)
{
    if (!desc) return CSA_ERR_INVALID_ARG;
    const csa_attn_desc &d = *desc;
    if (d.B < 1 || d.S < 0 || d.T < 0 || d.n_sel < 0 || d.reserved0 != 0)
        return CSA_ERR_INVALID_ARG;
    // list positions (entry + tile padding) are 32-bit in the kernel
    if (d.n_sel > INT32_MAX - 64) return CSA_ERR_INVALID_ARG;
    if (!((d.H == 32 || d.H == 64 || d.H == 128) && (d.D == 64 || d.D == 128)))
        return CSA_ERR_UNSUPPORTED;
    // element counts must stay addressable with 64-bit byte offsets
    constexpr int64_t kMaxElems = int64_t(1) << 56;
    if (d.S > kMaxElems / d.B || d.T > kMaxElems / d.B) return CSA_ERR_INVALID_ARG;
    const int64_t rows = d.B * d.S;
    if (rows > kMaxElems / (int64_t(d.H) * d.D) || (d.n_sel > 0 && rows > kMaxElems / d.n_sel) ||
        d.B * d.T > kMaxElems / d.D)
        return CSA_ERR_INVALID_ARG;
    if (opt && (opt->entry_splits < 0 || opt->num_cus < 0 || opt->reserved != 0))
        return CSA_ERR_INVALID_ARG;
    p->rows = rows;
    p->splits = 1;
    p->split_entries = d.n_sel;
    p->ws_bytes = 0;
    const int tiles = (d.n_sel + kAttnTile - 1) / kAttnTile;
    const int req = opt ? opt->entry_splits : 1;
    if (rows == 0 || d.T == 0 || tiles <= 1 || req == 1) return CSA_OK;
    int G = 1;
    if (req > 1) {
        G = req < tiles ? req : tiles;
    } else {
        int cus = opt && opt->num_cus > 0 ? opt->num_cus : 0;
        if (cus == 0) {
            const int rc = device_cus(&cus);
            if (rc != CSA_OK) return rc;
        }
        const int64_t target = int64_t(kAttnUnitsPerCu) * cus;
        if (rows >= target) return CSA_OK;
        const int64_t want = (target + rows - 1) / rows;
        const int cap = tiles / kAttnMinRangeTiles > 1 ? tiles / kAttnMinRangeTiles : 1;
        G = want < cap ? int(want) : cap;
    }
    if (G <= 1) return CSA_OK;
    const int range_tiles = (tiles + G - 1) / G;
    G = (tiles + range_tiles - 1) / range_tiles;  // no empty trailing range
    if (G <= 1) return CSA_OK;
    if (double(rows) * G * d.H * (d.D + 2) * 4.0 > double(int64_t(1) << 56))
        return CSA_ERR_INVALID_ARG;  // partial results beyond any device
    p->splits = G;
    p->split_entries = range_tiles * kAttnTile;
    p->ws_bytes = size_t(rows) * size_t(G) * size_t(d.H) * size_t(d.D + 2) * 4u;
    return CSA_OK;
}

}  // namespace

extern "C" size_t csa_sparse_attention_workspace_bytes(const csa_attn_desc *desc,
                                                       const csa_attn_options *opt,
                                                       int32_t *entry_splits)
{
    AttnPlan p;
    if (attn_plan(desc, opt, &p) != CSA_OK) return 0;
    if (entry_splits) *entry_splits = p.splits;
    return p.ws_bytes;
}

extern "C" int csa_sparse_attention_ex(const void *q, const void *k, const void *v,
                                       const int32_t *idx, const csa_attn_desc *desc, float scale,
                                       void *out, float *lse, const csa_attn_options *opt,
                                       hipStream_t stream)
{
    AttnPlan p;
    int rc = attn_plan(desc, opt, &p);
    if (rc != CSA_OK) return rc;
    const csa_attn_desc &d = *desc;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return CSA_ERR_INVALID_ARG;
    if (p.rows == 0) return CSA_OK;
    if (!q || !out || (d.n_sel > 0 && !idx) || (d.T > 0 && (!k || !v)))
        return CSA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(idx, 4) || !aligned(lse, 4))
        return CSA_ERR_INVALID_ARG;

    void *ws = nullptr;
    bool owned = false;
    if (p.ws_bytes > 0) {
        if (opt && opt->workspace) {
            if (opt->workspace_bytes < p.ws_bytes || !aligned(opt->workspace, 256))
                return CSA_ERR_WORKSPACE;
            ws = opt->workspace;
        } else {
            if (hipMallocAsync(&ws, p.ws_bytes, stream) != hipSuccess) return CSA_ERR_HIP;
            owned = true;
        }
    }

    csa::AttnArgs a;
    a.q = static_cast<const unsigned char *>(q);
    a.k = static_cast<const unsigned char *>(k);
    a.v = static_cast<const unsigned char *>(v);
    a.idx = idx;
    a.out = static_cast<unsigned char *>(out);
    a.lse = lse;
    a.B = d.B;
    a.S = d.S;
    a.T = d.T;
    a.n_sel = d.n_sel;
    a.scale = scale;
    a.n_splits = p.splits;
    a.split_entries = p.split_entries;
    a.part_o = static_cast<float *>(ws);
    a.part_ml = p.ws_bytes > 0
        ? static_cast<float *>(ws) + size_t(p.rows) * size_t(p.splits) * size_t(d.H) * size_t(d.D)
        : nullptr;
    rc = csa::launch_sparse_attention(a, d.H, d.D, stream) == hipSuccess ? CSA_OK : CSA_ERR_HIP;
    if (owned && hipFreeAsync(ws, stream) != hipSuccess && rc == CSA_OK) rc = CSA_ERR_HIP;
    return rc;
}

extern "C" int csa_sparse_attention(const void *q, const void *k, const void *v,
                                    const int32_t *idx, const csa_attn_desc *desc, float scale,
                                    void *out, float *lse, hipStream_t stream)
{
    return csa_sparse_attention_ex(q, k, v, idx, desc, scale, out, lse, nullptr, stream);
}
