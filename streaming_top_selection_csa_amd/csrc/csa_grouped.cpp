// csa_grouped.cpp -- csa_index_grouped: the approximate, query-group form of
// the indexer step (the shared prefix scan of the PIVOT news item,
// themodelwire: nearby query positions share one scan of the keys they all
// see, then each refines the shared result).
//
// For every group of g consecutive positions, on the caller's stream:
//   1. pool_queries_kernel: the group's pooled query (bf16 mean of the
//      members' q rows per head, fp32 mean of their weights);
//   2. the scoring kernel on the pooled queries over the keys visible to the
//      group's first member (every member sees them), keeping the top C;
//   3. build_lists_kernel: those C keys in ascending order, followed by the
//      keys that only later members see;
//   4. the scoring kernel over each group's list with every member's own
//      query: exact scores, each member's top-k among the list keys it sees,
//      sorted.
// A member's result is exact whenever its true top-k lies among the shared
// candidates and its own extra keys; the exact path (csa_index) is separate.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>

#include "csa_abi_internal.hpp"
#include "csa_group.hpp"
#include "csa_index.h"
#include "csa_kernels.hpp"
#include "csa_plan.hpp"

namespace {

constexpr int kListTile = 128;   // the re-rank kernel's staged key tile
constexpr int kMaxCandidates = 8192;  // the list kernel sorts them in 32 KB of LDS

struct GroupPlan {
    csa::Plan scan, rerank;
    int cus = 0;
    int64_t Sg = 0;
    int g = 0, C = 0, cap = 0;
    size_t off_qp = 0, off_wp = 0, off_cand = 0, off_lists = 0, off_lens = 0, off_ws = 0;
    size_t total = 0;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int plan_grouped(const csa_desc *desc, int32_t m, int32_t k, const csa_group_options *gopt,
                 const csa_options *opt, bool no_score, GroupPlan *gp)
{
    if (!desc || !gopt || gopt->reserved[0] != 0 || gopt->reserved[1] != 0)
        return CSA_ERR_INVALID_ARG;
    if (desc->dtype != CSA_BF16 || desc->H != 64 || desc->D != 128) {
        // validate the rest first: invalid sizes stay CSA_ERR_INVALID_ARG
        csa::Plan p;
        const int rc = csa::make_plan(desc, m, k, opt, 1, &p, no_score);
        return rc != CSA_OK ? rc : CSA_ERR_UNSUPPORTED;
    }
    const int g = gopt->group;
    if (g < 8 || g % 8 != 0 || g > (1 << 16)) return CSA_ERR_INVALID_ARG;
    if (k < 1) return CSA_ERR_INVALID_ARG;
    const int C = gopt->candidates ? gopt->candidates : std::min(2 * int64_t(k),
                                                                 int64_t(kMaxCandidates));
    if (C < k || C > kMaxCandidates) return CSA_ERR_INVALID_ARG;
    if (opt && ((opt->key_tile != 0 && opt->key_tile != kListTile) || opt->key_splits > 1 ||
                opt->chunk_keys < 0))
        return CSA_ERR_UNSUPPORTED;
    gp->g = g;
    gp->C = C;

    csa_options o{};
    if (opt) o = *opt;
    o.workspace = nullptr;
    o.workspace_bytes = 0;
    o.timing[0] = o.timing[1] = nullptr;
    // the re-rank (planned first: it validates the sizes): every row, one
    // key range, rows sorted in the kernel
    csa_options orr = o;
    orr.key_splits = 1;
    orr.key_tile = kListTile;
    orr.flags = no_score ? CSA_FLAG_NO_SCORE : 0;
    int rc = csa::plan_call(desc, m, k, &orr, &gp->rerank, &gp->cus, no_score, 1);
    if (rc != CSA_OK) return rc;
    if (gp->rerank.sort_e <= 0 || gp->rerank.n_splits != 1) return CSA_ERR_UNSUPPORTED;
    // the shared scan: pooled rows at every g-th position, no scores
    gp->Sg = (desc->S + g - 1) / g;
    csa_desc ds = *desc;
    ds.S = gp->Sg;
    csa_options os = o;
    os.key_tile = 0;
    os.flags = CSA_FLAG_NO_SCORE;
    rc = csa::plan_call(&ds, m, C, &os, &gp->scan, &gp->cus, true, g);
    if (rc != CSA_OK) return rc;

    const int64_t groups = desc->B * gp->Sg;
    gp->cap = int((int64_t(C) + (g - 1) / m + 1 + kListTile - 1) / kListTile * kListTile);
    size_t off = 0;
    gp->off_qp = off;
    off = align256(off + size_t(groups) * 64 * 128 * 2);
    gp->off_wp = off;
    off = align256(off + size_t(groups) * 64 * 4);
    gp->off_cand = off;
    off = align256(off + size_t(groups) * size_t(C) * 4);
    gp->off_lists = off;
    off = align256(off + size_t(groups) * size_t(gp->cap) * 4);
    gp->off_lens = off;
    off = align256(off + size_t(groups) * 4);
    gp->off_ws = off;
    gp->total = off + std::max(gp->scan.ws_bytes, gp->rerank.ws_bytes);
    return CSA_OK;
}

}  // namespace

extern "C" size_t csa_grouped_workspace_bytes(const csa_desc *desc, int32_t m, int32_t k,
                                              const csa_group_options *gopt,
                                              const csa_options *opt)
{
    GroupPlan gp;
    const bool no_score = opt && (opt->flags & CSA_FLAG_NO_SCORE);
    if (plan_grouped(desc, m, k, gopt, opt, no_score, &gp) != CSA_OK) return 0;
    return gp.total;
}

extern "C" int csa_index_grouped(const void *q, const float *w, const void *k_cmp,
                                 const csa_desc *desc, int32_t m, int32_t k,
                                 const csa_group_options *gopt, int32_t *out_idx,
                                 float *out_score, const csa_options *opt, hipStream_t stream)
{
    GroupPlan gp;
    int rc = plan_grouped(desc, m, k, gopt, opt, out_score == nullptr, &gp);
    if (rc != CSA_OK) return rc;
    const csa_desc &d = *desc;
    if (d.S == 0) return CSA_OK;
    if (!q || !w || !out_idx || (d.T > 0 && !k_cmp)) return CSA_ERR_INVALID_ARG;
    if (!csa::aligned(q, 16) || !csa::aligned(k_cmp, 16) || !csa::aligned(w, 4) ||
        !csa::aligned(out_idx, 4) || !csa::aligned(out_score, 4))
        return CSA_ERR_INVALID_ARG;

    void *ws = nullptr;
    bool owned = false;
    if (opt && opt->workspace) {
        if (opt->workspace_bytes < gp.total || !csa::aligned(opt->workspace, 256))
            return CSA_ERR_WORKSPACE;
        ws = opt->workspace;
    } else {
        if (hipMallocAsync(&ws, gp.total, stream) != hipSuccess) return CSA_ERR_HIP;
        owned = true;
    }
    unsigned char *base = static_cast<unsigned char *>(ws);
    void *qp = base + gp.off_qp;
    float *wp = reinterpret_cast<float *>(base + gp.off_wp);
    int32_t *cand = reinterpret_cast<int32_t *>(base + gp.off_cand);
    int32_t *lists = reinterpret_cast<int32_t *>(base + gp.off_lists);
    int32_t *lens = reinterpret_cast<int32_t *>(base + gp.off_lens);
    void *sws = base + gp.off_ws;

    if (opt && opt->timing[0] && hipEventRecord(opt->timing[0], stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    if (rc == CSA_OK &&
        csa::launch_pool_queries(q, w, qp, wp, d.B, d.S, d.H, d.D, gp.g, gp.cus, stream) !=
            hipSuccess)
        rc = CSA_ERR_HIP;
    if (rc == CSA_OK)
        rc = csa::run_index(gp.scan, gp.cus, qp, wp, k_cmp, nullptr, nullptr, cand, nullptr, sws,
                            nullptr, stream, nullptr);
    if (rc == CSA_OK &&
        csa::launch_build_lists(cand, lists, lens, d.B, d.S, d.T, gp.rerank.row_offset, m, gp.g,
                                gp.C, gp.cap, gp.cus, stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    const csa::ListArgs la{lists, lens, gp.Sg, gp.cap, gp.g};
    if (rc == CSA_OK)
        rc = csa::run_index(gp.rerank, gp.cus, q, w, k_cmp, nullptr, nullptr, out_idx, out_score,
                            sws, nullptr, stream, &la);
    if (rc == CSA_OK && opt && opt->timing[1] && hipEventRecord(opt->timing[1], stream) != hipSuccess)
        rc = CSA_ERR_HIP;
    if (owned && hipFreeAsync(ws, stream) != hipSuccess && rc == CSA_OK) rc = CSA_ERR_HIP;
    return rc;
}
