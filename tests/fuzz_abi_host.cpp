// Host-only fuzz driver for the C ABI's planning and validation code
// (csa_plan.cpp, csa_abi.cpp), built with g++ under AddressSanitizer and
// UBSan by tests/test_abi_cpu.py.  The HIP runtime calls and the kernel
// launchers are stubbed here: no device is involved.  Every entry point is
// called with random, extreme and hostile sizes; the driver checks that
// nothing faults or hits undefined behaviour and that the plans it gets
// back are consistent.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "csa_group.hpp"
#include "csa_index.h"
#include "csa_kernels.hpp"

// ---- stubs: a device with 256 compute units that cannot allocate or launch
extern "C" hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int)
{
    *v = 256;
    return hipSuccess;
}
extern "C" hipError_t hipMallocAsync(void **p, size_t, hipStream_t)
{
    *p = nullptr;
    return hipErrorOutOfMemory;
}
extern "C" hipError_t hipFreeAsync(void *, hipStream_t) { return hipSuccess; }
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace csa {
static int g_launches = 0;
hipError_t launch_stream_topk(const Plan &, const StreamArgs &, hipStream_t)
{
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_merge_splits(const Plan &, const int32_t *, const float *, int32_t *, float *,
                               int, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_sort_rows(const Plan &, int32_t *, float *, int, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_sparse_attention(const AttnArgs &, int, int, hipStream_t)
{
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_stream_list(const StreamArgs &, int, hipStream_t)
{
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_stream_pooled(const StreamArgs &, int, hipStream_t)
{
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_pool_queries(const void *, const float *, void *, float *, int64_t, int64_t,
                               int, int, int, int, hipStream_t)
{
    ++g_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_build_lists(const int32_t *, int32_t *, int32_t *, int64_t, int64_t, int64_t,
                              int64_t, int, int, int, int, int, hipStream_t)
{
    return hipErrorInvalidValue;
}
}  // namespace csa

static void fail(const char *what, long i)
{
    std::fprintf(stderr, "fuzz: %s (case %ld)\n", what, i);
    std::exit(1);
}

int main(int argc, char **argv)
{
    const long cases = argc > 1 ? std::atol(argv[1]) : 200000;
    std::mt19937_64 rng(12345);
    const int64_t edge64[] = {0, 1, 2, 3, 63, 64, 65, 1000, 4095, 65536, 262144, 1 << 20,
                              int64_t(1) << 31, int64_t(1) << 40, INT64_MAX / 2, INT64_MAX, -1,
                              INT64_MIN};
    const int32_t edge32[] = {0, 1, 2, 3, 4, 8, 16, 31, 32, 33, 64, 100, 128, 256, 2048, 4096,
                              16384, 16385, 1 << 24, INT32_MAX, -1, INT32_MIN};
    auto pick64 = [&]() -> int64_t {
        return (rng() & 1) ? edge64[rng() % (sizeof(edge64) / 8)] : int64_t(rng() % 300000);
    };
    auto pick32 = [&]() -> int32_t {
        return (rng() & 1) ? edge32[rng() % (sizeof(edge32) / 4)] : int32_t(rng() % 5000);
    };
    void *p = reinterpret_cast<void *>(uintptr_t(4096));  // aligned, never dereferenced
    long ok_plans = 0, ok_attn = 0;
    for (long i = 0; i < cases; ++i) {
        // ---- indexer
        csa_desc d{};
        d.B = pick64();
        d.S = pick64();
        d.T = pick64();
        const int32_t Hs[] = {1, 4, 16, 64, 3, 0, 128, -4};
        const int32_t Ds[] = {32, 64, 128, 96, 0, 256};
        d.H = Hs[rng() % 8];
        d.D = Ds[rng() % 6];
        d.dtype = int32_t(rng() % 3);
        d.reserved0 = (rng() % 16 == 0) ? 1 : 0;
        d.q_scale = (rng() & 1) ? static_cast<const float *>(p) : nullptr;
        d.k_scale = (rng() & 1) ? static_cast<const float *>(p) : nullptr;
        csa_options o{};
        o.chunk_keys = pick32();
        o.num_cus = (rng() % 4 == 0) ? 0 : 1 + int32_t(rng() % 512);
        o.row_offset = pick64();
        o.key_splits = (rng() % 3 == 0) ? pick32() : 0;
        o.flags = int32_t(rng() % 16 == 0 ? 2 : rng() % 4 == 0 ? CSA_FLAG_NO_SCORE : 0);
        const int32_t tiles[] = {0, 0, 0, 64, 32, 128, 192, 256, 96, -64};
        o.key_tile = tiles[rng() % 10];
        o.reserved2 = (rng() % 32 == 0) ? 1 : 0;
        o.workspace = (rng() & 1) ? p : nullptr;
        o.workspace_bytes = size_t(rng() % (size_t(1) << 34));
        const int32_t m = pick32(), k = pick32();
        const csa_options *op = (rng() % 8 == 0) ? nullptr : &o;
        csa_plan_info info{};
        const int rc = csa_plan_query(&d, m, k, op, &info);
        const size_t ws = csa_workspace_bytes(&d, m, k, op);
        if (rc == CSA_OK) {
            ++ok_plans;
            if (ws != info.workspace_bytes) fail("workspace bytes differ from the plan", i);
            if (info.grid < 0 || info.key_splits < 1 || info.n_blocks < 0 || info.log_capacity < k)
                fail("implausible plan", i);
        } else if (rc > 0 || ws != 0) {
            fail("invalid arguments planned", i);
        }
        const int rx = csa_index_ex(p, static_cast<const float *>(p), p, &d, m, k,
                                    static_cast<int32_t *>(p), static_cast<float *>(p), op, nullptr);
        if (rc != CSA_OK && rx != rc) fail("csa_index_ex disagrees with the plan's status", i);

        // ---- grouped indexer (same arguments plus a group and a candidate count)
        csa_group_options go{};
        const int32_t gs[] = {8, 16, 64, 0, 7, 12, -8, 1 << 20};
        go.group = gs[rng() % 8];
        go.candidates = (rng() & 1) ? 0 : pick32();
        go.reserved[0] = (rng() % 32 == 0) ? 1 : 0;
        const size_t gws = csa_grouped_workspace_bytes(&d, m, k, &go, op);
        const int rg = csa_index_grouped(p, static_cast<const float *>(p), p, &d, m, k, &go,
                                         static_cast<int32_t *>(p), (rng() & 1) ? nullptr
                                         : static_cast<float *>(p), op, nullptr);
        if (gws == 0 && rg == CSA_OK && d.S > 0) fail("grouped call ran without a workspace", i);
        if (rc != CSA_OK && rg == CSA_OK) fail("grouped call accepted an invalid plan", i);

        // ---- sparse attention
        csa_attn_desc ad{};
        ad.B = pick64();
        ad.S = pick64();
        ad.T = pick64();
        const int32_t AH[] = {32, 64, 128, 16, 0};
        const int32_t AD[] = {64, 128, 32, 0};
        ad.H = AH[rng() % 5];
        ad.D = AD[rng() % 4];
        ad.n_sel = pick32();
        ad.reserved0 = (rng() % 16 == 0) ? 1 : 0;
        csa_attn_options ao{};
        ao.entry_splits = (rng() % 2) ? pick32() : 0;
        ao.num_cus = (rng() % 4 == 0) ? 0 : 1 + int32_t(rng() % 512);
        ao.workspace = (rng() & 1) ? p : nullptr;
        ao.workspace_bytes = size_t(rng() % (size_t(1) << 34));
        ao.reserved = (rng() % 16 == 0) ? 1 : 0;
        const csa_attn_options *aop = (rng() % 8 == 0) ? nullptr : &ao;
        int32_t G = -1;
        const size_t aws = csa_sparse_attention_workspace_bytes(&ad, aop, &G);
        const float scales[] = {0.f, 0.125f, -1.f, 1e30f, __builtin_nanf(""), __builtin_inff()};
        const float sc = scales[rng() % 6];
        const int ra = csa_sparse_attention_ex(p, p, p, static_cast<const int32_t *>(p), &ad, sc, p,
                                               static_cast<float *>(p), aop, nullptr);
        if (ra == CSA_OK) ++ok_attn;  // no rows: nothing launched
        if (G > 1 && aws == 0) fail("split without workspace bytes", i);
        if (aws > 0 && G < 2) fail("workspace without a split", i);
    }
    std::printf("fuzz ok: %ld cases, %ld valid indexer plans, %ld no-op attention calls, %d "
                "launch attempts reached\n",
                cases, ok_plans, ok_attn, csa::g_launches);
    return 0;
}
