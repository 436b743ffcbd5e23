/*
 * csa_index.h -- C ABI of the MI355X (gfx950) CSA lightning-indexer top-k
 * and of the sparse attention over the keys it selects.
 *
 * Operation (StreamIndex: Memory-Bounded Compressed Sparse Attention via
 * Streaming Top-k, Abstract): each query position rates every compressed key
 * with the lightning indexer and keeps its k best keys; the [B, S, H_I, T]
 * tensor of per-head scores is never formed.  For query position t
 * (batch entry b) and compressed key s the score is
 *
 *     I(t, s) = sum_{j < H} w[b,t,j] * max(0, q[b,t,j,:] . k_cmp[b,s,:])
 *
 * and key s is visible to t iff (s+1)*m - 1 <= t, i.e. s < min(T, (t+1)/m).
 * For every t the library returns the min(k, n_vis) visible keys with the
 * largest scores, ordered by (score descending, key index ascending) -- ties
 * go to the lower key index -- followed by padding (index -1, score -inf).
 *
 * fp8 inputs (OCP E4M3, "fn" finite-only encoding; FP8 Formats for Deep
 * Learning) carry one positive fp32 scale per row: the dequantised operands
 * are q_scale[b,t,j] * q[b,t,j,:] and k_scale[b,s] * k_cmp[b,s,:].
 *
 * Arithmetic: products of bf16 / e4m3 operands are accumulated in fp32 by
 * the matrix cores; ReLU, the head weights and the head sum are applied in
 * fp32.  Integer-valued inputs whose partial sums stay below 2^24 are exact.
 *
 * Conventions for every entry point:
 *   - Device pointers are hipMalloc'd (or torch-allocated) device memory of
 *     the current device; the caller owns all of them.  The library keeps no
 *     pointer after a call returns and has no mutable global state.
 *   - All tensors are dense row-major (C order), innermost dimension last.
 *   - Calls are asynchronous on `stream`: inputs must stay alive, and outputs
 *     must not be read, until the stream reaches the work.
 *   - Every argument is validated before anything is launched; on any error
 *     nothing is written and a negative csa_status is returned.  No C++
 *     exception crosses this boundary.
 *   - Results are deterministic: bitwise identical across runs, chunk sizes,
 *     key splits and launch shapes (no floating-point atomics).
 *   - Diagnostics: with the environment variable CSA_LOG set (not "0"),
 *     every csa_index / csa_index_ex call prints its launch plan to stderr.
 */
#ifndef CSA_INDEX_H
#define CSA_INDEX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, k < 1, m < 1 ... */
    CSA_ERR_UNSUPPORTED = -2,  /* (dtype, H, D) combination not built       */
    CSA_ERR_WORKSPACE = -3,    /* caller workspace smaller than required     */
    CSA_ERR_HIP = -4           /* a HIP runtime call or a launch failed      */
} csa_status;

typedef enum {
    CSA_BF16 = 0,          /* q and k_cmp are bfloat16; no scales          */
    CSA_FP8_E4M3FN = 1     /* q and k_cmp are OCP e4m3fn with fp32 scales  */
} csa_dtype;

/*
 * Shapes and dtype of one call.
 *   q       [B, S, H, D]  dtype      (device)
 *   w       [B, S, H]     fp32       (device)
 *   k_cmp   [B, T, D]     dtype      (device)
 *   q_scale [B, S, H]     fp32 > 0   (device; fp8 only, NULL for bf16)
 *   k_scale [B, T]        fp32 > 0   (device; fp8 only, NULL for bf16)
 * Supported: H in {1, 2, 4, 8, 16, 32, 64}; D in {32, 64, 128} for bf16 and
 * {64, 128} for fp8; B >= 1, S >= 0, 0 <= T <= 2^30.  Other (dtype, H, D)
 * combinations return CSA_ERR_UNSUPPORTED, other sizes CSA_ERR_INVALID_ARG.
 */
typedef struct {
    int64_t B;
    int64_t S;
    int64_t T;
    int32_t H;
    int32_t D;
    int32_t dtype;          /* csa_dtype */
    int32_t reserved0;      /* must be 0 */
    const float *q_scale;
    const float *k_scale;
} csa_desc;

/*
 * Optional controls (NULL = all defaults).
 *   chunk_keys   Number of candidate keys a query may buffer beyond its
 *                running top-k before they are merged into it (the
 *                partition size of the partition-merge top-k; rounded up to a
 *                multiple of 64).  0 = default.  Affects speed and workspace
 *                only, never the result.
 *   row_offset   Absolute position of q row 0: q row i is position
 *                row_offset + i (a shard of a longer sequence, or a decode
 *                step).  Must be >= 0.
 *   num_cus      Compute units to plan for; 0 = ask the current device.
 *   workspace    Device scratch of workspace_bytes bytes (256-byte aligned);
 *                NULL = the library allocates it stream-ordered
 *                (hipMallocAsync / hipFreeAsync on `stream`).
 *   timing       Optional pair of hipEvent_t recorded on `stream` right before
 *                and right after the scoring kernel (for measurements).
 *   key_splits   Number of key ranges each query block is split into (the
 *                chunks of the partition-merge top-k taken in parallel): each
 *                range yields the exact top-k of its keys and a merge pass
 *                selects the top-k of the ranges' lists.  0 = automatic: 1
 *                while the query blocks fill the device, otherwise enough
 *                ranges of at least max(9k/8, 1024) keys to fill it (short query
 *                blocks, decode steps).  n >= 1 asks for n ranges (at most one
 *                per 64 visible keys).  The partial lists take B*S*G*k*8
 *                bytes of workspace: an automatic G is lowered to keep them
 *                under 1 GiB, a requested one under 64 GiB.  Affects speed
 *                and workspace only, never the result.
 *   flags        0, or CSA_FLAG_NO_SCORE: the call will pass out_score = NULL.
 *                Only csa_workspace_bytes and csa_plan_query read it (a call
 *                with out_score = NULL plans for that by itself); other bits
 *                must be 0.
 *   key_tile     Compressed keys staged in LDS per workgroup step (one
 *                barrier each); 0 = the default: 128 for bf16 with H = 64,
 *                D = 128; 256 for fp8 with H = 64, D = 128 and rows sorted
 *                by the scoring kernel (next_pow2(k) <= 2048, one key
 *                range); else 64.  64 works everywhere.  With rows sorted
 *                by the scoring kernel and H = 64, D = 128, also 32, 128,
 *                192 and 256 (bf16) and 128 and 256 (fp8); otherwise also
 *                128 for bf16 with H = 64, D = 128.  Other values return
 *                CSA_ERR_UNSUPPORTED.  Affects speed only, never the
 *                result.
 *   reserved2    Must be 0.
 */
typedef struct {
    int32_t chunk_keys;
    int32_t num_cus;
    int64_t row_offset;
    void *workspace;
    size_t workspace_bytes;
    hipEvent_t timing[2];
    int32_t key_splits;
    int32_t flags;
    int32_t key_tile;
    int32_t reserved2;
} csa_options;

/* csa_options.flags: size the workspace for calls without a score output. */
#define CSA_FLAG_NO_SCORE 1

/* What a call will do; filled by csa_plan_query (host only, no device work). */
typedef struct {
    int32_t queries_per_block;   /* query positions per workgroup block     */
    int32_t keys_per_tile;       /* compressed keys per staged key tile     */
    int32_t chunk_keys;          /* effective partition (candidate) size   */
    int32_t log_capacity;        /* per-query candidate buffer (entries)    */
    int32_t grid;                /* workgroups of the scoring kernel        */
    int32_t key_splits;          /* key ranges per query block (G >= 1)     */
    int64_t n_blocks;            /* query blocks over all batch entries     */
    size_t workspace_bytes;      /* device scratch needed                   */
    int32_t keys_per_range;      /* keys of each range (G > 1), else 0      */
    int32_t reserved;            /* 0                                       */
} csa_plan_info;

/*
 * csa_index: top-k compressed keys for every query position.
 *   out_idx   [B, S, k] int32 (device): key indices, -1 = padding.
 *   out_score [B, S, k] fp32  (device): scores, -inf = padding; NULL = the
 *             scores are not returned.  out_idx is identical either way.
 *             Rows of next_pow2(k) <= 2048 keys without key ranges are
 *             sorted inside the scoring kernel and need no score storage at
 *             all; otherwise a separate sort pass keeps the scores in the
 *             workspace (B*S*k*4 more bytes, see csa_workspace_bytes).
 * Uses default options (library-allocated workspace).  Returns CSA_OK or a
 * negative csa_status.
 */
int csa_index(const void *q, const float *w, const void *k_cmp,
              const csa_desc *desc, int32_t m, int32_t k,
              int32_t *out_idx, float *out_score, hipStream_t stream);

/* csa_index with explicit options (see csa_options). */
int csa_index_ex(const void *q, const float *w, const void *k_cmp,
                 const csa_desc *desc, int32_t m, int32_t k,
                 int32_t *out_idx, float *out_score,
                 const csa_options *opt, hipStream_t stream);

/* Device scratch bytes csa_index_ex needs for these arguments (0 on invalid
 * arguments).  With one key range (key_splits resolving to 1, always the
 * case when the query blocks fill the device) it is independent of S and T
 * and scales with the number of resident queries and k + chunk_keys only;
 * G > 1 key ranges add B*S*G*k*8 bytes for the partial lists.  With
 * CSA_FLAG_NO_SCORE in opt->flags it is the size for out_score = NULL,
 * which adds B*S*k*4 bytes only when the rows are sorted by a separate pass
 * (key ranges, or next_pow2(k) > 2048). */
size_t csa_workspace_bytes(const csa_desc *desc, int32_t m, int32_t k,
                           const csa_options *opt);

/*
 * csa_index_static: csa_index_ex without any allocation, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, hosts that forbid allocation).  Same arguments, results and errors
 * as csa_index_ex, except:
 *   - opt->workspace must be NULL and opt->workspace_bytes 0
 *     (CSA_ERR_INVALID_ARG otherwise): the scratch is a fixed array of
 *     CSA_STATIC_SCRATCH_BYTES bytes in device memory, one per GPU, held from
 *     the library's load until the process ends;
 *   - with chunk_keys = 0 the partition size is lowered (halved, down to 64)
 *     until the call's workspace fits that array; a call that still needs
 *     more returns CSA_ERR_WORKSPACE before anything is launched.
 * It makes no hipMalloc, hipFree or other allocating call.  Every call on a
 * GPU uses that GPU's one array (nothing in it needs to start cleared):
 * calls that may overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.
 */
#define CSA_STATIC_SCRATCH_BYTES (128u << 20)

int csa_index_static(const void *q, const float *w, const void *k_cmp,
                     const csa_desc *desc, int32_t m, int32_t k,
                     int32_t *out_idx, float *out_score,
                     const csa_options *opt, hipStream_t stream);

/* Host-only planning: validates the arguments and reports the launch plan.
 * Makes no HIP call when opt->num_cus > 0. */
int csa_plan_query(const csa_desc *desc, int32_t m, int32_t k,
                   const csa_options *opt, csa_plan_info *out);

/* Static, human-readable text for a csa_status value. */
const char *csa_status_string(int status);

/* ------------------------------------------------------------------------
 * Grouped indexer (approximate).
 *
 * The query-group shared scan of the PIVOT news item (themodelwire, "PIVOT
 * reduces sparse attention indexing bottleneck"): nearby query positions
 * share one scan of the keys they all see, and each then refines the shared
 * result.  The item gives no formula; this entry point computes, for every
 * group of g consecutive positions t0 .. t0+g-1 (q rows grouped from row 0;
 * the last group may be shorter):
 *   1. the pooled query: per head j, bf16(mean_t q[t,j,:]) (fp32 sum over the
 *      members in order, divided by their count, rounded to nearest even)
 *      and the fp32 mean of w[t,j];
 *   2. its indexer scores over the keys the first member sees,
 *      s < n_vis(t0), and the C best of them (csa_index's order and ties);
 *   3. for every member t: the exact score I(t, s) of each of those C keys
 *      and of every key n_vis(t0) <= s < n_vis(t), and the top-k of them
 *      exactly as csa_index orders and pads them.
 * A member's result equals csa_index's whenever its true top-k keys are
 * among those candidates; otherwise it is an approximation (its set recall
 * below 1).  csa_index itself is never affected.
 * ------------------------------------------------------------------------ */

typedef struct {
    int32_t group;         /* g: positions per group, a multiple of 8       */
    int32_t candidates;    /* C: keys the shared scan keeps, k <= C <= 8192;
                              0 = min(2k, 8192)                             */
    int32_t reserved[2];   /* must be 0                                     */
} csa_group_options;

/*
 * csa_index_grouped: csa_index's outputs (same shapes, order and padding;
 * out_score may be NULL) from the grouped computation above.  Built for
 * bf16 q and k_cmp with H = 64, D = 128 and next_pow2(k) <= 2048; other
 * shapes return CSA_ERR_UNSUPPORTED.  opt: row_offset, chunk_keys, num_cus,
 * workspace (csa_grouped_workspace_bytes bytes), timing (recorded around the
 * whole sequence) as for csa_index_ex; key_splits must be 0 or 1 and
 * key_tile 0 or 128.  Deterministic for a given g and C.
 */
int csa_index_grouped(const void *q, const float *w, const void *k_cmp,
                      const csa_desc *desc, int32_t m, int32_t k,
                      const csa_group_options *gopt, int32_t *out_idx, float *out_score,
                      const csa_options *opt, hipStream_t stream);

/* Device scratch bytes csa_index_grouped needs (0 on invalid arguments);
 * CSA_FLAG_NO_SCORE in opt->flags sizes it for out_score = NULL. */
size_t csa_grouped_workspace_bytes(const csa_desc *desc, int32_t m, int32_t k,
                                   const csa_group_options *gopt, const csa_options *opt);

/* ------------------------------------------------------------------------
 * Sparse attention over the selected keys.
 *
 * Operation (StreamIndex: Memory-Bounded Compressed Sparse Attention via
 * Streaming Top-k, Abstract: once the indexer has chosen each query's keys,
 * the attention kernel reads only those).  The page gives no formula; this
 * entry point computes plain softmax attention restricted to the chosen
 * compressed entries, with one key row and one value row per entry shared
 * by all query heads:
 *
 *     E(b,t)  = entries e of idx[b,t,:] with 0 <= idx[b,t,e] < T
 *     z_e     = scale * (q[b,t,h,:] . k[b, idx[b,t,e], :])
 *     out[b,t,h,:] = sum_{e in E} softmax(z)_e * v[b, idx[b,t,e], :]
 *     lse[b,t,h]   = log(sum_{e in E} exp(z_e))
 *
 * Entries outside [0, T) are padding (the indexer writes -1) and are never
 * read.  Each valid entry counts once.  A row with no valid entry gets
 * out = 0 and lse = -inf.  `idx` is typically csa_index's out_idx.
 *
 * Arithmetic: q.k products accumulate in fp32 on the matrix cores; the
 * softmax runs in fp32 with a running maximum; the weights are rounded to
 * bf16 for the weighted sum of v (fp32 accumulation); the normaliser is the
 * fp32 sum of the unrounded weights; out is rounded to bf16 once.
 * ------------------------------------------------------------------------ */

/*
 * Shapes of one sparse-attention call.
 *   q    [B, S, H, D]   bf16   (device)
 *   k    [B, T, D]      bf16   (device)
 *   v    [B, T, D]      bf16   (device)
 *   idx  [B, S, n_sel]  int32  (device)
 *   out  [B, S, H, D]   bf16   (device)
 *   lse  [B, S, H]      fp32   (device; may be NULL)
 * Supported: H in {32, 64, 128}, D in {64, 128}; B >= 1, S >= 0, T >= 0,
 * 0 <= n_sel <= 2^31 - 65.  Other H or D return CSA_ERR_UNSUPPORTED.  q, k, v and out
 * must be 16-byte aligned, idx and lse 4-byte aligned.
 */
typedef struct {
    int64_t B;
    int64_t S;
    int64_t T;
    int32_t H;
    int32_t D;
    int32_t n_sel;          /* index entries per query row (csa_index's k) */
    int32_t reserved0;      /* must be 0 */
} csa_attn_desc;

/*
 * csa_sparse_attention: softmax attention of every query row over the
 * entries its index list selects (see above).  `scale` multiplies q.k (for
 * example 1/sqrt(D)) and must be finite.  Writes only out and lse.  No
 * device memory is allocated and rows are never split (entry_splits = 1).
 * Deterministic: bitwise identical across runs.
 * Returns CSA_OK or a negative csa_status; on error nothing is launched.
 */
int csa_sparse_attention(const void *q, const void *k, const void *v,
                         const int32_t *idx, const csa_attn_desc *desc,
                         float scale, void *out, float *lse, hipStream_t stream);

/*
 * Optional controls of csa_sparse_attention_ex (NULL = all defaults).
 *   entry_splits  Ranges each row's index list is split into, each handled by
 *                 its own workgroup, with a combine pass after (for short
 *                 query blocks such as a decode step, where rows alone leave
 *                 the device idle).  0 = automatic: 1 while B*S rows reach
 *                 four workgroups per compute unit, otherwise enough ranges
 *                 of at least 512 entries to get there.  1 = no split (the
 *                 plain csa_sparse_attention).  n > 1 asks for n ranges (at
 *                 most one per 32 entries).  Ranges change rounding only:
 *                 results stay within the documented bound, and are
 *                 deterministic for a given count.
 *   num_cus       Compute units to plan for; 0 = ask the current device.
 *   workspace     Device scratch of workspace_bytes bytes (256-byte aligned)
 *                 for the ranges' partial results, B*S*G*H*(D+2)*4 bytes;
 *                 NULL = the library allocates it stream-ordered
 *                 (hipMallocAsync / hipFreeAsync on `stream`) when G > 1.
 *   reserved      Must be 0.
 */
typedef struct {
    int32_t entry_splits;
    int32_t num_cus;
    void *workspace;
    size_t workspace_bytes;
    int64_t reserved;
} csa_attn_options;

/* csa_sparse_attention with explicit options (see csa_attn_options). */
int csa_sparse_attention_ex(const void *q, const void *k, const void *v,
                            const int32_t *idx, const csa_attn_desc *desc,
                            float scale, void *out, float *lse,
                            const csa_attn_options *opt, hipStream_t stream);

/* Device scratch bytes csa_sparse_attention_ex needs for these arguments
 * (0 when the rows are not split, and on invalid arguments).  The split
 * count it implies is written to *entry_splits when that is not NULL. */
size_t csa_sparse_attention_workspace_bytes(const csa_attn_desc *desc,
                                            const csa_attn_options *opt,
                                            int32_t *entry_splits);

#ifdef __cplusplus
}
#endif

#endif /* CSA_INDEX_H */
