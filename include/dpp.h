/*
 * dpp.h -- C ABI of libdpp: batch-invariant causal GQA prefill attention over a paged KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation (paged causal prefill attention, sglang PR #46351 page, "Motivation"; causal
 * placement from the same page, "Fix" section and the author's reply on tail alignment): for
 * request r with qo_len query tokens and kv_len cached-plus-new tokens, query row i of q head h
 * attends to keys 0..p of kv head h / (num_qo_heads / num_kv_heads), where
 * p = kv_len - qo_len + i, and returns
 *
 *     o[i, h, :]  = softmax_j( sm_scale * <q[i, h, :], k[j, :]> ) @ v[j, :]      (bf16)
 *     lse[i, h]   = log sum_j exp( sm_scale * <q[i, h, :], k[j, :]> )            (fp32, natural log)
 *
 * Batch invariance is the contract: the bits of a row depend only on its own query, keys
 * 0..p and the configuration below -- never on the other requests in the batch, on qo_len
 * (a prefix-cache hit that sends only the uncached tail returns exactly the rows of the full
 * prefill), on page placement, or on the workspace cap. The sglang PR #46351 page ("Root
 * cause") traces the failure of this contract in FlashInfer to a q-tile size chosen from the
 * batch's average query length; here every tile size, KV chunk and reduction order is a
 * constant of (num_qo_heads, num_kv_heads, head_dim).
 *
 * Long rows are cut into fixed KV splits of 4096 tokens at absolute positions 0, 4096, ...
 * (model-serving-minefield issue #73, correction comment, "What the flag actually does",
 * item 2). Each split's partial state goes to a caller-owned workspace whose size the plan
 * bounds (that page's "The failure" section describes the unbounded version killing a
 * server); a merge kernel then combines a row's partials in ascending split order.
 *
 * Memory layout (all device buffers are caller-owned; the library never allocates or frees
 * device memory and never synchronises a stream):
 *   q          [qo_indptr[B], num_qo_heads, head_dim]            bf16, contiguous
 *   k_pool     [num_pages, page_size, num_kv_heads, head_dim]     bf16 or fp8 E4M3 (OCP), contiguous
 *   v_pool     same as k_pool
 *   kv_indices [kv_indptr[B]] int32 page ids; request r owns kv_indices[kv_indptr[r] .. kv_indptr[r+1])
 *   o          [qo_indptr[B], num_qo_heads, head_dim]             bf16
 *   lse        [qo_indptr[B], num_qo_heads]                       fp32 (natural log)
 * Request r's KV is kv_len = (pages - 1) * page_size + kv_last_page_len[r] tokens (0 if it
 * owns no pages); token j lives in page kv_indices[kv_indptr[r] + j / page_size], slot
 * j % page_size. Slots past a request's kv_len are never read.
 *
 * Ragged (contiguous) KV, page_size == 0 in the config (the non-paged prefill the sglang PR
 * #46351 page names beside the paged one, "Motivation"): k_pool and v_pool are
 * [total_tokens, num_kv_heads, head_dim]; kv_indptr counts tokens, request r's keys are rows
 * kv_indptr[r] .. kv_indptr[r+1]-1; kv_last_page_len and kv_indices are ignored (may be
 * NULL); num_pages in dpp_run is total_tokens. Same kernels, same arithmetic: a row's bits are
 * those of the same row over a paged layout.
 *
 * Errors: every entry point returns a dpp_status and, on failure, records a message that
 * dpp_last_error() returns (thread-local). Nothing aborts, exits or throws across the ABI.
 */
#ifndef DPP_H
#define DPP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DPP_OK = 0,
  DPP_ERR_INVALID = 1,     /* null pointer, negative count, non-monotone or non-zero-based indptr */
  DPP_ERR_SHAPE = 2,       /* qo_len > kv_len, last-page length outside [1, page_size], q row
                              count != qo_indptr[B] (the check sglang PR #46351 reports as a
                              ValueError from FlashInfer's paged prefill) */
  DPP_ERR_UNSUPPORTED = 3, /* head_dim, page_size, head counts or kv dtype not built */
  DPP_ERR_WORKSPACE = 4,   /* workspace smaller than the plan needs, misaligned, or a cap too
                              small for one q tile's partials; reported before any launch */
  DPP_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} dpp_status;

typedef enum { DPP_KV_BF16 = 0, DPP_KV_FP8_E4M3 = 1 } dpp_kv_dtype;

/* Model-level constants. These, and only these, fix the arithmetic of every row. */
typedef struct {
  int32_t num_qo_heads;  /* Hq, a multiple of num_kv_heads, at most 1024 x it */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* 64, 128, 256 or 512 */
  int32_t page_size;     /* tokens per page, 1..1024; 0 = ragged (contiguous) KV */
  int32_t kv_dtype;      /* dpp_kv_dtype */
  float sm_scale;        /* softmax scale; 0 selects 1/sqrt(head_dim) */
  float k_scale;         /* fp8 dequantisation multipliers (value = decode(code) * scale);
                            ignored for bf16. Powers of two make the bf16 staging exact. */
  float v_scale;
} dpp_config;

/* Opaque host-side plan: the work list of one batch shape. Created from host copies of the
 * index arrays, reusable for every layer that runs on that batch. */
typedef struct dpp_plan dpp_plan;

/* Read-only facts about a plan (for tests and reporting). */
typedef struct {
  int32_t block_m;            /* packed query rows (token x q head of a group) per tile */
  int32_t block_n;            /* keys per KV tile, tiles start at multiples of block_n */
  int32_t split_tokens;       /* fixed KV split length (4096) */
  int32_t num_passes;         /* launches of (prefill, merge) needed under the cap */
  int64_t num_prefill_items;  /* (q tile, split) work items, all passes, per kv head */
  int64_t num_merge_items;    /* q tiles needing a merge, all passes, per kv head */
  int64_t max_partial_slots;  /* partial rows of the largest pass (each (head_dim+1)*4 bytes) */
  size_t header_bytes;        /* work list uploaded at the head of the workspace */
  size_t workspace_bytes;     /* what dpp_run needs */
  int64_t total_q_rows;       /* qo_indptr[B] */
} dpp_plan_info;

/*
 * Build the plan of one batch. Host only: no HIP call, no device memory.
 *
 * Defining passages: a paged prefill wrapper planned on the host from the batch's index
 * arrays, probed cold and on a radix hit (sglang PR #46351 page, "Validation"; its host-plan
 * test suite under "Tests"); what the plan may not do is size its q tile from the batch
 * ("Root cause"); its fixed 4096-token KV splits and the bounded
 * partial buffer they need come from the model-serving-minefield issue #73 correction comment
 * ("What the flag actually does", item 2, and "The failure").
 *
 *   cfg                  model constants (copied)
 *   batch_size           B >= 0
 *   qo_indptr_host       [B+1] int32, qo_indptr[0] == 0, non-decreasing
 *   kv_indptr_host       [B+1] int32, kv_indptr[0] == 0, non-decreasing (page counts; token
 *                        counts for ragged KV, where a request's K may not exceed 2 GiB)
 *   kv_last_page_len_host[B]  int32, in [1, page_size] for every request with pages (ignored,
 *                        and may be NULL, for ragged KV)
 *   workspace_cap_bytes  upper bound on dpp_plan_workspace_bytes(); 0 = no bound. Rows whose
 *                        partials do not fit are run in further passes; the cap changes the
 *                        number of launches, never a bit of the result.
 *   out_plan             receives the plan (NULL on failure); free with dpp_plan_destroy
 *
 * Errors: DPP_ERR_INVALID (null pointers, bad indptr), DPP_ERR_SHAPE (qo_len > kv_len, last
 * page length out of range), DPP_ERR_UNSUPPORTED (config), DPP_ERR_WORKSPACE (cap below the
 * smallest pass).
 */
dpp_status dpp_plan_create(const dpp_config* cfg, int32_t batch_size,
                           const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                           const int32_t* kv_last_page_len_host, size_t workspace_cap_bytes,
                           dpp_plan** out_plan);

/* dpp_plan_create_ex flags */
#define DPP_PLAN_ADAPTIVE_KV_TILE 1u
/* Test mode: shuffle the order of the work inside every pass (items, merges, and hence the
 * workgroup and persistent chain each unit lands in) with the seed in bits 16..31 of the
 * flags. Results must not change by a bit: the pages find the reduction order batch
 * invariant once the tile is fixed (sglang PR #46351 page, "Root cause"). */
#define DPP_PLAN_PERMUTE_WORK 2u
#define DPP_PLAN_PERMUTE_SEED(seed) (((uint32_t)(seed) & 0xFFFFu) << 16)

/*
 * dpp_plan_create with plan flags (0: identical to dpp_plan_create). DPP_PLAN_ADAPTIVE_KV_TILE
 * is a comparison mode that gives up batch invariance on purpose: like FlashInfer's tile rule
 * (the sglang PR #46351 page, "Root cause" and the author's A100 findings: a 16-row q tile when
 * the batch's average packed query length sum(qo_len * group) / batch_size is at most 16), a
 * batch whose tiles all have at most 16 packed rows and whose average is at most 16 runs with
 * 32-key KV tiles at head_dim 128 (bf16) instead of 64. Such a batch's rows then differ in
 * their last bits from the same rows planned in a larger batch; it exists to measure that
 * difference and what the fixed tile costs. dpp_plan_info.block_n reports the tile used.
 * DPP_PLAN_PERMUTE_WORK (with DPP_PLAN_PERMUTE_SEED) only reorders work; a test compares its
 * results with the default plan's bit for bit.
 * Errors: those of dpp_plan_create, and DPP_ERR_INVALID for unknown flag bits.
 */
dpp_status dpp_plan_create_ex(const dpp_config* cfg, int32_t batch_size,
                              const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                              const int32_t* kv_last_page_len_host, size_t workspace_cap_bytes,
                              uint32_t plan_flags, dpp_plan** out_plan);

/* Bytes of device workspace dpp_run needs for this plan (256-byte aligned buffer). */
size_t dpp_plan_workspace_bytes(const dpp_plan* plan);

/* Fill *info. DPP_ERR_INVALID on null arguments. */
dpp_status dpp_plan_get_info(const dpp_plan* plan, dpp_plan_info* info);

/* The work list exactly as dpp_run uploads it (host memory owned by the plan, valid until
 * dpp_plan_destroy). Layout: int32 words; see the planner source for the record format. */
dpp_status dpp_plan_header(const dpp_plan* plan, const void** data, size_t* bytes);

/*
 * Enqueue the copy of the plan's work list into the head of `workspace` on `stream`.
 * dpp_run does this itself unless called with DPP_RUN_REUSE_UPLOAD; a caller that runs the
 * same plan many times (every layer of a model on one batch) uploads once and passes the flag.
 * The plan's id is stamped into the copy; kernels launched for another plan, or over a
 * workspace whose head was overwritten, find a different id and write nothing.
 * Errors: DPP_ERR_INVALID (null), DPP_ERR_WORKSPACE (size / alignment), DPP_ERR_HIP.
 */
dpp_status dpp_plan_upload(const dpp_plan* plan, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Free a plan. The plan must outlive the stream work of every dpp_run that used it (the
 * upload of its work list reads the plan's pinned host buffer asynchronously). NULL is a no-op. */
void dpp_plan_destroy(dpp_plan* plan);

/* dpp_run flags */
#define DPP_RUN_REUSE_UPLOAD 1u /* the workspace already holds this plan's work list */

/*
 * Run the planned attention on `stream` (a hipStream_t; NULL = the null stream).
 *
 * Defining passages: the operation at the top of this header (sglang PR #46351 page,
 * "Motivation" and "Fix"); the shape check that q holds qo_indptr[-1] rows is the one that
 * page's Woody-Hu report shows FlashInfer raising as a ValueError; a workspace too small for
 * the plan is refused before any launch, the opposite of the overflow in the
 * model-serving-minefield issue #73 correction comment ("The failure").
 *
 *   q, k_pool, v_pool, kv_indices, o, lse   device pointers, layouts above
 *   q_rows        rows of q and o; must equal qo_indptr[B] of the plan (DPP_ERR_SHAPE)
 *   num_pages     pages in each pool. Page ids are the caller's contract: every id a request
 *                 reads must lie in [0, num_pages) (dpp_check_page_table checks a host copy);
 *                 the kernels never read outside the pools, and an id outside that range
 *                 reads as zeros. Ragged KV: the token rows of k_pool / v_pool; kv_indptr[B]
 *                 above it is DPP_ERR_SHAPE, and kv_indices may be NULL
 *   num_kv_indices  entries of kv_indices; below kv_indptr[B] of the plan is DPP_ERR_SHAPE
 *                 (ignored for ragged KV)
 *   workspace     device buffer of at least dpp_plan_workspace_bytes(plan) bytes, 256-byte
 *                 aligned; its contents are scratch (work list + split partials)
 *   flags         0, or DPP_RUN_REUSE_UPLOAD when dpp_plan_upload (or an earlier dpp_run) has
 *                 already put this plan's work list into this workspace on this stream. The
 *                 plan remembers the workspace of its last upload: reusing an upload with any
 *                 other workspace (or with none made) is DPP_ERR_INVALID. Writing over the
 *                 head of the workspace between the upload and the run is the caller's fault:
 *                 the kernels then find no work list of this plan and write nothing
 *
 * Enqueues: the async copy of the work list into the workspace (unless reused), then per pass
 * one prefill launch and (if some row spans several splits) one merge launch. Returns without
 * waiting.
 * On DPP_ERR_INVALID / DPP_ERR_SHAPE / DPP_ERR_WORKSPACE / DPP_ERR_UNSUPPORTED nothing is
 * enqueued.
 */
dpp_status dpp_run(const dpp_plan* plan, const void* q, int64_t q_rows, const void* k_pool,
                   const void* v_pool, int64_t num_pages, const int32_t* kv_indices,
                   int64_t num_kv_indices, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, uint32_t flags, void* stream);

/* Size of the scratch array dpp_run_static uses in place of a workspace (32 MiB per device). */
#define DPP_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * dpp_run without a workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It calls no
 * hipMalloc, hipFree or other allocating routine. The work list and the split partials live
 * in a file-scope device array of DPP_STATIC_SCRATCH_BYTES, one per device, held by the
 * library until the process ends; the caller still passes q, the pools, the page list and the
 * outputs, with dpp_run's layouts, checks and bits.
 *
 *   flags   0 (upload the plan's work list into the device's scratch, from the plan's pinned
 *           copy if an earlier dpp_run made one, else from its host memory), or
 *           DPP_RUN_REUSE_UPLOAD when the last dpp_run_static on this device uploaded this
 *           same plan (otherwise DPP_ERR_INVALID)
 *
 * A plan whose workspace exceeds DPP_STATIC_SCRATCH_BYTES is DPP_ERR_WORKSPACE before any HIP
 * call: plan with workspace_cap_bytes <= DPP_STATIC_SCRATCH_BYTES, which bounds every plan by
 * running more passes. Every call on one device shares that device's scratch and leaves its
 * contents behind: calls that overlap on one GPU (other streams, other threads) race, and
 * must be ordered by the caller. Other errors as dpp_run.
 */
dpp_status dpp_run_static(const dpp_plan* plan, const void* q, int64_t q_rows, const void* k_pool,
                          const void* v_pool, int64_t num_pages, const int32_t* kv_indices,
                          int64_t num_kv_indices, void* o, float* lse, uint32_t flags,
                          void* stream);

/*
 * Read-only streaming reference of a plan's KV gather (a measurement tool, not part of the
 * attention): every K and V byte the plan's prefill units read, each once, is moved into LDS
 * by LDS-DMA and dropped, by `split` workgroups per unit (item, kv head) with `depth` (4, 8, 16
 * or 32) 1 KiB loads in flight per wave. The workgroups of a unit divide its keys; with
 * DPP_STREAM_HEAD_SPLIT (split 2 only) both read all of its K and each one half of every V row,
 * as the head_dim-split attention launch does. Its time is the ceiling the memory-bound
 * launches of the same plan (short extends, long-KV decodes) are measured against. Arguments as
 * dpp_run; paged plans only; flags: DPP_RUN_REUSE_UPLOAD (the workspace already holds this
 * plan's work list) and DPP_STREAM_HEAD_SPLIT. Writes only the workspace head.
 */
#define DPP_STREAM_HEAD_SPLIT 2u

dpp_status dpp_stream_kv(const dpp_plan* plan, const void* k_pool, const void* v_pool,
                         int64_t num_pages, const int32_t* kv_indices, int64_t num_kv_indices,
                         void* workspace, size_t workspace_bytes, int32_t split, int32_t depth,
                         uint32_t flags, void* stream);

/*
 * Host check of a page table against a plan: kv_indices_host holds at least kv_indptr[B]
 * entries and every page id that a request of the plan reads lies in [0, num_pages).
 * DPP_ERR_SHAPE names the first offending (request, page); DPP_ERR_INVALID on null or
 * negative arguments. A ragged plan has no page table: DPP_OK. Host only, no HIP call.
 */
dpp_status dpp_check_page_table(const dpp_plan* plan, const int32_t* kv_indices_host,
                                int64_t num_kv_indices, int64_t num_pages);

/*
 * Combine softmax partial states, the same device merge dpp_run uses for split rows.
 *
 * Defining passage: the fixed KV splits whose partial (o, lse) states are combined afterwards
 * (model-serving-minefield issue #73, correction comment, "What the flag actually does",
 * item 2); the combination is the log-sum-exp identity, taken in ascending split order.
 *
 *   o_partial   [num_rows, num_splits, num_heads, head_dim] fp32 device
 *   lse_partial [num_rows, num_splits, num_heads] fp32 device, natural log; -inf marks an
 *               empty partial (weight 0)
 *   o           [num_rows, num_heads, head_dim] bf16 device out
 *   lse         [num_rows, num_heads] fp32 device out (natural log)
 * Partials are combined in ascending split order with weights exp(lse_s - max_s lse_s).
 * A row whose partials are all empty gets o = 0, lse = -inf.
 * head_dim must be a multiple of 4 and at most 1024; num_splits in [1, 1024].
 */
dpp_status dpp_merge_states(const float* o_partial, const float* lse_partial, int64_t num_rows,
                            int32_t num_splits, int32_t num_heads, int32_t head_dim, void* o,
                            float* lse, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* dpp_last_error(void);

/* Name of a status code. */
const char* dpp_status_string(dpp_status status);

/* ABI version of the library (bumped when a signature or record format changes). */
int32_t dpp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DPP_H */
