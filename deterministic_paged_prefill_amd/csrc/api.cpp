// Launch glue of libdpp: argument checks, work-list upload, kernel launches.
//
// Nothing here allocates or frees device memory or synchronises a stream. The only HIP
// allocation is the pinned host staging copy of a plan's work list (made on its first upload,
// so that planning itself stays HIP-free), taken from a library-wide pool of pinned blocks
// that destroyed plans return to: a serving loop that plans every batch reuses them instead
// of allocating pinned memory per batch.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstring>
#include <map>
#include <cmath>
#include <string>

#include "kernels.h"
#include "plan.h"

using namespace dpp;

namespace {

dpp_status hip_fail(hipError_t e, const char* what) {
  return fail(DPP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Pool of pinned staging blocks, sizes rounded up to powers of two (64 KiB and up). A block
// goes back to the pool when its plan is destroyed -- after the stream work that read it, which
// the plan's lifetime contract guarantees -- and the pool keeps at most kPinnedPoolBytes.
constexpr size_t kPinnedMinBytes = 64 << 10;
constexpr size_t kPinnedPoolBytes = 64 << 20;
std::mutex g_pool_mu;
std::multimap<size_t, void*> g_pool;
size_t g_pool_bytes = 0;

size_t pinned_class(size_t bytes) {
  size_t c = kPinnedMinBytes;
  while (c < bytes) c <<= 1;
  return c;
}

hipError_t pinned_get(size_t bytes, void** out, size_t* cap) {
  const size_t c = pinned_class(bytes);
  {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    auto it = g_pool.find(c);
    if (it != g_pool.end()) {
      *out = it->second;
      *cap = c;
      g_pool_bytes -= c;
      g_pool.erase(it);
      return hipSuccess;
    }
  }
  *cap = c;
  return hipHostMalloc(out, c, hipHostMallocDefault);
}

void pinned_put(void* p, size_t cap) {
  {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (g_pool_bytes + cap <= kPinnedPoolBytes) {
      g_pool.emplace(cap, p);
      g_pool_bytes += cap;
      return;
    }
  }
  (void)hipHostFree(p);
}

}  // namespace


extern "C" void dpp_plan_destroy(dpp_plan* plan) {
  if (!plan) return;
  if (plan->pinned) pinned_put(plan->pinned, plan->pinned_cap);
  delete plan;
}

namespace {

dpp_status check_workspace(const dpp_plan* plan, const void* workspace, size_t workspace_bytes) {
  if (!workspace) return fail(DPP_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(DPP_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(DPP_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " B, the plan needs " + std::to_string(plan->workspace_bytes) + " B");
  return DPP_OK;
}

dpp_status enqueue_upload(const dpp_plan* plan, void* workspace, hipStream_t stream) {
  const size_t hbytes = plan->header.size() * sizeof(int32_t);
  {
    std::lock_guard<std::mutex> lock(plan->pinned_mu);
    if (!plan->pinned) {
      void* p = nullptr;
      size_t cap = 0;
      hipError_t e = pinned_get(hbytes, &p, &cap);
      if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(work list)");
      std::memcpy(p, plan->header.data(), hbytes);
      plan->pinned = p;
      plan->pinned_cap = cap;
    }
  }
  hipError_t e = hipMemcpyAsync(workspace, plan->pinned, hbytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
  std::lock_guard<std::mutex> lock(plan->pinned_mu);
  plan->uploaded_ws = workspace;
  return DPP_OK;
}

// A run that reuses an upload must name the workspace that upload went to: otherwise the
// kernels would find another plan's work list (or none) and write nothing.
dpp_status check_reuse(const dpp_plan* plan, const void* workspace) {
  std::lock_guard<std::mutex> lock(plan->pinned_mu);
  if (plan->uploaded_ws != workspace)
    return fail(DPP_ERR_INVALID, plan->uploaded_ws ? "DPP_RUN_REUSE_UPLOAD: this plan's work list was uploaded to "
                                                     "another workspace"
                                                   : "DPP_RUN_REUSE_UPLOAD: this plan was never uploaded");
  return DPP_OK;
}

}  // namespace

extern "C" dpp_status dpp_plan_upload(const dpp_plan* plan, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!plan) return fail(DPP_ERR_INVALID, "dpp_plan_upload: null plan");
  dpp_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != DPP_OK) return st;
  return enqueue_upload(plan, workspace, (hipStream_t)stream);
}

namespace dpp {

dpp_status launch_passes(const dpp_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                         int64_t num_pages, const int32_t* kv_indices, void* o, float* lse, void* workspace,
                         void* stream_ptr) {
  hipStream_t stream = (hipStream_t)stream_ptr;
  hipError_t e;
  char* ws = (char*)workspace;
  PrefillArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  // ragged: every unit's one page id (0) comes from the work list's zero chunk
  a.kv_indices = plan->ragged ? (const int32_t*)workspace + offsetof(HeaderPreamble, zero_chunk) / 4 : kv_indices;
  a.ragged = plan->ragged ? 1 : 0;
  a.o = o;
  a.lse = lse;
  a.header = (const int32_t*)workspace;
  a.part_o = (float*)(ws + plan->partial_o_offset);
  a.part_lse2 = (float*)(ws + plan->partial_lse_offset);
  a.num_pages = num_pages;
  a.plan_id = plan->plan_id;
  a.num_qo_heads = plan->cfg.num_qo_heads;
  a.num_kv_heads = plan->cfg.num_kv_heads;
  a.group = plan->group;
  a.page_size = plan->ragged ? kRaggedPage : plan->cfg.page_size;
  a.page_slots = plan->page_slots;
  a.item_offset = plan->item_offset;
  a.scale_log2 = plan->scale_log2;
  a.k_scale = plan->cfg.k_scale;
  a.v_scale = plan->cfg.v_scale;
  auto pow2_in_range = [](float x) {
    int e = 0;
    const float m = std::frexp(x, &e);  // x = m 2^e, m in [0.5, 1)
    return m == 0.5f && e - 1 >= -64 && e - 1 <= 64;
  };
  a.kv_scale_pow2 = pow2_in_range(a.k_scale) && pow2_in_range(a.v_scale) ? 1 : 0;
  {
    const int64_t token_bytes = (int64_t)plan->cfg.num_kv_heads * plan->cfg.head_dim *
                                (plan->cfg.kv_dtype == DPP_KV_FP8_E4M3 ? 1 : 2);
    const int64_t pool = plan->ragged ? -1 : num_pages * plan->cfg.page_size * token_bytes;
    a.pool_bytes = pool >= 0 && pool < (int64_t)0xFFFFFFC0u ? (uint32_t)pool : 0u;
  }

  MergeArgs m{};
  m.header = a.header;
  m.part_o = a.part_o;
  m.part_lse2 = a.part_lse2;
  m.o = o;
  m.lse = lse;
  m.num_qo_heads = plan->cfg.num_qo_heads;
  m.group = plan->group;
  m.plan_id = plan->plan_id;
  m.block_m = block_m_for(plan->cfg.head_dim);

  const int passes = (int)plan->item_pass.size() - 1;
  for (int p = 0; p < passes; ++p) {
    for (int narrow = 0; narrow < 2; ++narrow) {
      a.item_begin = narrow ? plan->item_narrow[(size_t)p] : plan->item_pass[(size_t)p];
      const int32_t end = narrow ? plan->item_pass[(size_t)p + 1] : plan->item_narrow[(size_t)p];
      a.num_items = end - a.item_begin;
      a.chain_offset = narrow ? -1 : plan->chain_offset[(size_t)p];
      a.num_chains = narrow ? 0 : plan->chain_blocks[(size_t)p];
      // A wide launch that is not persistent runs the planner's block table (cost-balanced
      // XCD runs); the narrow launches run equal-count runs (xcd_chunked).
      const bool table = !narrow && a.chain_offset < 0;
      a.block_table = table ? plan->block_table_offset[(size_t)p] : -1;
      a.table_blocks = table ? plan->block_table_blocks[(size_t)p] : 0;
      if (a.num_items > 0) {
        e = launch_prefill(a, plan->cfg.head_dim, plan->cfg.kv_dtype, narrow != 0, plan->block_n, stream);
        if (e != hipSuccess) return hip_fail(e, "prefill launch");
      }
    }
    m.merge_begin = plan->merge_pass[(size_t)p];
    m.num_merges = plan->merge_pass[(size_t)p + 1] - m.merge_begin;
    if (m.num_merges > 0) {
      const bool all_narrow = plan->item_narrow[(size_t)p] == plan->item_pass[(size_t)p];
      e = launch_merge(m, plan->cfg.head_dim, plan->cfg.num_kv_heads, all_narrow ? kNarrowRows : m.block_m, stream);
      if (e != hipSuccess) return hip_fail(e, "merge launch");
    }
  }
  return DPP_OK;
}

}  // namespace dpp

extern "C" dpp_status dpp_run(const dpp_plan* plan, const void* q, int64_t q_rows,
                              const void* k_pool, const void* v_pool, int64_t num_pages,
                              const int32_t* kv_indices, int64_t num_kv_indices, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, uint32_t flags, void* stream_ptr) {
  dpp_status st = check_run_args(plan, "dpp_run", q, q_rows, k_pool, v_pool, num_pages, kv_indices, num_kv_indices,
                                 o, lse, flags);
  if (st != DPP_OK) return st;
  st = check_workspace(plan, workspace, workspace_bytes);
  if (st != DPP_OK) return st;
  hipStream_t stream = (hipStream_t)stream_ptr;
  if (plan->num_items == 0) return DPP_OK;
  if (flags & DPP_RUN_REUSE_UPLOAD) {
    st = check_reuse(plan, workspace);
  } else {
    st = enqueue_upload(plan, workspace, stream);
  }
  if (st != DPP_OK) return st;
  return launch_passes(plan, q, k_pool, v_pool, num_pages, kv_indices, o, lse, workspace, stream_ptr);
}

extern "C" dpp_status dpp_merge_states(const float* o_partial, const float* lse_partial,
                                       int64_t num_rows, int32_t num_splits, int32_t num_heads,
                                       int32_t head_dim, void* o, float* lse, void* stream_ptr) {
  if (num_rows < 0 || num_heads <= 0 || num_splits < 1 || num_splits > 1024)
    return fail(DPP_ERR_INVALID, "dpp_merge_states: need num_rows >= 0, num_heads >= 1, 1 <= num_splits <= 1024");
  if (head_dim <= 0 || head_dim % 4 != 0 || head_dim > 1024)
    return fail(DPP_ERR_UNSUPPORTED, "dpp_merge_states: head_dim must be a multiple of 4 in [4, 1024]");
  if (num_rows == 0) return DPP_OK;
  if (!o_partial || !lse_partial || !o || !lse) return fail(DPP_ERR_INVALID, "dpp_merge_states: null pointer");
  if (!aligned(o_partial, 16) || !aligned(o, 8) || !aligned(lse_partial, 4) || !aligned(lse, 4))
    return fail(DPP_ERR_INVALID, "dpp_merge_states: o_partial must be 16-byte and o 8-byte aligned");
  MergeDenseArgs a{o_partial, lse_partial, o, lse, num_rows, num_splits, num_heads, head_dim};
  hipError_t e = launch_merge_dense(a, (hipStream_t)stream_ptr);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return DPP_OK;
}
