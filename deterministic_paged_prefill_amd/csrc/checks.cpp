// Host checks of libdpp's run-time arguments: no HIP call, no device memory, so the same code
// is built with the host sanitizers by the CPU test suite.
#include <cstdint>
#include <string>

#include "plan.h"

namespace dpp {

namespace {
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
}  // namespace

dpp_status check_run_args(const dpp_plan* plan, const char* who, const void* q, int64_t q_rows,
                          const void* k_pool, const void* v_pool, int64_t num_pages,
                          const int32_t* kv_indices, int64_t num_kv_indices, const void* o,
                          const float* lse, uint32_t flags) {
  const std::string w(who);
  if (!plan) return fail(DPP_ERR_INVALID, w + ": null plan");
  if (q_rows != plan->total_q_rows)
    return fail(DPP_ERR_SHAPE, "q has " + std::to_string(q_rows) + " rows but qo_indptr[-1] is " +
                                   std::to_string(plan->total_q_rows));
  if (num_pages < 0) return fail(DPP_ERR_INVALID, w + ": negative num_pages");
  if (flags & ~DPP_RUN_REUSE_UPLOAD) return fail(DPP_ERR_INVALID, w + ": unknown flags");
  if (plan->total_q_rows > 0 && (!q || !o || !lse)) return fail(DPP_ERR_INVALID, w + ": null q, o or lse");
  if (plan->num_items > 0 && (!k_pool || !v_pool || (!kv_indices && !plan->ragged)))
    return fail(DPP_ERR_INVALID, w + ": null k_pool, v_pool or kv_indices");
  // ragged KV: num_pages counts the token rows of k_pool / v_pool, which every request's
  // [kv_indptr[r], kv_indptr[r+1]) must lie within (the kernels do not check it per key)
  if (plan->ragged && plan->total_kv_tokens > num_pages)
    return fail(DPP_ERR_SHAPE, "ragged KV: kv_indptr[-1] = " + std::to_string(plan->total_kv_tokens) +
                                   " tokens but k/v hold " + std::to_string(num_pages));
  // paged KV: the kernels read kv_indices[kv_indptr[r] ..) for every request
  if (!plan->ragged && plan->total_kv_entries > num_kv_indices)
    return fail(DPP_ERR_SHAPE, "kv_indices holds " + std::to_string(num_kv_indices) +
                                   " page ids but kv_indptr[-1] is " + std::to_string(plan->total_kv_entries));
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(lse, 4) || (!plan->ragged && !aligned(kv_indices, 4)))
    return fail(DPP_ERR_INVALID, w + ": q/o/k_pool/v_pool must be 16-byte aligned");
  return DPP_OK;
}

}  // namespace dpp

using namespace dpp;

extern "C" dpp_status dpp_check_page_table(const dpp_plan* plan, const int32_t* kv_indices_host,
                                           int64_t num_kv_indices, int64_t num_pages) {
  if (!plan) return fail(DPP_ERR_INVALID, "dpp_check_page_table: null plan");
  if (num_pages < 0 || num_kv_indices < 0) return fail(DPP_ERR_INVALID, "dpp_check_page_table: negative count");
  if (plan->ragged) return DPP_OK;  // no page table
  if (plan->total_kv_entries > num_kv_indices)
    return fail(DPP_ERR_SHAPE, "kv_indices holds " + std::to_string(num_kv_indices) +
                                   " page ids but kv_indptr[-1] is " + std::to_string(plan->total_kv_entries));
  if (plan->total_kv_entries > 0 && !kv_indices_host) return fail(DPP_ERR_INVALID, "dpp_check_page_table: null kv_indices");
  // every page a request reads: ceil(kv_len / page_size) ids from its page_start
  const HeaderPreamble* pre = reinterpret_cast<const HeaderPreamble*>(plan->header.data());
  const RequestDesc* reqs = reinterpret_cast<const RequestDesc*>(plan->header.data() + pre->request_offset);
  const int64_t P = plan->cfg.page_size;
  for (int32_t r = 0; r < plan->batch_size; ++r) {
    const int64_t n = (reqs[r].kv_len + P - 1) / P;
    for (int64_t j = 0; j < n; ++j) {
      const int64_t id = kv_indices_host[reqs[r].page_start + j];
      if (id < 0 || id >= num_pages)
        return fail(DPP_ERR_SHAPE, "request " + std::to_string(r) + ", page " + std::to_string(j) + ": id " +
                                       std::to_string(id) + " outside [0, " + std::to_string(num_pages) + ")");
    }
  }
  return DPP_OK;
}
