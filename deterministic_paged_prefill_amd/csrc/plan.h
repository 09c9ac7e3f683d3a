// Host planner of libdpp: turns one batch shape into the work list the kernels run.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dpp.h"
#include "dpp_internal.h"

struct dpp_plan {
  dpp_config cfg{};
  int32_t group = 1;
  float scale_log2 = 0.f;  // sm_scale * log2(e), rounded once to fp32
  int32_t batch_size = 0;
  int64_t total_q_rows = 0;

  // Work list (int32 words): preamble, requests, prefill items, merge items.
  std::vector<int32_t> header;
  int32_t num_items = 0;
  int32_t num_merges = 0;

  // Pass p runs prefill items [item_pass[p], item_pass[p+1]) and merge items
  // [merge_pass[p], merge_pass[p+1]).
  std::vector<int32_t> item_pass;
  std::vector<int32_t> merge_pass;
  // Pass p runs items [item_pass[p], item_narrow[p]) on the wide kernel and
  // [item_narrow[p], item_pass[p+1]) on the narrow one (one of the two ranges is empty).
  std::vector<int32_t> item_narrow;
  // Pass p's wide launch is persistent if chain_offset[p] >= 0: chain_blocks[p] workgroups
  // over the unit records at that word offset of the header.
  std::vector<int32_t> chain_offset;
  std::vector<int32_t> chain_blocks;
  // Pass p's wide launch when it is not persistent: block_table_blocks[p] workgroups, block b
  // running the unit at word block_table_offset[p] + b of the header (-1: none).
  std::vector<int32_t> block_table_offset;
  std::vector<int32_t> block_table_blocks;

  int64_t max_partial_slots = 0;
  size_t header_bytes = 0;
  size_t partial_o_offset = 0;    // byte offsets inside the workspace
  size_t partial_lse_offset = 0;
  size_t workspace_bytes = 0;
  int32_t page_slots = 0;         // LDS page-id entries one item may need
  bool ragged = false;            // page_size 0: contiguous KV, kv_indptr counts tokens
  int32_t block_n = 0;            // keys per KV tile: block_n_for(head_dim), except in the
                                  // adaptive-tile comparison mode
  int64_t total_kv_tokens = 0;    // ragged: kv_indptr[B], the KV rows the kernels may read
  int64_t total_kv_entries = 0;   // kv_indptr[B]: page ids the kernels read from kv_indices
                                  // (paged), or KV token rows (ragged)
  int32_t item_offset = 0;        // word offset of the item records in the header
  uint32_t plan_id = 0;           // stamped into the work list

  // Pinned host copy of `header`, created on first dpp_run (plan creation stays HIP-free).
  mutable std::mutex pinned_mu;
  mutable void* pinned = nullptr;
  mutable size_t pinned_cap = 0;  // bytes of the pinned block (a pool size class)
  // Workspace of the last enqueued upload of this plan's work list (guarded by pinned_mu):
  // a run that reuses an upload must name the same workspace.
  mutable const void* uploaded_ws = nullptr;
};

namespace dpp {

// Thread-local error text behind dpp_last_error().
void set_error(const std::string& msg);
dpp_status fail(dpp_status st, const std::string& msg);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host checks of a run's arguments (everything but the workspace), shared by the entry points.
dpp_status check_run_args(const dpp_plan* plan, const char* who, const void* q, int64_t q_rows,
                          const void* k_pool, const void* v_pool, int64_t num_pages,
                          const int32_t* kv_indices, int64_t num_kv_indices, const void* o,
                          const float* lse, uint32_t flags);

// Enqueue the prefill and merge launches of every pass over a workspace that holds the plan's
// work list (stream-ordered after its upload).
dpp_status launch_passes(const dpp_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                         int64_t num_pages, const int32_t* kv_indices, void* o, float* lse, void* workspace,
                         void* stream);

}  // namespace dpp
