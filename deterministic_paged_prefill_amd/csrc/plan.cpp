// Host planner: batch shape -> work list. Pure integer host code; no HIP calls.
//
// What it decides, and what it never decides:
//  * tile geometry (block_m_for(head_dim) packed rows x block_n_for(head_dim) keys) and the
//    4096-token split length are constants of the configuration; nothing here reads the batch's average or maximum query length (the sglang
//    PR #46351 page, "Root cause", is the failure this avoids);
//  * a request's query block is right-aligned to its KV: row i sits at position
//    kv_len - qo_len + i (same page, "Fix" section);
//  * a q tile visits KV tiles 0 .. floor(p_max / BN) of every split its last row reaches;
//    rows needing one split finish in the prefill kernel, longer rows leave one partial per
//    split in the workspace and are combined by the merge kernel;
//  * passes: partials are bounded by the caller's cap by running tiles in several launches
//    (the model-serving-minefield issue #73 correction, "The failure", shows an unbounded
//    split buffer crashing a server);
//  * order: inside a pass, requests with the longest item first, a request's items kept
//    together and longest first (load balance, and L2 reuse of the request's KV); a pass of
//    tiles with at most kNarrowRows rows each runs on the narrow kernel;
//  * persistent chains: a wide bf16 pass at head_dim <= 256 runs as kPersistentBlocks
//    workgroups, each over a chain of units (item, kv head). Each group of XCDs (as many as
//    share one kv head's units) takes a contiguous run of the plain launch order (unit
//    kv_head * items + item) holding its share of the pass's cost; the run is dealt longest
//    first to the least loaded of the group's workgroups (b % kXcds in the group), each chain
//    then rotated by its workgroup's rank in the group;
//  * block tables: a wide pass that is not persistent gets each group's run, longest first,
//    dealt round-robin over the group's XCDs. Order, passes, cap, chains, tables and kernel
//    instantiation change when and where a row is computed, never its arithmetic.
#include "plan.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <memory>
#include <new>

namespace dpp {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

dpp_status fail(dpp_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

namespace {

struct TileInfo {
  int32_t request;
  int32_t row_start;
  int32_t rows;
  int64_t p_max;
  int32_t splits;
  int32_t pass = 0;
  int64_t slot_base = -1;
};

// Cost of a unit (item, kv head) for load balance: its KV tiles plus a start-up allowance.
int64_t unit_cost(const PrefillItem& it) { return (int64_t)(it.kv_tile_end - it.kv_tile_begin) + kUnitOverheadTiles; }

// XCD groups: xg neighbouring XCDs (x / xg == g) share one run of the plain launch order
// (unit w = kv_head * n + item, the n items of one wide launch): group g takes units
// [run[g], run[g+1]), a contiguous run (so that the units of one kv head share few L2s) holding
// its share of the total cost. With `blocks` > 0 the shares follow the workgroups b < blocks of
// each group and every run holds at least one unit per workgroup; otherwise the shares are
// equal. Runs of equal unit counts per XCD would not balance (with 4 kv heads on 8 XCDs, one XCD
// of each pair would take the long tiles of its head and the other the short ones), and a run
// that holds part of one kv head leaves an XCD units of one size, which its compute units
// cannot share out evenly. So a group is as many XCDs as share one kv head's units (8 / kv
// heads, rounded down to a power of two; one XCD at 8 or more kv heads), and it deals the long
// and the short units of its run among them.
int xcd_group_size(int32_t num_kv_heads) {
  int xg = 1;
  while (xg * 2 <= kXcds && xg * 2 * num_kv_heads <= kXcds) xg *= 2;
  return xg;
}
std::vector<int64_t> group_runs(const PrefillItem* items, int32_t n, int32_t num_kv_heads, int32_t blocks, int xg) {
  const int groups = kXcds / xg;
  const int64_t n_units = (int64_t)n * num_kv_heads;
  std::vector<int64_t> prefix((size_t)n_units + 1, 0);
  for (int64_t u = 0; u < n_units; ++u) prefix[(size_t)u + 1] = prefix[(size_t)u] + unit_cost(items[u % n]);
  auto blocks_of = [&](int g) {  // workgroups b < blocks with b % kXcds in group g
    int64_t c = 0;
    for (int x = g * xg; x < (g + 1) * xg; ++x) c += blocks > x ? (blocks - 1 - x) / kXcds + 1 : 0;
    return c;
  };
  std::vector<int64_t> run((size_t)groups + 1, 0);
  const int64_t weight_total = blocks > 0 ? blocks : groups;
  int64_t weight_before = 0, start = 0;
  for (int g = 0; g < groups; ++g) {
    const int64_t bg = blocks > 0 ? blocks_of(g) : 0;
    weight_before += blocks > 0 ? bg : 1;
    const int64_t min_after = blocks > 0 ? blocks - weight_before : 0;
    int64_t e = n_units;
    if (g < groups - 1) {
      // the first end whose prefix reaches the target, or the one before it if that is closer
      const int64_t target = (prefix[(size_t)n_units] * weight_before + weight_total / 2) / weight_total;
      e = std::lower_bound(prefix.begin() + start, prefix.end(), target) - prefix.begin();
      if (e > start && target - prefix[(size_t)e - 1] < prefix[(size_t)std::min<int64_t>(e, n_units)] - target) --e;
      e = std::min(std::max(e, start + bg), n_units - min_after);
    }
    run[(size_t)g + 1] = e;
    start = e;
  }
  return run;
}

// Block table of a wide launch that is not persistent: entry b (block b, which the dispatcher
// hands to XCD b % kXcds) is the unit that block runs, or -1 (the block exits). Group g's run,
// longest first, is dealt round-robin to its XCDs, so every XCD starts its longest units first
// and its compute units fill in behind them with the short ones.
std::vector<int32_t> block_table(const PrefillItem* items, int32_t n, int32_t num_kv_heads) {
  const int xg = xcd_group_size(num_kv_heads);
  const std::vector<int64_t> run = group_runs(items, n, num_kv_heads, 0, xg);
  std::vector<std::vector<int32_t>> per_xcd(kXcds);
  for (int g = 0; g < kXcds / xg; ++g) {
    std::vector<int64_t> order;
    for (int64_t u = run[(size_t)g]; u < run[(size_t)g + 1]; ++u) order.push_back(u);
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return unit_cost(items[a % n]) > unit_cost(items[b % n]); });
    for (size_t r = 0; r < order.size(); ++r) per_xcd[(size_t)(g * xg) + r % (size_t)xg].push_back((int32_t)order[r]);
  }
  size_t len = 0;
  for (const auto& l : per_xcd) len = std::max(len, l.size());
  std::vector<int32_t> table(len * kXcds, -1);
  for (int x = 0; x < kXcds; ++x)
    for (size_t k = 0; k < per_xcd[(size_t)x].size(); ++k) table[k * kXcds + (size_t)x] = per_xcd[(size_t)x][k];
  return table;
}

// Largest slot count n with align(n*D*4) + align(n*4) <= avail.
// Persistent chains of one wide pass whose units are (item i, kv head h), unit w = h * n + i
// for the n items at `items`: records placed so that workgroup b starts at record b.
std::vector<UnitRecord> build_chains(const PrefillItem* items, int32_t n, int32_t num_kv_heads,
                                     int32_t pass) {
  const int64_t n_units = (int64_t)n * num_kv_heads;
  const int32_t nb = (int32_t)std::min<int64_t>(n_units, kPersistentBlocks);
  std::vector<UnitRecord> rec((size_t)n_units);
  int32_t next_free = nb;
  auto cost = [&](int64_t u) { return unit_cost(items[u % n]); };
  const int xg = xcd_group_size(num_kv_heads);
  const std::vector<int64_t> run_begin = group_runs(items, n, num_kv_heads, nb, xg);
  for (int g = 0; g < kXcds / xg; ++g) {
    const int64_t u0 = run_begin[(size_t)g], len = run_begin[(size_t)g + 1] - u0;
    std::vector<int32_t> blocks;
    for (int32_t b = 0; b < nb; ++b)
      if ((b % kXcds) / xg == g) blocks.push_back(b);
    if (len == 0) continue;
    std::vector<int64_t> order((size_t)len);
    for (int64_t k = 0; k < len; ++k) order[(size_t)k] = u0 + k;
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return cost(a) > cost(b); });
    std::vector<int64_t> load(blocks.size(), 0);
    std::vector<std::vector<int64_t>> chain(blocks.size());
    for (int64_t u : order) {
      size_t k = 0;
      for (size_t j = 1; j < blocks.size(); ++j)
        if (load[j] < load[k]) k = j;
      load[k] += cost(u);
      chain[k].push_back(u);
    }
    // A workgroup's finish time is the sum over its chain, whatever the order; rotating the
    // j-th workgroup's chain (of its group) by j keeps neighbours from switching units (a
    // burst of Q reads and O writes) at the same moments.
    for (size_t k = 0; k < blocks.size(); ++k) {
      std::vector<int64_t>& c = chain[k];
      if (c.empty()) continue;
      std::rotate(c.begin(), c.begin() + (std::ptrdiff_t)(k % c.size()), c.end());
      const int32_t b = blocks[k];
      int32_t prev_idx = -1;
      for (size_t j = 0; j < c.size(); ++j) {
        const int64_t u = c[j];
        const int32_t idx = j == 0 ? b : next_free++;
        if (prev_idx >= 0) rec[(size_t)prev_idx].next = idx;
        prev_idx = idx;
        const PrefillItem& it = items[u % n];
        UnitRecord& ur = rec[(size_t)idx];
        ur.request = it.request;
        ur.row_start = it.row_start;
        ur.split = it.split;
        ur.tile_splits = it.tile_splits;
        ur.kv_tile_begin = it.kv_tile_begin;
        ur.kv_tile_end = it.kv_tile_end;
        ur.slot_base = it.slot_base;
        ur.next = -1;
        ur.req = it.req;
        ur.kv_head = (int32_t)(u / n);
        ur.block = b;
        ur.pass = pass;
        ur.pad = 0;
      }
    }
  }
  return rec;
}

int64_t max_slots_for(size_t avail, int head_dim) {
  const size_t per_slot = (size_t)(head_dim + 1) * 4;
  int64_t n = (int64_t)(avail / per_slot);
  while (n > 0 && align_up((size_t)n * head_dim * 4, 256) + align_up((size_t)n * 4, 256) > avail) --n;
  return n;
}

}  // namespace
}  // namespace dpp

using namespace dpp;

extern "C" dpp_status dpp_plan_create(const dpp_config* cfg, int32_t batch_size,
                                      const int32_t* qo_indptr, const int32_t* kv_indptr,
                                      const int32_t* last_page_len, size_t workspace_cap,
                                      dpp_plan** out_plan) {
  return dpp_plan_create_ex(cfg, batch_size, qo_indptr, kv_indptr, last_page_len, workspace_cap, 0u, out_plan);
}

extern "C" dpp_status dpp_plan_create_ex(const dpp_config* cfg, int32_t batch_size,
                                         const int32_t* qo_indptr, const int32_t* kv_indptr,
                                         const int32_t* last_page_len, size_t workspace_cap,
                                         uint32_t plan_flags, dpp_plan** out_plan) {
  if (out_plan) *out_plan = nullptr;
  if (plan_flags & ~(uint32_t)(DPP_PLAN_ADAPTIVE_KV_TILE | DPP_PLAN_PERMUTE_WORK | DPP_PLAN_PERMUTE_SEED(0xFFFF)))
    return fail(DPP_ERR_INVALID, "dpp_plan_create_ex: unknown plan flags");
  if (!(plan_flags & DPP_PLAN_PERMUTE_WORK) && (plan_flags >> 16))
    return fail(DPP_ERR_INVALID, "dpp_plan_create_ex: a permutation seed without DPP_PLAN_PERMUTE_WORK");
  if (!cfg || !out_plan) return fail(DPP_ERR_INVALID, "dpp_plan_create: null cfg or out_plan");
  if (batch_size < 0) return fail(DPP_ERR_INVALID, "dpp_plan_create: negative batch_size");
  const bool ragged = cfg && cfg->page_size == 0;
  if (!qo_indptr || !kv_indptr || (batch_size > 0 && !last_page_len && !ragged))
    return fail(DPP_ERR_INVALID, "dpp_plan_create: null index array");

  const dpp_config c = *cfg;
  if (c.num_qo_heads <= 0 || c.num_kv_heads <= 0 || c.num_qo_heads % c.num_kv_heads != 0)
    return fail(DPP_ERR_UNSUPPORTED,
                "num_qo_heads must be a positive multiple of num_kv_heads (got " +
                    std::to_string(c.num_qo_heads) + "/" + std::to_string(c.num_kv_heads) + ")");
  if (c.num_qo_heads / c.num_kv_heads > kMaxGroup)
    return fail(DPP_ERR_UNSUPPORTED, "num_qo_heads / num_kv_heads must be at most " + std::to_string(kMaxGroup));
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256 && c.head_dim != 512)
    return fail(DPP_ERR_UNSUPPORTED, "head_dim " + std::to_string(c.head_dim) +
                                         " not built (64, 128, 256 and 512 are)");
  if (c.page_size < 0 || c.page_size > 1024)
    return fail(DPP_ERR_UNSUPPORTED, "page_size must be in [1, 1024], or 0 for ragged KV");
  if (c.kv_dtype != DPP_KV_BF16 && c.kv_dtype != DPP_KV_FP8_E4M3)
    return fail(DPP_ERR_UNSUPPORTED, "kv_dtype must be DPP_KV_BF16 or DPP_KV_FP8_E4M3");
  if (!(c.sm_scale >= 0.f) || !std::isfinite(c.sm_scale))
    return fail(DPP_ERR_INVALID, "sm_scale must be finite and >= 0");
  if (c.kv_dtype == DPP_KV_FP8_E4M3 &&
      (!std::isfinite(c.k_scale) || !std::isfinite(c.v_scale) || c.k_scale <= 0.f || c.v_scale <= 0.f))
    return fail(DPP_ERR_INVALID, "fp8 k_scale / v_scale must be finite and > 0");

  if (qo_indptr[0] != 0 || kv_indptr[0] != 0)
    return fail(DPP_ERR_INVALID, "qo_indptr[0] and kv_indptr[0] must be 0");
  const int32_t group = c.num_qo_heads / c.num_kv_heads;
  const int64_t P = ragged ? kRaggedPage : c.page_size;
  // ragged: a request's keys are addressed by 32-bit byte offsets from its first token
  const int64_t token_bytes = (int64_t)c.num_kv_heads * c.head_dim * (c.kv_dtype == DPP_KV_FP8_E4M3 ? 1 : 2);

  int32_t block_n = block_n_for(c.head_dim);
  const int32_t block_m = block_m_for(c.head_dim);
  std::vector<RequestDesc> reqs((size_t)batch_size);
  std::vector<TileInfo> tiles;
  for (int32_t r = 0; r < batch_size; ++r) {
    const int64_t qo_len = (int64_t)qo_indptr[r + 1] - qo_indptr[r];
    const int64_t np = (int64_t)kv_indptr[r + 1] - kv_indptr[r];
    if (qo_len < 0 || np < 0)
      return fail(DPP_ERR_INVALID, "indptr not non-decreasing at request " + std::to_string(r));
    int64_t kv_len = 0;
    if (ragged) {
      kv_len = np;  // kv_indptr counts tokens
      // (a load descriptor of the last KV tile may start up to one tile past kv_len)
      if ((kv_len + 256) * token_bytes > std::numeric_limits<int32_t>::max())
        return fail(DPP_ERR_UNSUPPORTED, "ragged request " + std::to_string(r) + " holds more than 2 GiB of K");
    } else if (np > 0) {
      if (last_page_len[r] < 1 || last_page_len[r] > c.page_size)
        return fail(DPP_ERR_SHAPE, "kv_last_page_len[" + std::to_string(r) + "] = " +
                                       std::to_string(last_page_len[r]) + " outside [1, page_size]");
      kv_len = (np - 1) * P + last_page_len[r];
    }
    if (kv_len > std::numeric_limits<int32_t>::max() / 2)
      return fail(DPP_ERR_UNSUPPORTED, "kv_len too large at request " + std::to_string(r));
    if (qo_len > kv_len)
      return fail(DPP_ERR_SHAPE, "request " + std::to_string(r) + ": qo_len " +
                                     std::to_string(qo_len) + " > kv_len " + std::to_string(kv_len));
    reqs[(size_t)r] = RequestDesc{qo_indptr[r], (int32_t)qo_len, kv_indptr[r], (int32_t)kv_len};
    const int64_t packed = qo_len * group;
    if (packed > std::numeric_limits<int32_t>::max() - block_m)
      return fail(DPP_ERR_UNSUPPORTED, "too many query rows in request " + std::to_string(r));
    for (int64_t rs = 0; rs < packed; rs += block_m) {
      TileInfo t{};
      t.request = r;
      t.row_start = (int32_t)rs;
      t.rows = (int32_t)std::min<int64_t>(block_m, packed - rs);
      t.p_max = kv_len - qo_len + (rs + t.rows - 1) / group;
      t.splits = (int32_t)(t.p_max / kSplitTokens + 1);
      tiles.push_back(t);
    }
  }

  // Adaptive-tile comparison mode (never batch invariant): FlashInfer's rule on the sglang PR
  // #46351 page ("Root cause"; the author's A100 findings) gives a 16-row q tile when the
  // batch's average packed query length sum(qo_len * group) / batch_size is at most 16, and
  // the tile moves the reduction split. Here the q tile never touches a row's arithmetic, so
  // the mode moves what does: such a batch of narrow tiles runs with 32-key KV tiles at
  // head_dim 128 instead of 64, and its rows stop matching the same rows of a larger batch.
  if ((plan_flags & DPP_PLAN_ADAPTIVE_KV_TILE) && c.head_dim == 128 && c.kv_dtype == DPP_KV_BF16 &&
      batch_size > 0 && !tiles.empty()) {
    int64_t packed = 0;
    for (int32_t r = 0; r < batch_size; ++r) packed += (int64_t)reqs[(size_t)r].qo_len * group;
    const bool all_narrow = std::all_of(tiles.begin(), tiles.end(), [](const TileInfo& t) { return t.rows <= kNarrowRows; });
    if (all_narrow && packed <= 16 * (int64_t)batch_size) block_n = 32;
  }
  const int32_t tiles_per_split = kSplitTokens / block_n;

  int64_t n_items = 0, n_merges = 0;
  for (const auto& t : tiles) {
    n_items += t.splits;
    n_merges += t.splits > 1 ? 1 : 0;
  }
  if (n_items > std::numeric_limits<int32_t>::max() / 2 / c.num_kv_heads / kItemWords)
    return fail(DPP_ERR_UNSUPPORTED, "batch too large for one plan");
  // Unit records of persistent launches: at most one per (item, kv head).
  const bool chain_kind = chained_launch(c.head_dim, c.kv_dtype == DPP_KV_FP8_E4M3, false);
  const int64_t max_units = chain_kind ? n_items * c.num_kv_heads : 0;
  // block tables of the wide launches that are not persistent: per pass 2 words and kXcds
  // entries per unit of the longest XCD list, at most half a group's run (a persistent kind
  // that falls back to tables needs fewer words than its unit records would)
  const int64_t max_table_words = chain_kind ? 0 : 4 * n_items * c.num_kv_heads + (2 + kXcds) * n_items;
  const int64_t words_max =
      kHeaderWords + 4 * (int64_t)batch_size + kItemWords * (n_items + max_units) + 4 * n_merges + max_table_words;
  if (words_max > std::numeric_limits<int32_t>::max() / 2)
    return fail(DPP_ERR_UNSUPPORTED, "batch too large for one plan");
  // The cap is checked against the largest header this plan can have (its unit records
  // depend on the passes, which depend on the cap).
  const size_t header_bytes_max = align_up((size_t)words_max * 4, 256);

  int64_t slot_limit = std::numeric_limits<int32_t>::max() / 2;
  if (workspace_cap > 0) {
    if (workspace_cap < header_bytes_max)
      return fail(DPP_ERR_WORKSPACE, "workspace cap " + std::to_string(workspace_cap) +
                                         " B is below the work list's " +
                                         std::to_string(header_bytes_max) + " B");
    slot_limit = std::min<int64_t>(slot_limit, max_slots_for(workspace_cap - header_bytes_max, c.head_dim));
  }

  // Passes: tiles in request order; a tile needing partials takes S_t * Hkv * slot_rows_for(rows)
  // slots.
  int32_t pass = 0;
  int64_t used = 0, max_used = 0;
  for (auto& t : tiles) {
    const int64_t need = t.splits > 1 ? (int64_t)t.splits * c.num_kv_heads * slot_rows_for(t.rows) : 0;
    if (need > slot_limit)
      return fail(DPP_ERR_WORKSPACE,
                  "workspace cap too small: one q tile needs " +
                      std::to_string(need * (c.head_dim + 1) * 4 + header_bytes_max) + " B");
    if (used + need > slot_limit) {
      ++pass;
      used = 0;
    }
    t.pass = pass;
    if (need > 0) {
      t.slot_base = used;
      used += need;
      max_used = std::max(max_used, used);
    }
  }
  const int32_t num_passes = tiles.empty() ? 0 : pass + 1;

  std::unique_ptr<dpp_plan> plan(new (std::nothrow) dpp_plan());
  if (!plan) return fail(DPP_ERR_INVALID, "out of host memory");
  plan->cfg = c;
  if (plan->cfg.sm_scale == 0.f) plan->cfg.sm_scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  if (c.kv_dtype == DPP_KV_BF16) plan->cfg.k_scale = plan->cfg.v_scale = 1.f;
  plan->group = group;
  plan->scale_log2 = (float)((double)plan->cfg.sm_scale * 1.4426950408889634);
  plan->batch_size = batch_size;
  plan->total_q_rows = batch_size > 0 ? qo_indptr[batch_size] : 0;
  plan->num_items = (int32_t)n_items;
  plan->num_merges = (int32_t)n_merges;

  // Emit items pass by pass in the order described at the top of this file.
  std::vector<PrefillItem> items;
  std::vector<MergeItem> merges;
  items.reserve((size_t)n_items);
  merges.reserve((size_t)n_merges);
  plan->item_pass.assign(1, 0);
  plan->merge_pass.assign(1, 0);
  plan->item_narrow.clear();
  int64_t max_page_span = 1;
  size_t tile_cursor = 0;
  for (int32_t p = 0; p < num_passes; ++p) {
    const size_t first = items.size();
    while (tile_cursor < tiles.size() && tiles[tile_cursor].pass == p) {
      const TileInfo& t = tiles[tile_cursor++];
      const RequestDesc& rq = reqs[(size_t)t.request];
      const int64_t last_tile = t.p_max / block_n;
      for (int32_t s = 0; s < t.splits; ++s) {
        PrefillItem it{};
        it.request = t.request;
        it.row_start = t.row_start;
        it.split = s;
        it.tile_splits = t.splits;
        it.kv_tile_begin = s * tiles_per_split;
        it.kv_tile_end = (int32_t)std::min<int64_t>((int64_t)(s + 1) * tiles_per_split, last_tile + 1);
        it.slot_base = (int32_t)t.slot_base;
        it.pass = p;
        it.req = rq;
        const int64_t key_lo = (int64_t)it.kv_tile_begin * block_n;
        const int64_t key_hi = std::min<int64_t>((int64_t)it.kv_tile_end * block_n, rq.kv_len);
        if (key_hi > key_lo) max_page_span = std::max(max_page_span, (key_hi - 1) / P - key_lo / P + 1);
        items.push_back(it);
      }
      if (t.splits > 1) merges.push_back(MergeItem{t.request, t.row_start, t.splits, (int32_t)t.slot_base});
    }
    // Requests whose longest item is longer go first; a request's items stay together
    // (they read the same KV, and the launch hands contiguous runs of items to one XCD),
    // longest first among them.
    std::vector<int32_t> req_len((size_t)batch_size, 0);
    for (size_t i = first; i < items.size(); ++i) {
      int32_t& m = req_len[(size_t)items[i].request];
      m = std::max(m, items[i].kv_tile_end - items[i].kv_tile_begin);
    }
    std::stable_sort(items.begin() + (std::ptrdiff_t)first, items.end(),
                     [&](const PrefillItem& a, const PrefillItem& b) {
                       const int32_t ra = req_len[(size_t)a.request], rb = req_len[(size_t)b.request];
                       if (ra != rb) return ra > rb;
                       if (a.request != b.request) return a.request < b.request;
                       return (a.kv_tile_end - a.kv_tile_begin) > (b.kv_tile_end - b.kv_tile_begin);
                     });
    if (plan_flags & DPP_PLAN_PERMUTE_WORK) {
      // test mode: any order of the pass's work must give the same bits
      uint64_t st = 0x9E3779B97F4A7C15ull ^ ((uint64_t)(plan_flags >> 16) << 32) ^ (uint64_t)p;
      auto next = [&](uint64_t n) {  // splitmix64, reduced to [0, n)
        st += 0x9E3779B97F4A7C15ull;
        uint64_t z = st;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return (z ^ (z >> 31)) % n;
      };
      for (size_t k = items.size() - first; k > 1; --k) std::swap(items[first + k - 1], items[first + next(k)]);
      const size_t mfirst = (size_t)plan->merge_pass.back();  // this pass's first merge
      for (size_t k = merges.size() - mfirst; k > 1; --k) std::swap(merges[mfirst + k - 1], merges[mfirst + next(k)]);
    }
    // A pass whose tiles all have at most kNarrowRows rows (extends) runs on the narrow
    // kernel; a pass with wider tiles runs all its items in one launch of the wide kernel,
    // so that its short tiles fill in behind the long ones instead of running after them.
    const bool all_narrow = std::all_of(items.begin() + (std::ptrdiff_t)first, items.end(),
                                        [&](const PrefillItem& it) {
                                          const RequestDesc& rq = reqs[(size_t)it.request];
                                          return (int64_t)rq.qo_len * group - it.row_start <= kNarrowRows;
                                        });
    plan->item_narrow.push_back(all_narrow ? (int32_t)first : (int32_t)items.size());
    plan->item_pass.push_back((int32_t)items.size());
    plan->merge_pass.push_back((int32_t)merges.size());
  }

  // Persistent chains for the wide launches, where two page tables fit beside the ring.
  const bool chains_fit =
      ring_bytes_for(c.head_dim) + 2 * page_table_bytes(max_page_span, c.head_dim) + kOutStageBytes <= (int64_t)kLdsLimit;
  std::vector<UnitRecord> units;
  plan->chain_offset.assign((size_t)num_passes, -1);
  plan->chain_blocks.assign((size_t)num_passes, 0);
  const int32_t unit_offset = kHeaderWords + 4 * batch_size + kItemWords * (int32_t)n_items + 4 * (int32_t)n_merges;
  for (int32_t p = 0; p < num_passes && chain_kind && chains_fit; ++p) {
    const int32_t b0 = plan->item_pass[(size_t)p], b1 = plan->item_narrow[(size_t)p];
    if (b1 <= b0) continue;
    std::vector<UnitRecord> r = build_chains(items.data() + b0, b1 - b0, c.num_kv_heads, p);
    plan->chain_offset[(size_t)p] = unit_offset + kItemWords * (int32_t)units.size();
    plan->chain_blocks[(size_t)p] = (int32_t)std::min<int64_t>(r.size(), kPersistentBlocks);
    units.insert(units.end(), r.begin(), r.end());
  }
  // Block tables of the wide launches that are not persistent, after the unit records: per
  // pass, its index and block count, then the entries.
  const int32_t table_offset = unit_offset + kItemWords * (int32_t)units.size();
  std::vector<int32_t> tables;
  int32_t num_tables = 0;
  plan->block_table_offset.assign((size_t)num_passes, -1);
  plan->block_table_blocks.assign((size_t)num_passes, 0);
  for (int32_t p = 0; p < num_passes; ++p) {
    const int32_t b0 = plan->item_pass[(size_t)p], b1 = plan->item_narrow[(size_t)p];
    if (b1 <= b0 || plan->chain_offset[(size_t)p] >= 0) continue;
    const std::vector<int32_t> t = block_table(items.data() + b0, b1 - b0, c.num_kv_heads);
    tables.push_back(p);
    tables.push_back((int32_t)t.size());
    plan->block_table_offset[(size_t)p] = table_offset + (int32_t)tables.size();
    plan->block_table_blocks[(size_t)p] = (int32_t)t.size();
    tables.insert(tables.end(), t.begin(), t.end());
    ++num_tables;
  }
  const int64_t words = table_offset + (int64_t)tables.size();
  if (words > words_max) return fail(DPP_ERR_INVALID, "internal error: work list longer than its bound");
  const size_t header_bytes = align_up((size_t)words * 4, 256);

  // Serialise: preamble | requests | items | merges | unit records | block tables.
  plan->header.assign((size_t)words, 0);
  HeaderPreamble pre{};
  pre.magic = kHeaderMagic;
  pre.num_requests = batch_size;
  pre.num_items = (int32_t)n_items;
  pre.num_merges = (int32_t)n_merges;
  pre.request_offset = kHeaderWords;
  pre.item_offset = kHeaderWords + 4 * batch_size;
  pre.merge_offset = pre.item_offset + kItemWords * (int32_t)n_items;
  pre.unit_offset = units.empty() ? 0 : unit_offset;
  pre.num_units = (int32_t)units.size();
  pre.table_offset = tables.empty() ? 0 : table_offset;
  pre.num_tables = num_tables;
  {
    // ids differ between plans of one process; mixing in the address makes a header left
    // behind by another process unlikely to match either
    static std::atomic<uint32_t> counter{0x9E3779B9u};
    uint32_t id = counter.fetch_add(0x61C88647u) ^ (uint32_t)(uintptr_t)plan.get();
    pre.plan_id = id == 0 ? 1u : id;
    plan->plan_id = pre.plan_id;
  }
  std::memcpy(plan->header.data(), &pre, sizeof pre);
  plan->item_offset = pre.item_offset;
  if (batch_size > 0)
    std::memcpy(plan->header.data() + pre.request_offset, reqs.data(), reqs.size() * sizeof(RequestDesc));
  if (!items.empty())
    std::memcpy(plan->header.data() + pre.item_offset, items.data(), items.size() * sizeof(PrefillItem));
  if (!merges.empty())
    std::memcpy(plan->header.data() + pre.merge_offset, merges.data(), merges.size() * sizeof(MergeItem));
  if (!units.empty())
    std::memcpy(plan->header.data() + unit_offset, units.data(), units.size() * sizeof(UnitRecord));
  if (!tables.empty()) std::memcpy(plan->header.data() + table_offset, tables.data(), tables.size() * sizeof(int32_t));

  plan->max_partial_slots = max_used;
  plan->header_bytes = header_bytes;
  plan->partial_o_offset = header_bytes;
  plan->partial_lse_offset = header_bytes + align_up((size_t)max_used * c.head_dim * 4, 256);
  plan->workspace_bytes = plan->partial_lse_offset + align_up((size_t)max_used * 4, 256);
  plan->page_slots = (int32_t)max_page_span;
  plan->ragged = ragged;
  plan->block_n = block_n;
  plan->total_kv_tokens = ragged && batch_size > 0 ? kv_indptr[batch_size] : 0;
  plan->total_kv_entries = batch_size > 0 ? kv_indptr[batch_size] : 0;
  *out_plan = plan.release();
  return DPP_OK;
}

extern "C" size_t dpp_plan_workspace_bytes(const dpp_plan* plan) {
  return plan ? plan->workspace_bytes : 0;
}

extern "C" dpp_status dpp_plan_get_info(const dpp_plan* plan, dpp_plan_info* info) {
  if (!plan || !info) return fail(DPP_ERR_INVALID, "dpp_plan_get_info: null argument");
  info->block_m = block_m_for(plan->cfg.head_dim);
  info->block_n = plan->block_n;
  info->split_tokens = kSplitTokens;
  info->num_passes = (int32_t)plan->item_pass.size() - 1;
  info->num_prefill_items = plan->num_items;
  info->num_merge_items = plan->num_merges;
  info->max_partial_slots = plan->max_partial_slots;
  info->header_bytes = plan->header_bytes;
  info->workspace_bytes = plan->workspace_bytes;
  info->total_q_rows = plan->total_q_rows;
  return DPP_OK;
}

extern "C" dpp_status dpp_plan_header(const dpp_plan* plan, const void** data, size_t* bytes) {
  if (!plan || !data || !bytes) return fail(DPP_ERR_INVALID, "dpp_plan_header: null argument");
  *data = plan->header.data();
  *bytes = plan->header.size() * sizeof(int32_t);
  return DPP_OK;
}

extern "C" const char* dpp_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* dpp_status_string(dpp_status st) {
  switch (st) {
    case DPP_OK: return "DPP_OK";
    case DPP_ERR_INVALID: return "DPP_ERR_INVALID";
    case DPP_ERR_SHAPE: return "DPP_ERR_SHAPE";
    case DPP_ERR_UNSUPPORTED: return "DPP_ERR_UNSUPPORTED";
    case DPP_ERR_WORKSPACE: return "DPP_ERR_WORKSPACE";
    case DPP_ERR_HIP: return "DPP_ERR_HIP";
  }
  return "DPP_ERR_UNKNOWN";
}

extern "C" int32_t dpp_abi_version(void) { return 3; }
