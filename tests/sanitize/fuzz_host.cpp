// Randomised fuzz of libdpp's host code (planner and argument checks) and of the CPU oracle,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
// Every plan the planner accepts is checked against its contract: the workspace stays under
// the cap, every needed (row, split) of every request is covered by exactly one item of its
// tile per split, multi-split tiles own slot blocks inside their pass's partial region and
// single-split tiles none, the merge list agrees with the items. Malformed batches must be
// refused with a status. Exit status 0 means every check held (and the sanitizers found
// nothing, since they abort on the first finding).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "plan.h"

extern "C" {
int oracle_paged_prefill(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t page_size,
                         int32_t kv_dtype, double sm_scale, double k_scale, double v_scale,
                         const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* kv_last_page_len, const uint16_t* q, const void* k_pool,
                         const void* v_pool, int64_t n_sel, const int64_t* sel, int64_t key_lo,
                         int64_t key_hi, double* o, double* lse);
void oracle_merge_states(int64_t R, int32_t S, int32_t H, int32_t d, const double* o_part,
                         const double* lse_part, double* o, double* lse);
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "check failed: %s: ", #cond);  \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      ++failures;                                         \
    }                                                     \
  } while (0)

static void check_plan(const dpp_plan* p, const std::vector<int32_t>& qo, const std::vector<int32_t>& kvp,
                       const std::vector<int32_t>& last, int page, int group, size_t cap) {
  dpp_plan_info info{};
  CHECK(dpp_plan_get_info(p, &info) == DPP_OK, "info");
  if (cap) CHECK(info.workspace_bytes <= cap, "workspace %zu over cap %zu", info.workspace_bytes, cap);
  const int32_t* w = p->header.data();
  const dpp::HeaderPreamble* pre = reinterpret_cast<const dpp::HeaderPreamble*>(w);
  CHECK(pre->magic == dpp::kHeaderMagic, "magic");
  const auto* items = reinterpret_cast<const dpp::PrefillItem*>(w + pre->item_offset);
  const auto* merges = reinterpret_cast<const dpp::MergeItem*>(w + pre->merge_offset);
  const int bm = info.block_m, bn = info.block_n, tps = dpp::kSplitTokens / bn;
  const int B = (int)qo.size() - 1;
  // (request, row, split) -> count; tile -> (splits, slot base)
  std::map<std::tuple<int, int, int>, int> cov;
  std::map<std::pair<int, int>, std::pair<int, int>> tiles;
  for (int i = 0; i < pre->num_items; ++i) {
    const auto& it = items[i];
    CHECK(it.request >= 0 && it.request < B, "item request");
    if (it.request < 0 || it.request >= B) continue;
    const int qo_len = qo[it.request + 1] - qo[it.request];
    const int np = kvp[it.request + 1] - kvp[it.request];
    const int kv_len = page == 0 ? np : (np > 0 ? (np - 1) * page + last[it.request] : 0);
    CHECK(it.req.qo_len == qo_len && it.req.kv_len == kv_len, "descriptor copy");
    const int rows = std::min(bm, qo_len * group - it.row_start);
    CHECK(rows > 0, "empty tile");
    const int64_t pmax = (int64_t)kv_len - qo_len + (it.row_start + rows - 1) / group;
    CHECK(it.tile_splits == pmax / dpp::kSplitTokens + 1, "split count");
    CHECK(it.kv_tile_begin == it.split * tps && it.kv_tile_end <= (it.split + 1) * tps, "tile range");
    CHECK(it.pass >= 0 && it.pass < info.num_passes, "pass");
    if (it.tile_splits > 1) {
      const int64_t size = (int64_t)it.tile_splits * p->cfg.num_kv_heads * dpp::slot_rows_for(rows);
      CHECK(it.slot_base >= 0 && it.slot_base + size <= info.max_partial_slots, "slot block");
    } else {
      CHECK(it.slot_base == -1, "single-split slot");
    }
    auto key = std::make_pair(it.request, it.row_start);
    auto val = std::make_pair(it.tile_splits, it.slot_base);
    auto f = tiles.find(key);
    if (f == tiles.end()) tiles[key] = val; else CHECK(f->second == val, "tile items agree");
    for (int lr = 0; lr < rows; ++lr) cov[{it.request, it.row_start + lr, it.split}] += 1;
  }
  for (int r = 0; r < B; ++r) {
    const int qo_len = qo[r + 1] - qo[r];
    const int np = kvp[r + 1] - kvp[r];
    const int kv_len = page == 0 ? np : (np > 0 ? (np - 1) * page + last[r] : 0);
    for (int R = 0; R < qo_len * group; ++R) {
      const int pos = kv_len - qo_len + R / group;
      for (int s = 0; s <= pos / dpp::kSplitTokens; ++s) {
        auto c = cov.find({r, R, s});
        CHECK(c != cov.end() && c->second == 1, "row %d/%d split %d covered once", r, R, s);
      }
    }
  }
  int n_multi = 0;
  for (auto& t : tiles) n_multi += t.second.first > 1;
  CHECK(n_multi == pre->num_merges, "merge count %d vs %d", n_multi, pre->num_merges);
  for (int m = 0; m < pre->num_merges; ++m) {
    auto f = tiles.find({merges[m].request, merges[m].row_start});
    CHECK(f != tiles.end() && f->second == std::make_pair(merges[m].tile_splits, merges[m].slot_base), "merge item");
  }
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937_64 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int dims[] = {64, 128, 256, 512};
  const int pages[] = {0, 1, 5, 16, 64, 1024};
  int accepted = 0, refused = 0;
  for (int round = 0; round < rounds; ++round) {
    dpp_config c{};
    c.num_kv_heads = 1 << uni(0, 3);
    const int group = uni(1, 8);
    c.num_qo_heads = c.num_kv_heads * group;
    c.head_dim = dims[uni(0, 3)];
    c.page_size = pages[uni(0, 5)];
    c.kv_dtype = uni(0, 1);
    c.sm_scale = 0.f;
    c.k_scale = c.v_scale = 0.5f;
    const int B = uni(0, 24);
    std::vector<int32_t> qo{0}, kvp{0}, last;
    bool malformed = false;
    for (int r = 0; r < B; ++r) {
      int kv = uni(0, 3) == 0 ? uni(0, 40) : (uni(0, 1) ? uni(0, 3000) : uni(3000, 20000));
      int ql = uni(0, 2) == 0 ? kv : std::min(kv, uni(0, 40));
      const int P = c.page_size == 0 ? 1 : c.page_size;
      int np = c.page_size == 0 ? kv : (kv + P - 1) / P;
      int lp = c.page_size == 0 ? 0 : (np > 0 ? kv - (np - 1) * P : 0);
      if (uni(0, 40) == 0) { ql = kv + 1; malformed = true; }                          // qo_len > kv_len
      if (c.page_size && np > 0 && uni(0, 40) == 0) { lp = P + 1; malformed = true; }  // bad last page
      qo.push_back(qo.back() + ql);
      kvp.push_back(kvp.back() + np);
      last.push_back(lp);
    }
    size_t cap = 0;
    switch (uni(0, 3)) {
      case 0: cap = 0; break;
      case 1: cap = (size_t)uni(1, 64) << 20; break;
      case 2: cap = (size_t)uni(1, 4096) << 10; break;
      default: cap = 256u << 20; break;
    }
    uint32_t flags = uni(0, 3) == 0 ? (DPP_PLAN_PERMUTE_WORK | DPP_PLAN_PERMUTE_SEED(uni(0, 65535))) : 0u;
    if (uni(0, 5) == 0) flags |= DPP_PLAN_ADAPTIVE_KV_TILE;
    dpp_plan* p = nullptr;
    const dpp_status st = dpp_plan_create_ex(&c, B, qo.data(), kvp.data(), last.data(), cap, flags, &p);
    if (malformed) CHECK(st != DPP_OK, "malformed batch accepted");
    if (st != DPP_OK) {
      CHECK(p == nullptr && std::strlen(dpp_last_error()) > 0, "refusal leaves no plan and a message");
      ++refused;
      continue;
    }
    ++accepted;
    check_plan(p, qo, kvp, last, c.page_size, group, cap);
    // page-table check: valid ids pass, one id out of range is named, a short list is refused
    const int64_t n_ids = kvp.back();
    std::vector<int32_t> ids((size_t)n_ids + 3);
    for (auto& x : ids) x = uni(0, 999);
    if (c.page_size != 0) {
      CHECK(dpp_check_page_table(p, ids.data(), n_ids, 1000) == DPP_OK, "valid ids");
      if (n_ids > 0) {
        ids[(size_t)uni(0, (int)n_ids - 1)] = uni(0, 1) ? -1 : 1000;
        CHECK(dpp_check_page_table(p, ids.data(), n_ids, 1000) == DPP_ERR_SHAPE, "bad id");
        CHECK(dpp_check_page_table(p, ids.data(), n_ids - 1, 1000) == DPP_ERR_SHAPE, "short list");
      }
    }
    // run-argument checks (host only)
    alignas(256) static unsigned char dummy[1024];
    const int64_t rows = qo.back();
    CHECK(dpp::check_run_args(p, "fuzz", dummy, rows + 1, dummy, dummy, 10, (const int32_t*)dummy, n_ids,
                              dummy, (const float*)dummy, 0) == DPP_ERR_SHAPE, "row count");
    CHECK(dpp::check_run_args(p, "fuzz", dummy, rows, dummy, dummy, 10, (const int32_t*)dummy, n_ids,
                              dummy, (const float*)dummy, 8) == DPP_ERR_INVALID, "flags");
    delete p;
  }
  // the oracle on small random batches, with row subsets and key ranges (bf16 and fp8 pools)
  for (int round = 0; round < 60; ++round) {
    const int hkv = 1 << uni(0, 2), g = uni(1, 4), hq = hkv * g, d = 8 * uni(1, 8), P = uni(1, 9);
    const int kv_dtype = uni(0, 1), B = uni(1, 5);
    std::vector<int32_t> qo{0}, kvp{0}, last, ids;
    int pages = 0;
    for (int r = 0; r < B; ++r) {
      const int kv = uni(0, 40), ql = uni(0, kv);
      const int np = (kv + P - 1) / P;
      qo.push_back(qo.back() + ql);
      kvp.push_back(kvp.back() + np);
      last.push_back(np ? kv - (np - 1) * P : 0);
      for (int j = 0; j < np; ++j) ids.push_back(pages++);
    }
    const int nq = qo.back();
    std::vector<uint16_t> q((size_t)nq * hq * d + 1);
    for (auto& x : q) x = (uint16_t)(0x3F00 + uni(0, 255) - 128 * uni(0, 1) * 0);  // bf16 near 0.5..1
    const size_t pool = (size_t)(pages + 1) * P * hkv * d;
    std::vector<uint16_t> kb(pool), vb(pool);
    std::vector<uint8_t> k8(pool), v8(pool);
    for (size_t i = 0; i < pool; ++i) {
      kb[i] = (uint16_t)(0x3C00 + uni(0, 511)); vb[i] = (uint16_t)(0xBC00 + uni(0, 511));
      k8[i] = (uint8_t)uni(0, 0x6F); v8[i] = (uint8_t)(0x80 | uni(0, 0x6F));
    }
    std::vector<int64_t> sel;
    for (int i = 0; i < nq; i += uni(1, 3)) sel.push_back(uni(0, nq - 1));
    const int n = (int)sel.size();
    std::vector<double> o((size_t)std::max(n, 1) * hq * d), lse((size_t)std::max(n, 1) * hq);
    const void* K = kv_dtype ? (const void*)k8.data() : (const void*)kb.data();
    const void* V = kv_dtype ? (const void*)v8.data() : (const void*)vb.data();
    int rc = oracle_paged_prefill(B, hq, hkv, d, P, kv_dtype, 0.3, 0.25, 0.5, qo.data(), kvp.data(), ids.data(),
                                  last.data(), q.data(), K, V, n, n ? sel.data() : nullptr, uni(0, 8), uni(0, 1) ? -1 : uni(8, 40),
                                  o.data(), lse.data());
    CHECK(rc == 0, "oracle rc");
    for (int i = 0; i < n * hq * d; ++i) CHECK(std::isfinite(o[(size_t)i]), "oracle o finite");
    // merge of two random partial sets
    const int R = uni(1, 4), S = uni(1, 6);
    std::vector<double> op((size_t)R * S * hq * d), lp((size_t)R * S * hq), om((size_t)R * hq * d), lm((size_t)R * hq);
    for (auto& x : op) x = uni(-100, 100) / 50.0;
    for (auto& x : lp) x = uni(0, 4) == 0 ? -INFINITY : uni(-300, 300) / 30.0;
    oracle_merge_states(R, S, hq, d, op.data(), lp.data(), om.data(), lm.data());
  }
  std::printf("fuzz: %d plans accepted, %d refused, %d failed checks\n", accepted, refused, failures);
  return failures == 0 ? 0 : 1;
}
