// Drives the host planner (plan.cpp) over seeded random chunk tables, well-formed and corrupted,
// with every option combination, and reads back every description.  Built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py (host code only, no GPU), so an
// out-of-bounds access, leak, overflow or misaligned read in the planner ends the run.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

#include "wfattn.h"

int main() {
  std::mt19937 rng(20241203u);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int planned = 0, refused = 0;
  for (int it = 0; it < 400; ++it) {
    const int n = uni(1, 8);
    const int page = 64 << uni(0, 3);
    const bool ties = uni(0, 1);
    std::vector<int32_t> tokens(n), order(n), offs(n + 1, 0);
    for (int c = 0; c < n; ++c) tokens[c] = uni(0, 2) == 0 ? uni(1, 64) : uni(65, 1200);
    if (ties) {
      for (int c = 0; c < n; ++c) order[c] = uni(0, n - 1);
    } else {
      std::iota(order.begin(), order.end(), 0);
      std::shuffle(order.begin(), order.end(), rng);
    }
    for (int c = 0; c < n; ++c) offs[c + 1] = offs[c] + (tokens[c] + page - 1) / page;
    const int spare = uni(0, 3);
    std::vector<int32_t> perm(offs[n] + spare);
    std::iota(perm.begin(), perm.end(), 0);
    std::shuffle(perm.begin(), perm.end(), rng);
    std::vector<int32_t> ids(perm.begin(), perm.begin() + offs[n]);
    std::vector<int32_t> q(n);
    std::iota(q.begin(), q.end(), 0);
    std::shuffle(q.begin(), q.end(), rng);
    q.resize(uni(1, n));
    wfattn_chunk_table t{};
    t.num_chunks = n;
    t.chunk_tokens = tokens.data();
    t.chunk_order = order.data();
    t.page_offsets = offs.data();
    t.page_ids = ids.data();
    t.num_pages = (int32_t)perm.size();
    t.page_size = page;
    t.num_query_chunks = (int32_t)q.size();
    t.query_chunks = q.data();
    t.num_heads = uni(1, 40);
    t.head_dim = uni(0, 1) ? 128 : 64;
    t.softmax_scale = uni(0, 1) ? 0.f : 0.07f;
    switch (uni(0, 9)) {  // some tables are corrupted in one field
      case 0: tokens[uni(0, n - 1)] = 0; break;
      case 1: if (!ids.empty()) ids[uni(0, (int)ids.size() - 1)] = t.num_pages; break;
      case 2: if (ids.size() > 1) ids[1] = ids[0]; break;
      case 3: order[uni(0, n - 1)] = n; break;
      case 4: q.push_back(q[0]); t.num_query_chunks = (int32_t)q.size(); t.query_chunks = q.data(); break;
      case 5: t.head_dim = 96; break;
      case 6: t.page_size = 96; break;
      default: break;
    }
    wfattn_opts o{};
    const int splits[] = {0, 1, 3, 7, 64};
    o.split_k = splits[uni(0, 4)];
    o.xcd_remap = uni(-1, 1);
    o.order_ties = ties ? 1 : uni(0, 1);
    wfattn_plan_t* p = nullptr;
    const wfattn_status st = wfattn_plan(&t, &o, &p);
    if (st != WFATTN_OK) {
      if (p != nullptr) { std::printf("plan written on error\n"); return 1; }
      ++refused;
      continue;
    }
    ++planned;
    int64_t lq = 0;
    for (int a : q) lq += tokens[a];
    if (wfattn_query_rows(p) != lq) { std::printf("query rows\n"); return 1; }
    for (int mode = 0; mode < 3; ++mode)
      if (wfattn_workspace_bytes(p, mode) == 0) { std::printf("workspace\n"); return 1; }
    for (int what = 0; what <= 6; ++what) {
      size_t total = 0;
      if (wfattn_plan_describe(p, what, nullptr, 0, &total) != WFATTN_OK) { std::printf("describe\n"); return 1; }
      std::vector<int32_t> buf(total + 1);
      size_t again = 0;
      if (wfattn_plan_describe(p, what, buf.data(), total, &again) != WFATTN_OK || again != total) return 1;
      if (total > 2) wfattn_plan_describe(p, what, buf.data(), total / 2, &again);  // a short buffer
    }
    size_t dummy = 0;
    if (wfattn_plan_describe(p, 7, nullptr, 0, &dummy) == WFATTN_OK) { std::printf("what 7\n"); return 1; }
    wfattn_plan_free(p);
  }
  wfattn_plan_free(nullptr);
  std::printf("OK planned %d refused %d\n", planned, refused);
  return (planned > 50 && refused > 20) ? 0 : 1;
}
