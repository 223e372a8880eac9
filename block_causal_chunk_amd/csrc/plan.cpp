// plan.cpp -- validation and scheduling for block-causal chunk attention (host only, no HIP).
//
// The visible key set of query chunk a is every chunk b with order[b] <= order[a] (Wave Forcing
// project page, "01 - The design gap", directed frontier and "Key observation").  Sorting the
// chunks clean -> noisy makes that set a prefix of one key-tile list, which is how the consumer
// reads its prefix in place (project page, "03 - End-to-end KV transport", "Layout" panel).
// Query tiles never cross a chunk and key tiles never cross a page, so every (query tile, key
// tile) pair is either fully visible or never enumerated: masked tiles are never loaded.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>
#include <queue>

#include "plan.hpp"

namespace wfattn {
namespace {

std::atomic<uint64_t> g_nonce{0x5eed0001ull};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Item {
  int32_t head, q_row0, rows, kt_begin, kt_end, slot, qsb, qchunk;
  int64_t cost() const { return kt_end - kt_begin; }
};

wfattn_status validate(const wfattn_chunk_table* t) {
  if (!t->chunk_tokens || !t->chunk_order || !t->page_offsets || !t->page_ids || !t->query_chunks)
    return WFATTN_ERR_NULL;
  if (t->num_chunks < 1 || t->num_heads < 1 || t->num_query_chunks < 1 || t->page_size < 1 ||
      t->num_pages < 1)
    return WFATTN_ERR_INVALID;
  if (!std::isfinite(t->softmax_scale)) return WFATTN_ERR_INVALID;
  if (t->head_dim != 64 && t->head_dim != 128) return WFATTN_ERR_UNSUPPORTED;
  if (t->page_size % 64 != 0) return WFATTN_ERR_UNSUPPORTED;
  const int n = t->num_chunks;
  std::vector<char> seen(n, 0);
  for (int c = 0; c < n; ++c) {
    if (t->chunk_tokens[c] < 1) return WFATTN_ERR_INVALID;
    const int o = t->chunk_order[c];
    if (o < 0 || o >= n || seen[o]) return WFATTN_ERR_INVALID;  // not a permutation
    seen[o] = 1;
  }
  if (t->page_offsets[0] != 0) return WFATTN_ERR_INVALID;
  for (int c = 0; c < n; ++c) {
    const int64_t want = (static_cast<int64_t>(t->chunk_tokens[c]) + t->page_size - 1) / t->page_size;
    if (static_cast<int64_t>(t->page_offsets[c + 1]) - t->page_offsets[c] != want)
      return WFATTN_ERR_INVALID;
  }
  const int64_t logical = t->page_offsets[n];
  if (static_cast<int64_t>(t->num_pages) * t->page_size > INT32_MAX) return WFATTN_ERR_RANGE;
  std::vector<char> used(t->num_pages, 0);
  for (int64_t p = 0; p < logical; ++p) {
    const int32_t id = t->page_ids[p];
    if (id < 0 || id >= t->num_pages || used[id]) return WFATTN_ERR_RANGE;
    used[id] = 1;
  }
  std::vector<char> isq(n, 0);
  int64_t lq = 0;
  for (int i = 0; i < t->num_query_chunks; ++i) {
    const int a = t->query_chunks[i];
    if (a < 0 || a >= n || isq[a]) return WFATTN_ERR_INVALID;
    isq[a] = 1;
    lq += t->chunk_tokens[a];
  }
  if (lq > INT32_MAX) return WFATTN_ERR_RANGE;
  return WFATTN_OK;
}

// Greedy list scheduling of `costs` (in launch order) onto `slots` identical slots: an estimate
// of the makespan the hardware dispatcher reaches when it hands each next workgroup to the first
// slot that frees up.
int64_t makespan(const std::vector<int64_t>& costs, int slots) {
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> q;
  for (int i = 0; i < slots; ++i) q.push(0);
  int64_t worst = 0;
  for (int64_t c : costs) {
    int64_t t = q.top() + c;
    q.pop();
    q.push(t);
    worst = std::max(worst, t);
  }
  return worst;
}

constexpr int kCUs = 256;        // MI355X compute units
constexpr int kXCDs = 8;         // dies; workgroup i starts on XCD i % 8
constexpr int kWgPerCU = 2;      // resident attention workgroups per CU

}  // namespace
}  // namespace wfattn

using namespace wfattn;

extern "C" wfattn_status wfattn_plan(const wfattn_chunk_table* table, const wfattn_opts* opts,
                                     wfattn_plan_t** plan_out) {
  if (!table || !plan_out) return WFATTN_ERR_NULL;
  wfattn_opts o{};
  if (opts) o = *opts;
  if (o.reserved0 != 0 || o.reserved1 != 0 || o.split_k < 0 || o.split_k > 64 ||
      o.xcd_remap < -1 || o.xcd_remap > 1)
    return WFATTN_ERR_UNSUPPORTED;
  wfattn_status st = validate(table);
  if (st != WFATTN_OK) return st;

  wfattn_plan_s* ps = new (std::nothrow) wfattn_plan_s();
  if (!ps) return WFATTN_ERR_NOMEM;
  Plan& P = ps->impl;
  try {
    const int n = table->num_chunks;
    P.nonce = g_nonce.fetch_add(0x9E3779B97F4A7C15ull) ^ reinterpret_cast<uintptr_t>(ps);
    P.num_chunks = n;
    P.num_heads = table->num_heads;
    P.head_dim = table->head_dim;
    P.page_size = table->page_size;
    P.num_pages = table->num_pages;
    P.num_query_chunks = table->num_query_chunks;
    P.pool_rows = static_cast<int64_t>(table->num_pages) * table->page_size;
    P.scale = table->softmax_scale > 0.f ? table->softmax_scale
                                         : static_cast<float>(1.0 / std::sqrt((double)table->head_dim));
    P.xcd_remap = (o.xcd_remap == -1) ? 0 : 1;

    // Key tiles of all chunks, clean -> noisy; prefix_end[c] = tiles up to and including c.
    std::vector<int> by_order(n);
    for (int c = 0; c < n; ++c) by_order[table->chunk_order[c]] = c;
    std::vector<int32_t> tiles;
    std::vector<int32_t> prefix_end(n, 0);
    for (int r = 0; r < n; ++r) {
      const int c = by_order[r];
      const int32_t tok = table->chunk_tokens[c];
      for (int32_t p = table->page_offsets[c]; p < table->page_offsets[c + 1]; ++p) {
        const int32_t first_tok = (p - table->page_offsets[c]) * table->page_size;
        const int32_t valid = std::min(table->page_size, tok - first_tok);
        const int32_t base = table->page_ids[p] * table->page_size;
        for (int32_t off = 0; off < valid; off += kBlockN) {
          tiles.push_back(base + off);
          tiles.push_back(std::min(kBlockN, valid - off));
        }
      }
      prefix_end[c] = static_cast<int32_t>(tiles.size() / kTileInts);
    }
    P.n_tiles = static_cast<int32_t>(tiles.size() / kTileInts);

    // Base items: (query chunk, query tile, head) with the whole visible prefix.
    std::vector<Item> base;
    int64_t row0 = 0, qsb0 = 0;
    for (int i = 0; i < table->num_query_chunks; ++i) {
      const int a = table->query_chunks[i];
      const int32_t tok = table->chunk_tokens[a];
      for (int32_t qt = 0; qt * kBlockM < tok; ++qt) {
        const int32_t rows = std::min(kBlockM, tok - qt * kBlockM);
        for (int32_t h = 0; h < table->num_heads; ++h)
          base.push_back(Item{h, static_cast<int32_t>(row0 + qt * kBlockM), rows, 0, prefix_end[a],
                              -1, static_cast<int32_t>(qsb0 + qt * (kBlockM / 64)), i});
      }
      row0 += tok;
      qsb0 += (tok + 63) / 64;
    }
    P.lq = row0;
    P.nqb = qsb0;

    // Split-K: explicit, or the count that minimises the estimated makespan plus merge cost.
    const int slots = kCUs * kWgPerCU;
    auto split_items = [&](int s) {
      std::vector<Item> out;
      out.reserve(base.size() * s);
      for (const Item& it : base) {
        const int32_t nt = it.kt_end - it.kt_begin;
        const int parts = std::max(1, std::min<int>(s, nt));
        for (int k = 0; k < parts; ++k) {
          Item x = it;
          x.kt_begin = it.kt_begin + static_cast<int32_t>(static_cast<int64_t>(nt) * k / parts);
          x.kt_end = it.kt_begin + static_cast<int32_t>(static_cast<int64_t>(nt) * (k + 1) / parts);
          out.push_back(x);
        }
      }
      return out;
    };
    auto lpt = [](std::vector<Item>& v) {
      std::stable_sort(v.begin(), v.end(), [](const Item& a, const Item& b) { return a.cost() > b.cost(); });
    };
    int splits = 1;
    if (o.split_k >= 1) {
      splits = o.split_k;
    } else {
      // Each split adds a merge pass over its partial tile; price it at ~2 key tiles.
      double best = 1e300;
      for (int s = 1; s <= 8; ++s) {
        std::vector<Item> v = split_items(s);
        lpt(v);
        std::vector<int64_t> costs;
        costs.reserve(v.size());
        for (auto& it : v) costs.push_back(it.cost() + 1);  // +1: per-item prologue/epilogue
        const double est = static_cast<double>(makespan(costs, slots)) + (s > 1 ? 2.0 * s : 0.0);
        if (est < best * 0.97) {  // prefer fewer splits unless clearly better
          best = est;
          splits = s;
        }
      }
    }
    std::vector<Item> items = split_items(splits);
    P.splits = splits;

    // Partial slots and merge groups for the split items (items of one base are consecutive).
    std::vector<int32_t> groups;
    {
      size_t i = 0;
      int32_t slot = 0;
      while (i < items.size()) {
        size_t j = i + 1;
        while (j < items.size() && items[j].head == items[i].head && items[j].q_row0 == items[i].q_row0 &&
               items[j].kt_begin == items[j - 1].kt_end)
          ++j;
        if (j - i > 1) {
          groups.insert(groups.end(), {items[i].head, items[i].q_row0, items[i].rows, slot,
                                       static_cast<int32_t>(j - i), 0, 0, 0});
          for (size_t k = i; k < j; ++k) items[k].slot = slot++;
        }
        i = j;
      }
      P.n_partials = slot;
      P.n_groups = static_cast<int32_t>(groups.size() / kGroupInts);
    }

    // Launch order.  XCD-aware: split the head-major item list into 8 contiguous ranges of equal
    // cost, one per XCD (so each XCD streams the K/V of few heads through its own L2), order each
    // range longest-first, and interleave them so that workgroup 8*j + x is the j-th item of XCD x.
    std::vector<Item> launch;
    if (P.xcd_remap) {
      std::vector<Item> hm = items;
      std::stable_sort(hm.begin(), hm.end(), [](const Item& a, const Item& b) {
        if (a.head != b.head) return a.head < b.head;
        return a.q_row0 < b.q_row0;
      });
      int64_t total = 0;
      for (auto& it : hm) total += it.cost() + 1;
      std::vector<std::vector<Item>> per(kXCDs);
      int64_t acc = 0;
      for (auto& it : hm) {
        int x = static_cast<int>(std::min<int64_t>(kXCDs - 1, (acc * kXCDs + (it.cost() + 1) / 2) / std::max<int64_t>(total, 1)));
        per[x].push_back(it);
        acc += it.cost() + 1;
      }
      size_t longest = 0;
      for (auto& v : per) {
        lpt(v);
        longest = std::max(longest, v.size());
      }
      for (size_t j = 0; j < longest; ++j)
        for (int x = 0; x < kXCDs; ++x) {
          if (j < per[x].size()) launch.push_back(per[x][j]);
          else launch.push_back(Item{-1, 0, 0, 0, 0, -1, 0, -1});  // idle slot keeps the stride
        }
      // drop trailing idle items
      while (!launch.empty() && launch.back().head < 0) launch.pop_back();
    } else {
      launch = items;
      lpt(launch);
    }
    P.n_items = static_cast<int32_t>(launch.size());

    // Blob: header, items, tiles, groups.
    P.off_items = kHeaderInts;
    P.off_tiles = P.off_items + static_cast<size_t>(P.n_items) * kItemInts;
    P.off_groups = P.off_tiles + tiles.size();
    P.blob.assign(P.off_groups + groups.size(), 0);
    P.blob[H_MAGIC] = static_cast<int32_t>(kMagic);
    P.blob[H_NONCE_LO] = static_cast<int32_t>(P.nonce & 0xffffffffu);
    P.blob[H_NONCE_HI] = static_cast<int32_t>(P.nonce >> 32);
    P.blob[H_ITEMS] = P.n_items;
    P.blob[H_TILES] = P.n_tiles;
    P.blob[H_GROUPS] = P.n_groups;
    P.blob[H_OFF_ITEMS] = static_cast<int32_t>(P.off_items);
    P.blob[H_OFF_TILES] = static_cast<int32_t>(P.off_tiles);
    P.blob[H_OFF_GROUPS] = static_cast<int32_t>(P.off_groups);
    for (size_t i = 0; i < launch.size(); ++i) {
      const Item& it = launch[i];
      int32_t* d = &P.blob[P.off_items + i * kItemInts];
      d[0] = it.head; d[1] = it.q_row0; d[2] = it.rows; d[3] = it.kt_begin;
      d[4] = it.kt_end; d[5] = it.slot; d[6] = it.qsb; d[7] = it.qchunk;
    }
    std::copy(tiles.begin(), tiles.end(), P.blob.begin() + P.off_tiles);
    std::copy(groups.begin(), groups.end(), P.blob.begin() + P.off_groups);

    // Workspace layout.
    const size_t D = static_cast<size_t>(P.head_dim);
    P.ws_blob = 0;
    size_t off = align_up(P.blob.size() * sizeof(int32_t), 256);
    P.ws_part_o = off;
    off = align_up(off + static_cast<size_t>(P.n_partials) * kBlockM * D * sizeof(float), 256);
    P.ws_part_lse = off;
    off = align_up(off + static_cast<size_t>(P.n_partials) * kBlockM * sizeof(float), 256);
    P.ws_base_bytes = off;
    const size_t pool_elems = static_cast<size_t>(P.pool_rows) * P.num_heads * D;
    const size_t q_elems = static_cast<size_t>(P.lq) * P.num_heads * D;
    P.stage_q_off = off;
    off = align_up(off + q_elems * 2, 256);
    P.stage_k_off = off;
    off = align_up(off + pool_elems * 2, 256);
    P.stage_v_off = off;
    off = align_up(off + pool_elems * 2, 256);
    P.ws_fp32_bytes = off;
  } catch (const std::bad_alloc&) {
    delete ps;
    return WFATTN_ERR_NOMEM;
  }
  *plan_out = ps;
  return WFATTN_OK;
}

extern "C" void wfattn_plan_free(wfattn_plan_t* plan) {
  if (plan_ok(plan)) {
    plan->impl.magic = 0;
    delete plan;
  }
}

extern "C" int64_t wfattn_query_rows(const wfattn_plan_t* plan) {
  return plan_ok(plan) ? as_plan(plan)->lq : -1;
}

extern "C" size_t wfattn_workspace_bytes(const wfattn_plan_t* plan, int32_t mode) {
  if (!plan_ok(plan)) return 0;
  const Plan* P = as_plan(plan);
  switch (mode) {
    case WFATTN_WS_BF16:
    case WFATTN_WS_FP8:
      return P->ws_base_bytes;
    case WFATTN_WS_FP32:
      return P->ws_fp32_bytes;
    default:
      return 0;
  }
}

extern "C" wfattn_status wfattn_plan_describe(const wfattn_plan_t* plan, int32_t what, int32_t* buf,
                                              size_t cap, size_t* n) {
  if (!plan || !n || (cap > 0 && !buf)) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  const Plan* P = as_plan(plan);
  std::vector<int32_t> tmp;
  const int32_t* src = nullptr;
  size_t total = 0;
  switch (what) {
    case 0:
      tmp = {P->n_items, P->n_tiles, P->n_groups, P->n_partials, P->block_m, P->block_n, P->splits,
             P->num_query_chunks};
      src = tmp.data();
      total = tmp.size();
      break;
    case 1:
      src = P->blob.data() + P->off_items;
      total = static_cast<size_t>(P->n_items) * kItemInts;
      break;
    case 2:
      src = P->blob.data() + P->off_tiles;
      total = static_cast<size_t>(P->n_tiles) * kTileInts;
      break;
    case 3:
      src = P->blob.data() + P->off_groups;
      total = static_cast<size_t>(P->n_groups) * kGroupInts;
      break;
    default:
      return WFATTN_ERR_INVALID;
  }
  if (cap > 0) std::memcpy(buf, src, std::min(cap, total) * sizeof(int32_t));
  *n = total;
  return WFATTN_OK;
}

extern "C" const char* wfattn_status_str(wfattn_status s) {
  switch (s) {
    case WFATTN_OK: return "ok";
    case WFATTN_ERR_NULL: return "null pointer";
    case WFATTN_ERR_INVALID: return "invalid chunk table or plan";
    case WFATTN_ERR_RANGE: return "value out of range";
    case WFATTN_ERR_UNSUPPORTED: return "unsupported argument";
    case WFATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case WFATTN_ERR_DEVICE: return "HIP device error";
    case WFATTN_ERR_NOMEM: return "out of host memory";
  }
  return "unknown status";
}

extern "C" int32_t wfattn_abi_version(void) { return 1; }
