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
  int32_t head, q_row0, rows, qsb, qchunk, n_tiles;
};

struct Seg {
  int32_t item, kt0, kt1, slot;
};

wfattn_status validate(const wfattn_chunk_table* t, bool ties) {
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
    if (o < 0 || o >= n || (seen[o] && !ties)) return WFATTN_ERR_INVALID;  // not a permutation
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

constexpr int kCUs = 256;      // MI355X compute units (the default); workgroup w starts on XCD w % 8
constexpr int kXCDs = 8;
constexpr int kSegOverhead = 3; // a segment's Q load + epilogue, in key-tile units
constexpr int kMinSplit = 8;    // never cut a segment shorter than this many key tiles

// Longest-processing-time list scheduling of whole segments onto `bins` workgroups: returns
// per-bin segment lists (longest first) and the makespan in key-tile units.
int64_t lpt(const std::vector<Seg>& segs, int bins, std::vector<std::vector<int>>& out) {
  std::vector<int> order(segs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return segs[a].kt1 - segs[a].kt0 > segs[b].kt1 - segs[b].kt0;
  });
  out.assign(bins, {});
  typedef std::pair<int64_t, int> Load;
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> q;
  for (int b = 0; b < bins; ++b) q.push(Load(0, b));
  int64_t worst = 0;
  for (int i : order) {
    Load l = q.top();
    q.pop();
    l.first += segs[i].kt1 - segs[i].kt0 + kSegOverhead;
    out[l.second].push_back(i);
    worst = std::max(worst, l.first);
    q.push(l);
  }
  return worst;
}

}  // namespace
}  // namespace wfattn

using namespace wfattn;

extern "C" wfattn_status wfattn_plan(const wfattn_chunk_table* table, const wfattn_opts* opts,
                                     wfattn_plan_t** plan_out) {
  if (!table || !plan_out) return WFATTN_ERR_NULL;
  wfattn_opts o{};
  if (opts) o = *opts;
  if (o.order_ties < 0 || o.order_ties > 1 || o.split_k < 0 || o.split_k > 64 || o.xcd_remap < -1 ||
      o.xcd_remap > 1 || o.num_cus < 0 || o.num_cus > 4096 || o.num_xcds < 0 ||
      (o.block_m != 0 && o.block_m != kBlockM) || (o.block_n != 0 && o.block_n != kBlockN))
    return WFATTN_ERR_UNSUPPORTED;
  const int32_t n_cus = o.num_cus ? o.num_cus : kCUs;
  const int32_t n_xcds = o.num_xcds ? o.num_xcds : (o.num_cus ? 1 : kXCDs);
  if (n_xcds > n_cus || n_cus % n_xcds != 0) return WFATTN_ERR_UNSUPPORTED;
  wfattn_status st = validate(table, o.order_ties == 1);
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
    P.n_cus = n_cus;
    P.n_xcds = n_xcds;
    const int CU = n_cus, XCD = n_xcds;

    // Key tiles of all chunks, clean -> noisy (chunks of equal order by index); prefix_end[c] =
    // tiles up to and including the last chunk whose order is not above c's, so the visible keys
    // of every query chunk are a prefix of this list.
    std::vector<int> by_order(n);
    std::iota(by_order.begin(), by_order.end(), 0);
    std::stable_sort(by_order.begin(), by_order.end(),
                     [&](int x, int y) { return table->chunk_order[x] < table->chunk_order[y]; });
    std::vector<int32_t> tiles;
    std::vector<int32_t> prefix_end(n, 0), first_tile(n, 0), rank(n, 0), last_rank(n, 0);
    for (int r = 0; r < n; ++r) {
      const int c = by_order[r];
      first_tile[c] = static_cast<int32_t>(tiles.size() / kTileInts);
      rank[c] = last_rank[c] = r;
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
    for (int r = n - 2; r >= 0; --r)  // a tie group ends where its last member ends
      if (table->chunk_order[by_order[r]] == table->chunk_order[by_order[r + 1]]) {
        prefix_end[by_order[r]] = prefix_end[by_order[r + 1]];
        last_rank[by_order[r]] = last_rank[by_order[r + 1]];
      }
    P.n_tiles = static_cast<int32_t>(tiles.size() / kTileInts);
    for (int i = 0; i < table->num_query_chunks; ++i)
      P.n_vis_tiles = std::max(P.n_vis_tiles, prefix_end[table->query_chunks[i]]);

    // Items: (query chunk, query tile of up to kBlockM rows, head) with the whole visible prefix.
    std::vector<Item> items;
    int64_t row0 = 0, qsb0 = 0;
    for (int i = 0; i < table->num_query_chunks; ++i) {
      const int a = table->query_chunks[i];
      const int32_t tok = table->chunk_tokens[a];
      for (int32_t h = 0; h < table->num_heads; ++h)
        for (int32_t qt = 0; qt * kBlockM < tok; ++qt)
          items.push_back(Item{h, static_cast<int32_t>(row0 + qt * kBlockM), std::min(kBlockM, tok - qt * kBlockM),
                               static_cast<int32_t>(qsb0 + qt * (kBlockM / 64)), i, prefix_end[a]});
      row0 += tok;
      qsb0 += (tok + 63) / 64;
    }
    // head-major order: consecutive items read the same K/V
    std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
      return x.head != y.head ? x.head < y.head : x.q_row0 < y.q_row0;
    });
    P.lq = row0;
    P.nqb = qsb0;
    const int n_items = static_cast<int>(items.size());

    // Segments (a key range of one item) and the workgroup that runs each.
    std::vector<Seg> segs;
    std::vector<std::vector<int>> per_wg;  // segment indices per workgroup, in run order
    int64_t total = 0;
    for (const Item& it : items) total += it.n_tiles;
    auto whole_items_lpt = [&](int parts) {
      segs.clear();
      for (int i = 0; i < n_items; ++i) {
        const int32_t nt = items[i].n_tiles;
        const int k = std::max(1, std::min(parts, nt));
        for (int j = 0; j < k; ++j)
          segs.push_back(Seg{i, static_cast<int32_t>(static_cast<int64_t>(nt) * j / k),
                             static_cast<int32_t>(static_cast<int64_t>(nt) * (j + 1) / k), -1});
      }
      const int n_segs = static_cast<int>(segs.size());
      if (n_segs <= CU && P.xcd_remap) {
        // one segment per workgroup: the head-major segment list laid out XCD by XCD, so the
        // workgroups of one XCD walk the same heads' keys side by side and share them in L2
        per_wg.assign(CU, {});
        int64_t worst = 0;
        for (int L = 0; L < n_segs; ++L) {
          per_wg[(L / (CU / XCD)) + XCD * (L % (CU / XCD))].push_back(L);
          worst = std::max<int64_t>(worst, segs[L].kt1 - segs[L].kt0 + kSegOverhead);
        }
        return worst;
      }
      const int bins = std::min<int>(CU, n_segs);
      return lpt(segs, bins, per_wg);
    };
    // Stream-K: the head-major list of key tiles cut into CU ranges of equal cost; logical range L
    // runs on workgroup (L / (CU/XCD)) + XCD * (L % (CU/XCD)) (on MI355X (L / 32) + 8 * (L % 32)),
    // so the workgroups of one XCD share a contiguous run of heads and hence their K/V in its L2.
    auto stream_k = [&]() {
      const int G = CU;
      segs.clear();
      per_wg.assign(G, {});
      // item i owns tiles [first[i], first[i] + n_tiles) of one global axis; logical range L is
      // [cut[L], cut[L+1]); a cut closer than kMinSplit to an item boundary snaps to it
      std::vector<int64_t> first(n_items + 1, 0);
      for (int i = 0; i < n_items; ++i) first[i + 1] = first[i] + items[i].n_tiles;
      std::vector<int64_t> cut(G + 1);
      int it_idx = 0;
      for (int L = 0; L <= G; ++L) {
        int64_t c = (total * L + G / 2) / G;
        while (it_idx < n_items && first[it_idx + 1] <= c) ++it_idx;
        if (L > 0 && L < G && it_idx < n_items) {
          if (c - first[it_idx] < kMinSplit) c = first[it_idx];
          else if (first[it_idx + 1] - c < kMinSplit) c = first[it_idx + 1];
        }
        cut[L] = (L == 0) ? 0 : std::max(c, cut[L - 1]);
      }
      cut[G] = total;
      int i = 0;
      for (int L = 0; L < G; ++L) {
        const int w = P.xcd_remap ? (L / (G / XCD)) + XCD * (L % (G / XCD)) : L;
        while (i < n_items && first[i + 1] <= cut[L]) ++i;
        for (int j = i; j < n_items && first[j] < cut[L + 1]; ++j) {
          const int64_t a = std::max(cut[L], first[j]), b = std::min(cut[L + 1], first[j + 1]);
          if (b <= a) continue;
          segs.push_back(Seg{j, static_cast<int32_t>(a - first[j]), static_cast<int32_t>(b - first[j]), -1});
          per_wg[w].push_back(static_cast<int>(segs.size()) - 1);
        }
      }
      // A range is the tail of one item followed by the heads of the next ones.  Running the
      // tail last makes every workgroup start at key tile 0 of its first segment, so that the
      // workgroups of one head walk the keys side by side (the tails, all of about the same
      // length, run at one common offset) instead of at scattered offsets.
      for (auto& v : per_wg) {
        std::stable_partition(v.begin(), v.end(), [&](int k) { return segs[k].kt0 == 0; });
      }
      int64_t worst = 0;
      for (auto& v : per_wg) {
        int64_t c = 0;
        for (int k : v) c += segs[k].kt1 - segs[k].kt0 + kSegOverhead;
        worst = std::max(worst, c);
      }
      return worst;
    };
    if (o.split_k >= 1) {
      whole_items_lpt(o.split_k);
    } else {
      // Whole items when there are enough of them to balance; else stream-K with partial merges.
      std::vector<std::vector<int>> keep;
      const int64_t m_lpt = whole_items_lpt(1);
      std::vector<Seg> keep_segs = segs;
      keep.swap(per_wg);
      const int64_t m_sk = stream_k() + 2;  // +2: merge pass
      if (m_lpt <= m_sk) {
        segs.swap(keep_segs);
        per_wg.swap(keep);
      }
    }

    // Partial slots: every segment of an item that has more than one segment.
    std::vector<int> nseg(n_items, 0);
    for (const Seg& g : segs) ++nseg[g.item];
    std::vector<std::vector<int>> item_segs(n_items);
    for (int i = 0; i < static_cast<int>(segs.size()); ++i) item_segs[segs[i].item].push_back(i);
    std::vector<int32_t> groups;
    int32_t slot = 0;
    P.max_parts = 1;
    for (int i = 0; i < n_items; ++i) {
      if (nseg[i] < 2) continue;
      groups.insert(groups.end(), {i, slot, nseg[i], 0});
      for (int sidx : item_segs[i]) segs[sidx].slot = slot++;
      P.max_parts = std::max(P.max_parts, nseg[i]);
    }
    P.n_partials = slot;
    P.n_groups = static_cast<int32_t>(groups.size() / kGroupInts);
    P.n_items = n_items;

    // Segments in workgroup order; ranges[w] = [first, end) of workgroup w.
    while (!per_wg.empty() && per_wg.back().empty()) per_wg.pop_back();
    std::vector<int32_t> seg_ints, ranges;
    for (const auto& v : per_wg) {
      ranges.push_back(static_cast<int32_t>(seg_ints.size() / kSegInts));
      for (int i : v) seg_ints.insert(seg_ints.end(), {segs[i].item, segs[i].kt0, segs[i].kt1, segs[i].slot});
      ranges.push_back(static_cast<int32_t>(seg_ints.size() / kSegInts));
    }
    P.n_segs = static_cast<int32_t>(seg_ints.size() / kSegInts);
    P.n_wgs = static_cast<int32_t>(per_wg.size());

    // Blob: header, items, segments, ranges, tiles, groups, chunks, chunk ids by rank.
    P.off_items = kHeaderInts;
    P.off_segs = P.off_items + static_cast<size_t>(n_items) * kItemInts;
    P.off_ranges = P.off_segs + seg_ints.size();
    P.off_tiles = P.off_ranges + ranges.size();
    P.off_groups = P.off_tiles + tiles.size();
    P.off_chunks = P.off_groups + groups.size();
    P.off_byrank = P.off_chunks + static_cast<size_t>(n) * kChunkInts;
    P.blob.assign(P.off_byrank + n, 0);
    int32_t* B = P.blob.data();
    B[H_MAGIC] = static_cast<int32_t>(kMagic);
    B[H_NONCE_LO] = static_cast<int32_t>(P.nonce & 0xffffffffu);
    B[H_NONCE_HI] = static_cast<int32_t>(P.nonce >> 32);
    B[H_ITEMS] = n_items;
    B[H_TILES] = P.n_tiles;
    B[H_GROUPS] = P.n_groups;
    B[H_OFF_ITEMS] = static_cast<int32_t>(P.off_items);
    B[H_OFF_TILES] = static_cast<int32_t>(P.off_tiles);
    B[H_OFF_GROUPS] = static_cast<int32_t>(P.off_groups);
    B[H_SEGS] = P.n_segs;
    B[H_OFF_SEGS] = static_cast<int32_t>(P.off_segs);
    B[H_WGS] = P.n_wgs;
    B[H_OFF_RANGES] = static_cast<int32_t>(P.off_ranges);
    B[H_CHUNKS] = n;
    B[H_OFF_CHUNKS] = static_cast<int32_t>(P.off_chunks);
    B[H_OFF_BYRANK] = static_cast<int32_t>(P.off_byrank);
    for (int i = 0; i < n_items; ++i) {
      const Item& it = items[i];
      int32_t* d = B + P.off_items + static_cast<size_t>(i) * kItemInts;
      d[0] = it.head; d[1] = it.q_row0; d[2] = it.rows; d[3] = it.qsb; d[4] = it.qchunk; d[5] = it.n_tiles;
      d[6] = last_rank[table->query_chunks[it.qchunk]];  // chunks of rank 0..d[6] are visible
    }
    for (int c = 0; c < n; ++c) {
      int32_t* d = B + P.off_chunks + static_cast<size_t>(c) * kChunkInts;
      d[0] = first_tile[c]; d[1] = table->chunk_tokens[c]; d[2] = rank[c]; d[3] = last_rank[c];
      B[P.off_byrank + rank[c]] = c;
    }
    std::copy(seg_ints.begin(), seg_ints.end(), B + P.off_segs);
    std::copy(ranges.begin(), ranges.end(), B + P.off_ranges);
    std::copy(tiles.begin(), tiles.end(), B + P.off_tiles);
    std::copy(groups.begin(), groups.end(), B + P.off_groups);

    // Workspace layout.
    const size_t D = static_cast<size_t>(P.head_dim);
    P.ws_blob = 0;
    size_t off = align_up(P.blob.size() * sizeof(int32_t), 256);
    // split-K partials: O as fp16 with a power-of-two exponent per row; per row, the LSE and the
    // exponent side by side
    P.ws_part_o = off;
    off = align_up(off + static_cast<size_t>(P.n_partials) * kBlockM * D * sizeof(uint16_t), 256);
    P.ws_part_lse = off;
    off = align_up(off + static_cast<size_t>(P.n_partials) * kBlockM * 2 * sizeof(float), 256);
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
      tmp = {P->n_items, P->n_tiles, P->n_groups, P->n_partials, P->block_m, P->block_n, P->max_parts,
             P->num_query_chunks, P->n_segs, P->n_wgs};
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
    case 4:
      src = P->blob.data() + P->off_segs;
      total = static_cast<size_t>(P->n_segs) * kSegInts;
      break;
    case 5:
      src = P->blob.data() + P->off_ranges;
      total = static_cast<size_t>(P->n_wgs) * kRangeInts;
      break;
    case 6:
      src = P->blob.data() + P->off_chunks;
      total = static_cast<size_t>(P->num_chunks) * kChunkInts;
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

extern "C" int32_t wfattn_abi_version(void) { return 3; }
