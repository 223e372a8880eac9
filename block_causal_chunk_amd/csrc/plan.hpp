// plan.hpp -- host-side planner state shared by plan.cpp and the launch glue (no HIP here).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/wfattn.h"

namespace wfattn {

// Tile geometry of the attention kernels: 256 query rows per workgroup (4 waves x 64 rows),
// 64 keys per LDS tile.
constexpr int kBlockM = 256;
constexpr int kBlockN = 64;
constexpr int kItemInts = 8;   // ints per work item
constexpr int kSegInts = 4;    // ints per segment
constexpr int kRangeInts = 2;  // ints per workgroup range
constexpr int kTileInts = 2;   // ints per key tile
constexpr int kGroupInts = 4;  // ints per merge group
constexpr int kChunkInts = 4;  // ints per chunk: first key tile, tokens, rank, last rank it sees
constexpr int kHeaderInts = 16;
constexpr uint32_t kMagic = 0x57464132u;  // "WFA2"

// Header words of the uploaded blob (int32 index).
enum HeaderWord {
  H_MAGIC = 0,
  H_NONCE_LO = 1,
  H_NONCE_HI = 2,
  H_ITEMS = 3,
  H_TILES = 4,
  H_GROUPS = 5,
  H_OFF_ITEMS = 6,
  H_OFF_TILES = 7,
  H_OFF_GROUPS = 8,
  H_SEGS = 9,
  H_OFF_SEGS = 10,
  H_WGS = 11,
  H_OFF_RANGES = 12,
  H_CHUNKS = 13,
  H_OFF_CHUNKS = 14,
  H_OFF_BYRANK = 15,
};

struct Plan {
  uint32_t magic = kMagic;
  uint64_t nonce = 0;
  // table facts
  int32_t num_chunks = 0, num_heads = 0, head_dim = 0, page_size = 0, num_pages = 0;
  int32_t num_query_chunks = 0;
  int64_t lq = 0;
  int64_t nqb = 0;          // Q-scale blocks (64-row, restarting per query chunk)
  int64_t pool_rows = 0;    // num_pages * page_size
  float scale = 0.f;        // resolved softmax scale
  // schedule
  int32_t block_m = kBlockM, block_n = kBlockN, max_parts = 1, xcd_remap = 1;
  int32_t n_cus = 256, n_xcds = 8;  // the device the schedule spreads over
  int32_t n_vis_tiles = 0;          // key tiles some query chunk sees (a prefix of the tile list)
  int32_t n_items = 0, n_tiles = 0, n_groups = 0, n_partials = 0, n_segs = 0, n_wgs = 0;
  std::vector<int32_t> blob;  // header, items, segments, ranges, key tiles, merge groups
  size_t off_items = 0, off_segs = 0, off_ranges = 0, off_tiles = 0, off_groups = 0;  // int32 offsets
  size_t off_chunks = 0, off_byrank = 0;
  // workspace layout (bytes)
  size_t ws_blob = 0, ws_part_o = 0, ws_part_lse = 0, ws_stage = 0;
  size_t ws_base_bytes = 0;   // blob + partials
  size_t ws_fp32_bytes = 0;   // + bf16 staging of q and both pools
  size_t stage_q_off = 0, stage_k_off = 0, stage_v_off = 0;
};

}  // namespace wfattn

struct wfattn_plan_s {
  wfattn::Plan impl;
};

namespace wfattn {
inline bool plan_ok(const wfattn_plan_t* p) { return p != nullptr && p->impl.magic == kMagic; }
inline const Plan* as_plan(const wfattn_plan_t* p) { return &p->impl; }
}  // namespace wfattn
