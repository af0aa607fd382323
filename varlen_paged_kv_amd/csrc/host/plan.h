// Host-side work planner for the attention launch (pure C++, no GPU needed).
#pragma once

#include <stdint.h>

#include <vector>

#include "../vpk_internal.h"

namespace vpk {

struct PlanInput {
  int32_t batch = 0;
  int32_t hq = 0;
  int32_t hkv = 0;
  int32_t head_dim = 0;
  bool has_cache = false;
  bool has_new = false;
  bool causal = false;
  int32_t page_size = 1;
  int32_t kv_bytes = 2;                 // bytes per cached element (2 bf16, 1 fp8)
  const int32_t* cu_q = nullptr;        // [B + 1] host (or null with q_start / q_len)
  const int32_t* q_start = nullptr;     // [B] host: first query row of each sequence (with q_len)
  const int32_t* q_len = nullptr;       // [B] host
  const int32_t* cu_kn = nullptr;       // [B + 1] host, or null
  const int32_t* cache_lens = nullptr;  // [B] host, or null
  const int32_t* bt_row = nullptr;      // [B] host: first page-id index per sequence, or null (b * max_pages)
  int32_t max_pages = 0;                // row length of a dense block_table
  int32_t num_cus = 256;
  int32_t wg_per_cu = 2;                // resident decode-mode workgroups per CU
  int32_t pre_wg_per_cu = 1;            // resident prefill-mode workgroups per CU
  // knobs
  int32_t force_splits = 0;             // 0: planner decides
  int32_t persistent = -1;              // -1 planner, 0 off, 1 on
  bool mixed = false;                   // a batch with both kinds of items also gets the one-launch grid
  bool one_grid = false;                // every unit in the one-launch grid only (Plan::mixed), whatever its kinds
  int32_t mixed_dec_parts = 1;          // with both kinds: decode-mode parts of total / (num_cus * this)
  int32_t split_min_keys = 256;
  // largest number of split-partial rows the workspace holds (< 0: no limit);
  // splits are reduced, down to none, until the plan fits
  int64_t max_part_rows = -1;
};

// One attention grid: items [first, first + count) of Plan::items, run by the
// prefill-mode kernel (tiles of more than 32 rows) or the decode-mode kernel
// (tiles of at most 32 rows, keys split over the four waves).
struct Launch {
  int32_t first = 0;                    // first unit in Plan::items
  int32_t count = 0;                    // units
  int32_t grid = 0;                     // workgroups
  int32_t queue_first = 0;              // persistent: its num_queues + 1 entries of queue_start
  int32_t work_first = 0;               // persistent: its entries of queue_work
  bool persistent = false;              // static per-workgroup queues
};

struct Plan {
  std::vector<SeqInfo> seqs;
  std::vector<WorkItem> items;          // prefill-mode units, then decode-mode units
  std::vector<MergeGroup> groups;
  std::vector<int32_t> queue_start;     // persistent only; offsets into the launch's queue_work
  std::vector<int32_t> queue_work;      // persistent only; unit (launch-relative) * hkv + kv head
  int64_t part_rows = 0;                // rows of split partials
  bool persistent = false;
  Launch prefill, decode;
  // with PlanInput::mixed and both kinds of items: every unit in one grid of
  // 512-thread workgroups (prefill-mode units first, then decode-mode ones)
  Launch mixed;
  int32_t num_pre_units = 0;            // prefill-mode units (they come first in items)
};

constexpr int32_t kMaxSplits = 64;

void build_plan(const PlanInput& in, Plan& out);

}  // namespace vpk
