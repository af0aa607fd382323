// Host-side work planner for the attention launch.
//
// Tiles every sequence's packed query rows (token * g + head_in_group) into
// items of at most 128 rows per kv head, gives each item the keys its rows can
// see (the causal bound of its last token), splits items whose cost is far
// above the average share of a workgroup slot into key-range parts that the
// merge pass recombines, orders the items longest-first, and (persistent mode)
// deals them to per-workgroup queues with a greedy least-loaded rule.
//
// This follows the scheduling idea of the FlashInfer PoD-Attention page
// ("[Refactor] Uniform PoDAttention API with Horizontal Fusion SMs Schedule",
// Key Changes: prefill and decode requests share one persistent launch and
// resources are partitioned by the KV-cache load), and the lesson from its
// discussion that a planner must accept a sequence with an empty KV range.
// Requests are not classified into prefill and decode by a threshold: every
// item carries its own row count and key range, so a batch mixing q_len 1 rows
// with long prefills ("Add flash_attn_varlen_func_with_kvcache", Aim) is one
// list, and the cost model weighs rows against keys.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <numeric>
#include <queue>

namespace vpk {

namespace {

struct Tile {
  int32_t seq, row0, nrows, kv_head, kend;
  double cost;
};

// Relative time of one 64-key block: staging K/V is paid once per block, the
// MFMA and softmax work once per active 32-row wave.
double block_cost(int32_t nrows, int32_t kv_bytes) {
  const int waves = (nrows + kWaveRows - 1) / kWaveRows;
  const double load = kv_bytes == 1 ? 0.6 : 1.0;
  return load + 1.0 * waves;
}

}  // namespace

void build_plan(const PlanInput& in, Plan& out) {
  out = Plan();
  const int32_t B = in.batch;
  const int32_t g = in.hq / in.hkv;
  out.seqs.resize(B);
  for (int32_t b = 0; b < B; ++b) {
    SeqInfo& s = out.seqs[b];
    s = SeqInfo{};
    s.q_start = in.cu_q[b];
    s.q_len = in.cu_q[b + 1] - in.cu_q[b];
    s.new_len = in.has_new ? in.cu_kn[b + 1] - in.cu_kn[b] : 0;
    s.kn_start = in.has_new ? in.cu_kn[b] : 0;
    s.cache_len = (in.has_cache && in.cache_lens) ? in.cache_lens[b] : 0;
    s.kv_len = s.cache_len + s.new_len;
  }

  // ---- tiles
  std::vector<Tile> tiles;
  double total = 0.0;
  for (int32_t b = 0; b < B; ++b) {
    const SeqInfo& s = out.seqs[b];
    if (s.q_len <= 0) continue;
    const int64_t rows = static_cast<int64_t>(s.q_len) * g;
    for (int64_t r0 = 0; r0 < rows; r0 += kTileRows) {
      const int32_t nr = static_cast<int32_t>(std::min<int64_t>(kTileRows, rows - r0));
      const int32_t t_last = static_cast<int32_t>((r0 + nr - 1) / g);
      int64_t kend = s.kv_len;
      if (in.causal) kend = std::min<int64_t>(kend, static_cast<int64_t>(t_last) + s.kv_len - s.q_len + 1);
      kend = std::max<int64_t>(kend, 0);
      const int32_t nblk = static_cast<int32_t>((kend + kBlockN - 1) / kBlockN);
      const double c = 0.05 + nblk * block_cost(nr, in.kv_bytes);
      for (int32_t h = 0; h < in.hkv; ++h) {
        tiles.push_back(Tile{b, static_cast<int32_t>(r0), nr, h, static_cast<int32_t>(kend), c});
        total += c;
      }
    }
  }

  // ---- split decision
  const int64_t slots = static_cast<int64_t>(std::max(1, in.num_cus)) * std::max(1, in.wg_per_cu);
  const double target = total / static_cast<double>(2 * slots);
  const int32_t min_blocks = std::max(1, (in.split_min_keys + kBlockN - 1) / kBlockN);

  struct Pending {
    WorkItem it;
    double cost;
  };
  std::vector<Pending> items;
  items.reserve(tiles.size());
  for (const Tile& t : tiles) {
    const int32_t nblk = (t.kend + kBlockN - 1) / kBlockN;
    int32_t n = 1;
    if (in.force_splits > 0) {
      n = std::min(in.force_splits, std::max(nblk, 1));
    } else if (t.cost > target && nblk > min_blocks) {
      n = static_cast<int32_t>(std::ceil(t.cost / std::max(target, 1e-9)));
      n = std::min(n, nblk / min_blocks);
      n = std::min(n, kMaxSplits);
      n = std::max(n, 1);
    }
    // every part must fit the LDS page-id list
    if (in.has_cache && nblk > 0) {
      const int64_t blocks_per_part_max =
          std::max<int64_t>(1, (static_cast<int64_t>(kMaxItemPages - 1) * in.page_size) / kBlockN);
      const int32_t need = static_cast<int32_t>((nblk + blocks_per_part_max - 1) / blocks_per_part_max);
      n = std::max(n, need);
    }
    if (n <= 1) {
      Pending p;
      p.it = WorkItem{t.seq, t.row0, t.nrows, t.kv_head, 0, t.kend, -1, 0};
      p.cost = t.cost;
      items.push_back(p);
      continue;
    }
    MergeGroup gr{t.seq, t.row0, t.nrows, t.kv_head, static_cast<int32_t>(out.part_rows), n, 0, 0};
    out.groups.push_back(gr);
    for (int32_t s = 0; s < n; ++s) {
      const int32_t b0 = static_cast<int32_t>(static_cast<int64_t>(nblk) * s / n);
      const int32_t b1 = static_cast<int32_t>(static_cast<int64_t>(nblk) * (s + 1) / n);
      Pending p;
      p.it = WorkItem{t.seq, t.row0, t.nrows, t.kv_head, b0 * kBlockN,
                      std::min(t.kend, b1 * kBlockN),
                      static_cast<int32_t>(out.part_rows + static_cast<int64_t>(s) * t.nrows), 0};
      p.cost = 0.05 + (b1 - b0) * block_cost(t.nrows, in.kv_bytes);
      items.push_back(p);
    }
    out.part_rows += static_cast<int64_t>(n) * t.nrows;
  }

  // ---- order: longest first (stable, so equal costs keep tile order)
  std::stable_sort(items.begin(), items.end(),
                   [](const Pending& a, const Pending& b) { return a.cost > b.cost; });

  const bool persistent = in.persistent == 1;
  out.persistent = persistent;
  if (!persistent) {
    out.items.reserve(items.size());
    for (const Pending& p : items) out.items.push_back(p.it);
    out.grid = static_cast<int32_t>(out.items.size());
    return;
  }

  // ---- persistent: greedy least-loaded queues
  const int32_t nq = static_cast<int32_t>(std::min<int64_t>(slots, static_cast<int64_t>(items.size())));
  out.grid = nq;
  out.queue_start.assign(nq + 1, 0);
  if (nq == 0) return;
  using Load = std::pair<double, int32_t>;
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int32_t q = 0; q < nq; ++q) heap.push(Load{0.0, q});
  std::vector<int32_t> count(nq, 0);
  for (Pending& p : items) {
    Load l = heap.top();
    heap.pop();
    p.it.queue = l.second;
    ++count[l.second];
    l.first += p.cost;
    heap.push(l);
  }
  for (int32_t q = 0; q < nq; ++q) out.queue_start[q + 1] = out.queue_start[q] + count[q];
  out.items.resize(items.size());
  std::vector<int32_t> fill(out.queue_start.begin(), out.queue_start.end() - 1);
  for (const Pending& p : items) out.items[fill[p.it.queue]++] = p.it;
}

}  // namespace vpk
