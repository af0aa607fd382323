// Host-side work planner for the attention launch.
//
// Tiles every sequence's packed query rows (token * g + head_in_group) into
// items of at most 256 rows per kv head, gives each item the keys its rows can
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
  bool dec;   // decode mode: the whole sequence has at most 32 packed rows
};

// Relative time of one 64-key block: staging K/V is paid once per block, the
// MFMA and softmax work once per active 32-row wave; decode-mode tiles (a
// sequence of at most 32 rows) spread their keys over the four waves.
double block_cost(int32_t nrows, int32_t kv_bytes, bool decode_mode) {
  const double load = kv_bytes == 1 ? 0.6 : 1.0;
  if (decode_mode) return load + 0.25;
  const int waves = (nrows + kWaveRows - 1) / kWaveRows;
  return load + 1.0 * waves;
}

// Fixed cost of one work item (its metadata, page ids, Q rows, the final
// combine and stores), in the units of block_cost, measured on MI355X: about
// 1.6 units for a decode-mode item; a prefill-mode item (Q load of 256 rows,
// the first blocks' staging round trip, the output stores) costs about
// 13,000 cycles against about 3,900 per 9-unit block of 256 rows, i.e. 30
// units.
constexpr double kItemCost = 1.6;
constexpr double kPrefillItemCost = 30.0;

}  // namespace

void build_plan(const PlanInput& in, Plan& out) {
  out.items.clear();
  out.groups.clear();
  out.queue_start.clear();
  out.queue_work.clear();
  out.part_rows = 0;
  out.persistent = false;
  out.prefill = Launch();
  out.decode = Launch();
  out.mixed = Launch();
  out.num_pre_units = 0;
  const int32_t B = in.batch;
  const int32_t g = in.hq / in.hkv;
  out.seqs.resize(B);
  for (int32_t b = 0; b < B; ++b) {
    SeqInfo& s = out.seqs[b];
    s = SeqInfo{};
    if (in.q_start) {
      s.q_start = in.q_start[b];
      s.q_len = in.q_len[b];
    } else {
      s.q_start = in.cu_q[b];
      s.q_len = in.cu_q[b + 1] - in.cu_q[b];
    }
    s.bt_row = in.bt_row ? in.bt_row[b] : static_cast<int32_t>(static_cast<int64_t>(b) * in.max_pages);
    s.new_len = in.has_new ? in.cu_kn[b + 1] - in.cu_kn[b] : 0;
    s.kn_start = in.has_new ? in.cu_kn[b] : 0;
    s.cache_len = (in.has_cache && in.cache_lens) ? in.cache_lens[b] : 0;
    s.kv_len = s.cache_len + s.new_len;
  }

  // ---- row tiles (shared by all kv heads: every head has the same rows and keys)
  static thread_local std::vector<Tile> tiles;
  tiles.clear();
  double total_pre = 0.0, total_dec = 0.0;
  for (int32_t b = 0; b < B; ++b) {
    const SeqInfo& s = out.seqs[b];
    if (s.q_len <= 0) continue;
    const int64_t rows = static_cast<int64_t>(s.q_len) * g;
    for (int64_t r0 = 0; r0 < rows; r0 += kPrefillRows) {
      const int32_t nr = static_cast<int32_t>(std::min<int64_t>(kPrefillRows, rows - r0));
      const int32_t t_last = static_cast<int32_t>((r0 + nr - 1) / g);
      int64_t kend = s.kv_len;
      if (in.causal) kend = std::min<int64_t>(kend, static_cast<int64_t>(t_last) + s.kv_len - s.q_len + 1);
      kend = std::max<int64_t>(kend, 0);
      const int32_t nblk = static_cast<int32_t>((kend + kBlockN - 1) / kBlockN);
      const double c = (rows <= kWaveRows ? kItemCost : kPrefillItemCost) +
                       nblk * block_cost(nr, in.kv_bytes, rows <= kWaveRows);
      tiles.push_back(Tile{b, static_cast<int32_t>(r0), nr, 0, static_cast<int32_t>(kend), c, rows <= kWaveRows});
      (rows <= kWaveRows ? total_dec : total_pre) += c * in.hkv;
    }
  }

  // ---- split decision per tile -> units (tile, part).
  //      Prefill-mode grid (MFMA-bound, many items): longest-first dealing
  //      ends the grid evenly when no tile is above the average load of a
  //      workgroup slot; only a tile above that average is split, into parts
  //      near that size (the fp32 partials of up to 256 rows per part and
  //      their merge pass cost more than a slightly uneven end of the grid).
  //      Decode-mode grid (HBM-bound, few long sequences): every item of a
  //      dispatch round takes about as long, so the grid lasts about
  //      ceil(items / slots) rounds of (work per item + fixed cost per item);
  //      tiles are cut into parts of a common size chosen so that the item
  //      count fills whole rounds of the slots.
  const int64_t cus = std::max(1, in.num_cus);
  const double target_pre = total_pre / static_cast<double>(cus * std::max(1, in.pre_wg_per_cu));
  const int32_t min_blocks = std::max(1, (in.split_min_keys + kBlockN - 1) / kBlockN);
  auto split_limit = [&](const Tile& t) {
    const int32_t nblk = (t.kend + kBlockN - 1) / kBlockN;
    return std::max(1, std::min(nblk / min_blocks, kMaxSplits));
  };
  double part_dec = 0.0;   // decode-mode part size (cost units), 0: no split
  bool ceil_dec = false;   // split only tiles above part_dec, into ceil(cost / part_dec) parts
  if (total_dec > 0.0 && total_pre > 0.0) {
    // both kinds share the device, so the decode-mode items have no fixed
    // number of slots: parts of 1 / mixed_dec_parts of the average decode
    // load of a CU (on the mixed fp8 batch, 1 part per CU gave the shortest
    // step with the grids side by side and in one launch alike: 309.5 / 321.6
    // us against 318.7 / 334.2 at 4 and 331.3 / 359.4 at 8)
    part_dec = total_dec / static_cast<double>(cus * std::max(1, in.mixed_dec_parts));
    ceil_dec = true;
  } else if (total_dec > 0.0) {
    const int64_t slots_dec = cus * std::max(1, in.wg_per_cu);
    const double work = total_dec - kItemCost * static_cast<double>(in.hkv) *
                                        std::count_if(tiles.begin(), tiles.end(), [](const Tile& t) { return t.dec; });
    double best = 0.0;
    for (int32_t m = 1; m <= 8; ++m) {
      const double w = work / static_cast<double>(m * slots_dec);
      if (w <= 0.0) break;
      int64_t n = 0;
      for (const Tile& t : tiles) {
        if (!t.dec) continue;
        const double parts = std::round((t.cost - kItemCost) / w);
        n += std::min<int64_t>(std::max<int64_t>(1, static_cast<int64_t>(parts)), split_limit(t)) * in.hkv;
      }
      const double rounds = std::ceil(static_cast<double>(n) / static_cast<double>(slots_dec));
      const double est = rounds * (work / static_cast<double>(n) + kItemCost);
      if (m == 1 || est < best) {
        best = est;
        part_dec = w;
      }
    }
  }
  struct Unit {
    double cost;
    int32_t tile, part, b0, b1, nsplit, group;
  };
  // parts per tile
  static thread_local std::vector<int32_t> nparts;
  nparts.assign(tiles.size(), 1);
  for (int32_t ti = 0; ti < static_cast<int32_t>(tiles.size()); ++ti) {
    const Tile& t = tiles[ti];
    const int32_t nblk = (t.kend + kBlockN - 1) / kBlockN;
    int32_t n = 1;
    if (in.force_splits > 0) {
      n = std::min(in.force_splits, std::max(nblk, 1));
    } else if (t.dec) {
      if (ceil_dec) {
        if (t.cost > part_dec && nblk > min_blocks)
          n = std::min(static_cast<int32_t>(std::ceil(t.cost / part_dec)), split_limit(t));
      } else if (part_dec > 0.0) {
        const double parts = std::round((t.cost - kItemCost) / part_dec);
        n = static_cast<int32_t>(std::min<double>(std::max(1.0, parts), split_limit(t)));
      }
    } else if (t.cost > target_pre && nblk > min_blocks) {
      n = static_cast<int32_t>(std::ceil(t.cost / std::max(target_pre, 1e-9)));
      n = std::min(n, split_limit(t));
    }
    nparts[ti] = std::max(n, 1);
  }
  // Every part must fit the LDS page-id list: the fewest parts a tile can have.
  auto min_parts = [&](const Tile& t) {
    const int32_t nblk = (t.kend + kBlockN - 1) / kBlockN;
    if (!in.has_cache || nblk == 0) return 1;
    const int64_t blocks_per_part_max =
        std::max<int64_t>(1, (static_cast<int64_t>(kMaxItemPages - 1) * in.page_size) / kBlockN);
    return static_cast<int32_t>((nblk + blocks_per_part_max - 1) / blocks_per_part_max);
  };
  auto part_rows_of = [&]() {
    int64_t r = 0;
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      const int32_t n = std::max(nparts[ti], min_parts(tiles[ti]));
      if (n > 1) r += static_cast<int64_t>(n) * tiles[ti].nrows * in.hkv;
    }
    return r;
  };
  if (in.max_part_rows >= 0) {
    // a bounded workspace: scale the split counts down until the partials fit
    // (with no split beyond the page-id limit the plan needs the least)
    for (int64_t r = part_rows_of(); r > in.max_part_rows;) {
      bool changed = false;
      for (int32_t& n : nparts)
        if (n > 1) {
          n = std::max(1, n / 2);
          changed = true;
        }
      r = part_rows_of();
      if (!changed) break;
    }
  }
  static thread_local std::vector<Unit> units;
  units.clear();
  int32_t ngroups = 0;
  for (int32_t ti = 0; ti < static_cast<int32_t>(tiles.size()); ++ti) {
    const Tile& t = tiles[ti];
    const int32_t nblk = (t.kend + kBlockN - 1) / kBlockN;
    const int32_t n = std::max(nparts[ti], min_parts(t));
    if (n <= 1) {
      units.push_back(Unit{t.cost, ti, 0, 0, nblk, 1, -1});
      continue;
    }
    for (int32_t s = 0; s < n; ++s) {
      const int32_t b0 = static_cast<int32_t>(static_cast<int64_t>(nblk) * s / n);
      const int32_t b1 = static_cast<int32_t>(static_cast<int64_t>(nblk) * (s + 1) / n);
      units.push_back(Unit{(t.dec ? kItemCost : kPrefillItemCost) + (b1 - b0) * block_cost(t.nrows, in.kv_bytes, t.dec),
                           ti, s, b0, b1, n, ngroups});
    }
    ++ngroups;
  }

  // partial-row bases: group gi of tile ti covers nsplit * nrows rows per kv head
  static thread_local std::vector<int64_t> group_base;
  group_base.assign(ngroups, 0);
  {
    int32_t gi = 0;
    for (const Unit& u : units) {
      if (u.group < 0 || u.part != 0) continue;
      const Tile& t = tiles[u.tile];
      for (int32_t h = 0; h < in.hkv; ++h) {
        out.groups.push_back(MergeGroup{t.seq, t.row0, t.nrows, h,
                                        static_cast<int32_t>(out.part_rows + static_cast<int64_t>(h) * u.nsplit * t.nrows),
                                        u.nsplit, t.dec ? 1 : 0, 0, out.seqs[t.seq]});
      }
      group_base[gi++] = out.part_rows;
      out.part_rows += static_cast<int64_t>(in.hkv) * u.nsplit * t.nrows;
    }
  }

  // ---- order: prefill-mode units, then decode-mode units.  Prefill-mode
  //      units are grouped by sequence (heaviest sequence first) and run
  //      longest first inside it: the workgroups resident at one time then
  //      share one sequence's keys and values, which stay in the L2 of their
  //      XCD (workgroup w runs on XCD w mod 8 and the grid index is
  //      unit * Hkv + kv head, so with 8 kv heads each XCD serves one head).
  //      Decode-mode units run longest first.  Ties in tile / part order.
  static thread_local std::vector<int32_t> order;
  static thread_local std::vector<double> seq_cost;
  order.resize(units.size());
  std::iota(order.begin(), order.end(), 0);
  seq_cost.assign(B, 0.0);
  for (const Unit& u : units) seq_cost[tiles[u.tile].seq] += u.cost;
  // decode mode for sequences whose packed rows all fit one wave (q_len * g <=
  // 32); a prefill sequence's short last tile stays with its other tiles
  auto is_dec = [&](int32_t ui) { return tiles[units[ui].tile].dec; };
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    const bool da = is_dec(a), db = is_dec(b);
    if (da != db) return !da;
    if (!da) {
      const int32_t sa = tiles[units[a].tile].seq, sb = tiles[units[b].tile].seq;
      if (sa != sb) {
        if (seq_cost[sa] != seq_cost[sb]) return seq_cost[sa] > seq_cost[sb];
        return sa < sb;
      }
    }
    if (units[a].cost != units[b].cost) return units[a].cost > units[b].cost;
    return a < b;
  });

  out.items.reserve(units.size());
  int32_t n_prefill_units = 0;
  for (int32_t ui : order) {
    const Unit& u = units[ui];
    const Tile& t = tiles[u.tile];
    if (!is_dec(ui)) ++n_prefill_units;
    const int32_t kb = u.b0 * kBlockN;
    const int32_t ke = u.group < 0 ? t.kend : std::min(t.kend, u.b1 * kBlockN);
    int32_t part = -1, stride = 0;
    if (u.group >= 0) {
      part = static_cast<int32_t>(group_base[u.group] + static_cast<int64_t>(u.part) * t.nrows);
      stride = u.nsplit * t.nrows;
    }
    out.items.push_back(WorkItem{t.seq, t.row0, t.nrows, stride, kb, ke, part, 0, out.seqs[t.seq]});
  }
  out.prefill.first = 0;
  out.prefill.count = n_prefill_units;
  out.decode.first = n_prefill_units;
  out.decode.count = static_cast<int32_t>(out.items.size()) - n_prefill_units;
  out.num_pre_units = n_prefill_units;
  const bool with_mixed =
      (in.mixed && out.prefill.count > 0 && out.decode.count > 0) || (in.one_grid && !out.items.empty());
  if (with_mixed) {
    out.mixed.first = 0;
    out.mixed.count = static_cast<int32_t>(out.items.size());
  }

  // ---- per launch: one workgroup per (unit, kv head), or (persistent)
  //      greedy least-loaded queues over its ordered work.  A persistent grid
  //      reads its queue's metadata once per workgroup instead of once per
  //      item, which pays off when each workgroup slot gets several items;
  //      with few items per slot the hardware's dynamic dispatch balances
  //      better than the static queues.
  static thread_local std::vector<int32_t> owner;
  static thread_local std::vector<int32_t> count;
  static thread_local std::vector<int32_t> fill;
  static thread_local std::vector<int32_t> by_unit;
  static thread_local std::vector<double> heap_key;
  static thread_local std::vector<int32_t> heap_queue;
  out.persistent = false;
  for (Launch* L : {&out.prefill, &out.decode, &out.mixed}) {
    if (L == &out.mixed && !with_mixed) continue;
    if (in.one_grid && L != &out.mixed) {
      L->grid = 0;
      continue;
    }
    const int64_t nwork = static_cast<int64_t>(L->count) * in.hkv;
    const int64_t lslots = static_cast<int64_t>(std::max(1, in.num_cus)) *
                           std::max(1, L == &out.decode ? in.wg_per_cu : in.pre_wg_per_cu);
    L->persistent = in.persistent == 1 || (in.persistent == -1 && nwork >= 4 * lslots);
    L->queue_first = static_cast<int32_t>(out.queue_start.size());
    L->work_first = static_cast<int32_t>(out.queue_work.size());
    if (!L->persistent) {
      L->grid = static_cast<int32_t>(nwork);
      continue;
    }
    out.persistent = true;
    const int32_t nq = static_cast<int32_t>(std::min<int64_t>(lslots, nwork));
    L->grid = nq;
    if (nq == 0) continue;
    const size_t q0 = out.queue_start.size();
    out.queue_start.resize(q0 + nq + 1, 0);
    // longest first onto the least-loaded queue (LPT); each queue then runs
    // its work in the launch order above.  Works of one unit (its kv heads)
    // cost the same, so units are sorted and their works dealt in turn.
    std::vector<int32_t>& own = owner;
    std::vector<int32_t>& cnt = count;
    std::vector<int32_t>& ub = by_unit;
    std::vector<double>& hk = heap_key;
    std::vector<int32_t>& hq = heap_queue;
    cnt.assign(nq, 0);
    own.resize(nwork);
    ub.resize(L->count);
    std::iota(ub.begin(), ub.end(), 0);
    const int32_t* const ord = order.data() + L->first;
    const Unit* const un = units.data();
    // in the mixed grid a decode-mode unit runs on all eight waves of a
    // workgroup that holds the whole CU: half the slot time of its cost,
    // which counts a four-wave workgroup sharing the CU with another
    const bool halve_dec = L == &out.mixed;
    auto cost_of = [&](int32_t u) {
      const double c = un[ord[u]].cost;
      return halve_dec && L->first + u >= n_prefill_units ? 0.5 * c : c;
    };
    std::stable_sort(ub.begin(), ub.end(), [&](int32_t a, int32_t b) { return cost_of(a) > cost_of(b); });
    // binary min-heap of (load, queue), ties to the lower queue index
    hk.assign(nq, 0.0);
    hq.resize(nq);
    std::iota(hq.begin(), hq.end(), 0);
    auto less = [&](int32_t i, int32_t j) { return hk[i] < hk[j] || (hk[i] == hk[j] && hq[i] < hq[j]); };
    for (const int32_t u : ub) {
      const double c = cost_of(u);
      for (int32_t h = 0; h < in.hkv; ++h) {
        const int64_t w = static_cast<int64_t>(u) * in.hkv + h;
        const int32_t q = hq[0];
        own[w] = q;
        ++cnt[q];
        hk[0] += c;
        for (int32_t i = 0;;) {   // sift the root down
          const int32_t l = 2 * i + 1, r = l + 1;
          int32_t m = i;
          if (l < nq && less(l, m)) m = l;
          if (r < nq && less(r, m)) m = r;
          if (m == i) break;
          std::swap(hk[i], hk[m]);
          std::swap(hq[i], hq[m]);
          i = m;
        }
      }
    }
    for (int32_t q = 0; q < nq; ++q) out.queue_start[q0 + q + 1] = out.queue_start[q0 + q] + count[q];
    fill.assign(out.queue_start.begin() + q0, out.queue_start.begin() + q0 + nq);
    const size_t w0 = out.queue_work.size();
    out.queue_work.resize(w0 + nwork);
    for (int64_t w = 0; w < nwork; ++w) out.queue_work[w0 + fill[owner[w]]++] = static_cast<int32_t>(w);
  }
}

}  // namespace vpk
