// Host-only fuzz harness for the work planner (csrc/host/plan.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_plan_sanitize.py
// (g++, no GPU code).  Seeded random batches, edge lengths included, every
// planner knob; after each plan it checks, from the inputs alone:
//   * the tiles of each (sequence) partition its packed rows [0, q_len * g);
//   * each tile's parts tile [0, kend) in order, kend being the tile's causal
//     key bound (min(Lk, last token + Lk - Lq + 1), or Lk), every part
//     non-empty, boundaries on 64-key blocks;
//   * split parts write disjoint partial rows inside part_rows, and the merge
//     groups name exactly the split tiles;
//   * every persistent queue entry names a unit of its launch, and each
//     (unit, kv head) of a launch appears exactly once.
// Exit status 0 when every check holds; the first failure is printed.
// Built with -DPLANT_MISTAKE it damages each plan, and must then fail.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "../varlen_paged_kv_amd/csrc/host/plan.h"

using namespace vpk;

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {   // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return static_cast<uint32_t>((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int pick(int n) { return static_cast<int>(next_u32() % static_cast<uint32_t>(n)); }

int length() {
  const int r = pick(100);
  if (r < 15) return 0;
  if (r < 35) return 1;
  if (r < 55) return 2 + pick(30);
  if (r < 90) return 32 + pick(700);
  return 700 + pick(5000);
}

#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "case %d: ", case_id);         \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      return false;                                       \
    }                                                     \
  } while (0)

bool one_case(int case_id) {
  PlanInput in;
  const int B = pick(13);
  const int gs[4] = {1, 2, 4, 8};
  in.batch = B;
  in.hkv = 1 + pick(4);
  in.hq = in.hkv * gs[pick(4)];
  in.head_dim = pick(2) ? 128 : 64;
  in.has_cache = pick(4) != 0;
  in.has_new = !in.has_cache || pick(3) != 0;
  in.causal = pick(3) != 0;
  const int pss[5] = {1, 4, 5, 16, 64};
  in.page_size = in.has_cache ? pss[pick(5)] : 1;
  in.kv_bytes = pick(2) ? 1 : 2;
  in.num_cus = pick(3) == 0 ? 1 + pick(8) : 256;
  const int fs[4] = {0, 1, 2, 7};
  in.force_splits = fs[pick(4)];
  in.persistent = pick(3) - 1;
  in.mixed = pick(2) != 0;
  in.one_grid = pick(5) == 0;
  in.mixed_dec_parts = 1 + pick(4);
  in.split_min_keys = pick(2) ? 256 : 64;
  const long long mpr[4] = {-1, 0, 100, 1 << 17};
  in.max_part_rows = mpr[pick(4)];

  std::vector<int32_t> cu_q(B + 1, 0), cu_kn(B + 1, 0), cache(B, 0);
  for (int b = 0; b < B; ++b) {
    const int q = length();
    cu_q[b + 1] = cu_q[b] + q;
    const int n = in.has_new ? (pick(4) ? q : length()) : 0;
    cu_kn[b + 1] = cu_kn[b] + n;
    cache[b] = in.has_cache ? length() : 0;
  }
  int max_pages = 1;
  for (int b = 0; b < B; ++b) {
    const int lk = cache[b] + cu_kn[b + 1] - cu_kn[b];
    max_pages = std::max(max_pages, (lk + in.page_size - 1) / in.page_size);
  }
  in.cu_q = cu_q.data();
  in.cu_kn = in.has_new ? cu_kn.data() : nullptr;
  in.cache_lens = in.has_cache ? cache.data() : nullptr;
  in.max_pages = max_pages;

  Plan plan;
  build_plan(in, plan);
#ifdef PLANT_MISTAKE
  // the checker's own test: a plan with one part's key range cut short
  if (!plan.items.empty()) plan.items[plan.items.size() / 2].key_end -= 1;
#endif

  const int g = in.hq / in.hkv;
  // tiles by (seq, row0): their rows and their parts' key ranges
  std::map<std::pair<int, int>, std::vector<const WorkItem*>> tiles;
  for (const WorkItem& it : plan.items) tiles[{it.seq, it.row0}].push_back(&it);
  std::map<int, std::vector<std::pair<int, int>>> rows_of;
  int split_tiles = 0;
  std::set<long long> part_rows;
  for (auto& kv : tiles) {
    const int b = kv.first.first, row0 = kv.first.second;
    auto& parts = kv.second;
    const WorkItem& f = *parts[0];
    CHECK(b >= 0 && b < B, "sequence %d out of range", b);
    const int q = cu_q[b + 1] - cu_q[b];
    const int lk = cache[b] + (cu_kn[b + 1] - cu_kn[b]);
    CHECK(f.nrows > 0 && row0 >= 0 && row0 + f.nrows <= q * g, "tile rows [%d, %d) outside [0, %d)", row0,
          row0 + f.nrows, q * g);
    rows_of[b].push_back({row0, row0 + f.nrows});
    long long kend = lk;
    if (in.causal) kend = std::min<long long>(kend, (row0 + f.nrows - 1) / g + lk - q + 1);
    kend = std::max<long long>(kend, 0);
    std::sort(parts.begin(), parts.end(), [](const WorkItem* a, const WorkItem* c) { return a->key_begin < c->key_begin; });
    int at = 0;
    for (const WorkItem* p : parts) {
      CHECK(p->nrows == f.nrows, "parts of one tile disagree on rows");
      CHECK(p->key_begin == at, "tile (%d, %d): part starts at %d, expected %d", b, row0, p->key_begin, at);
      CHECK(p->key_begin % kBlockN == 0, "part start %d not on a block", p->key_begin);
      CHECK(parts.size() == 1 || p->key_end > p->key_begin, "empty split part");
      at = p->key_end;
    }
    CHECK(at == kend, "tile (%d, %d): parts end at %d, key bound %lld", b, row0, at, kend);
    if (parts.size() > 1) {
      ++split_tiles;
      for (const WorkItem* p : parts) {
        CHECK(p->part >= 0, "split part without partial rows");
        for (int h = 0; h < in.hkv; ++h)
          for (int r = 0; r < p->nrows; ++r) {
            const long long pr = static_cast<long long>(p->part) + static_cast<long long>(h) * p->part_stride + r;
            CHECK(pr >= 0 && pr < plan.part_rows, "partial row %lld outside [0, %lld)", pr,
                  static_cast<long long>(plan.part_rows));
            CHECK(part_rows.insert(pr).second, "partial row %lld written twice", pr);
          }
      }
    } else {
      CHECK(f.part < 0, "unsplit tile with partial rows");
    }
  }
  for (int b = 0; b < B; ++b) {
    auto& v = rows_of[b];
    std::sort(v.begin(), v.end());
    int at = 0;
    for (auto& r : v) {
      CHECK(r.first == at, "sequence %d: rows jump from %d to %d", b, at, r.first);
      at = r.second;
    }
    CHECK(at == (cu_q[b + 1] - cu_q[b]) * g, "sequence %d: rows end at %d, expected %d", b, at,
          (cu_q[b + 1] - cu_q[b]) * g);
  }
  CHECK(static_cast<long long>(plan.groups.size()) == static_cast<long long>(split_tiles) * in.hkv,
        "%zu merge groups for %d split tiles", plan.groups.size(), split_tiles);
  // launches and their queues
  for (const Launch* L : {&plan.prefill, &plan.decode, &plan.mixed}) {
    if (L->grid == 0) continue;
    CHECK(L->first >= 0 && L->first + L->count <= static_cast<int>(plan.items.size()), "launch outside the items");
    if (!L->persistent) {
      CHECK(L->grid == L->count * in.hkv, "one workgroup per work expected");
      continue;
    }
    const int nq = L->grid;
    CHECK(L->queue_first + nq + 1 <= static_cast<int>(plan.queue_start.size()), "queue starts out of range");
    const int32_t* qs = plan.queue_start.data() + L->queue_first;
    std::vector<int> seen(static_cast<size_t>(L->count) * in.hkv, 0);
    for (int q = 0; q < nq; ++q) {
      CHECK(qs[q] <= qs[q + 1], "queue %d has negative length", q);
      for (int i = qs[q]; i < qs[q + 1]; ++i) {
        const long long at = static_cast<long long>(L->work_first) + i;
        CHECK(at >= 0 && at < static_cast<long long>(plan.queue_work.size()), "queue entry out of range");
        const int w = plan.queue_work[at];
        CHECK(w >= 0 && w < L->count * in.hkv, "work %d outside the launch", w);
        seen[w]++;
      }
    }
    for (size_t w = 0; w < seen.size(); ++w) CHECK(seen[w] == 1, "work %zu appears %d times", w, seen[w]);
  }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 2000;
  if (argc > 2) g_state ^= std::strtoull(argv[2], nullptr, 10) * 0x9E3779B97F4A7C15ull;
  for (int i = 0; i < n; ++i)
    if (!one_case(i)) return 1;
  std::printf("%d plans checked\n", n);
  return 0;
}
