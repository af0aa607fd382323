// Internal structures shared by the host runtime and the HIP kernels of libvpk.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace vpk {

// A row is one (token, query head) pair of a sequence; the g = Hq / Hkv heads
// that share a kv head are packed token-major (row = token * g +
// head_in_group), so every K/V tile staged in LDS serves all of them.  Each
// wavefront owns 32 rows.  Prefill-mode items (more than 32 rows) run on 8
// wavefronts, 256 rows per item; decode-mode items (at most 32 rows) on 4
// wavefronts that split the keys.
constexpr int kWaveRows = 32;
constexpr int kWaves = 4;                       // decode-mode workgroup
constexpr int kThreads = kWaves * 64;           // 256
constexpr int kPrefillWaves = 8;                // prefill-mode workgroup
constexpr int kPrefillRows = kPrefillWaves * kWaveRows;   // 256
constexpr int kBlockN = 64;                     // keys per inner iteration
// Page ids of one work item are staged in LDS; an item may span at most this
// many pages (the planner splits longer key ranges).
constexpr int kMaxItemPages = 1024;

// Per-sequence facts taken from the host mirrors (32 bytes).
struct SeqInfo {
  int32_t q_start;    // first query row of the sequence (cu_seqlens_q[b], or its own start)
  int32_t q_len;      // Lq
  int32_t kv_len;     // Lk = Lc + Ln (or Ln without a cache)
  int32_t kn_start;   // cu_seqlens_knew[b] (0 without new K/V)
  int32_t cache_len;  // Lc
  int32_t new_len;    // Ln
  int32_t bt_row;     // index of the sequence's first page id in block_table (b * max_pages, or its CSR offset)
  int32_t pad1;
};

// One unit of attention work (64 bytes): packed rows [row0, row0 + nrows) of
// sequence `seq` against keys [key_begin, key_end), for every kv head; the
// grid index (or the persistent queue entry) picks the head.  The sequence's
// facts travel with the item, so a workgroup learns everything about its
// work in one read of the plan.
struct WorkItem {
  int32_t seq;
  int32_t row0;
  int32_t nrows;
  int32_t part_stride; // partial rows between consecutive kv heads of a split part
  int32_t key_begin;   // multiple of kBlockN
  int32_t key_end;
  int32_t part;        // -1: write out/lse; >= 0: first partial row of kv head 0
  int32_t pad;
  SeqInfo s;           // copy of the sequence's SeqInfo
};

// A tile whose key range was split (64 bytes): parts s = 0..nsplit-1 wrote
// partial rows part + s * nrows + r.
struct MergeGroup {
  int32_t seq;
  int32_t row0;
  int32_t nrows;
  int32_t kv_head;
  int32_t part;
  int32_t nsplit;
  int32_t dec;         // 1: a decode-mode tile (its parts run in the decode-mode grid)
  int32_t pad1;
  SeqInfo s;           // copy of the sequence's SeqInfo
};

enum KvFormat : int32_t { kKvBf16 = 0, kKvFp8 = 1 };

// Rotary embedding applied inside the attention kernels (query rows, as they
// are loaded) and the append (new key rows, as they are stored).
struct RopeArgs {
  const float* cos;           // [max_positions, dim / 2]
  const float* sin;
  int32_t dim;                // rotary_dim (multiple of 16), or 0: no rotation
  int32_t interleaved;        // 0: pairs (i, i + dim / 2); 1: pairs (2i, 2i + 1)
};

// largest number of new tokens one append workgroup stores
constexpr int kAppendTokensMax = 32;

struct AppendParams {
  const uint16_t* k_new;      // bf16 [Tn, Hkv, D]
  const uint16_t* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* tok;         // [Tn][2]: block_table index of each new token's page id, and its slot
  int32_t* err_flag;
  int32_t batch;
  int32_t total_knew;
  int32_t tokens_per_wg;      // new tokens stored by one workgroup
  int32_t max_pages;
  int32_t num_pages;
  int32_t page_size;
  int32_t row_elems;          // Hkv * D
  int32_t fp8;
  float k_inv_scale;          // fp32(1 / k_scale)
  float v_inv_scale;
  const float* kv_scale_dev;  // fp8: {k_scale, v_scale} in device memory, read at run time (overrides the two above)
  RopeArgs rope;              // new key rows turned before they are stored (dim 0: none)
  const int32_t* kpos;        // with rope: [Tn] position of each new token
  int32_t head_dim;
};

struct AttnParams {
  const uint16_t* q;          // bf16 [Tq, Hq, D]
  const void* k;              // cache [P, S, Hkv, D] or k_new [Tn, Hkv, D]
  const void* v;
  const int32_t* block_table; // [B, max_pages] (paged only)
  const WorkItem* items;      // this grid's units
  const int32_t* queue_start; // persistent: [num_queues + 1] offsets into queue_work
  const int32_t* queue_work;  // persistent: unit * hkv + kv_head, grouped by queue
  const void* k_new;          // new tokens, read directly when new_direct is set
  const void* v_new;
  uint16_t* out;              // bf16 [Tq, Hq, D]
  float* lse;                 // [Hq, Tq] or null
  float* part_o;              // [rows, D] fp32, normalised partial outputs
  float* part_lse;            // [rows]
  int32_t* err_flag;
  const void* zeros;          // >= 256 zero bytes: source of rows past the keys
  int32_t num_items;
  int32_t num_pre_units;      // units of this launch below this index run in prefill mode
  int32_t persistent;
  int32_t new_direct;         // keys >= cache_len come from k_new / v_new (bf16 cache)
  // fp8 cache, decode-mode items (head_dim 128): the new tokens' codes are
  // formed from k_new / v_new by the item that reads them, which also stores
  // them into the cache (the standalone append skips those tokens)
  int32_t dec_append;
  int32_t attn_blocks;        // workgroups past this index run the append instead
  int32_t max_pages;
  int32_t num_pages;
  int32_t page_size;
  int32_t page_shift;         // log2(page_size) or -1
  int32_t hq;
  int32_t hkv;
  int32_t g;
  int32_t total_q;
  int32_t causal;
  float qk_scale_log2;        // scale * log2(e) (* k_scale for fp8)
  float v_scale;              // 1 (bf16) or v_scale (fp8)
  const float* kv_scale_dev;  // fp8: {k_scale, v_scale} in device memory (overrides the two above)
  double scale_log2e;         // scale * log2(e) in double, for the device-scale product
  RopeArgs rope;              // query rows turned as they are loaded (dim 0: none)
  AppendParams app;           // the append, when it runs inside this grid
  // fp8 "QKV-Prob" grid only (qk_scale_log2 then also holds q_scale, v_scale
  // the product p_scale * v_scale)
  float q_inv_scale;          // fp32(1 / q_scale): the query rows' quantiser
  float p_log2;               // log2(p_scale)
  // decode-mode items whose `part` is >= 0 keep their first-pass fp32 scores
  // here, from float 32 * (part + kv head * part_stride) on (32 per block
  // of 32 keys and row)
  float* scores;
};





struct MergeParams {
  const MergeGroup* groups;
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int32_t num_groups;
  int32_t hq;
  int32_t g;
  int32_t total_q;
  int32_t head_dim;
};

// Rotary embedding of the query rows and the new key rows into copies.
struct RopeParams {
  const uint16_t* q;          // bf16 [q_rows, hq, D]
  uint16_t* q_out;            // turned copy, same layout
  const int32_t* qpos;        // [q_rows] position of each row, -1 = row not read
  const uint16_t* k;          // bf16 [k_rows, hkv, D]
  uint16_t* k_out;
  const int32_t* kpos;        // [k_rows]
  const float* cos;           // [max_positions, rot_dim / 2]
  const float* sin;
  int32_t q_rows;
  int32_t k_rows;
  int32_t hq;
  int32_t hkv;
  int32_t rot_dim;            // multiple of 16, <= D
  int32_t interleaved;
};

// Size of the device scratch array of the allocation-free entry point, and
// its device address on the current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(64) << 20;
int scratch_address(void** ptr);

// Attention grids: prefill-mode items, decode-mode items, or both kinds in one
// launch (units below AttnParams::num_pre_units run in prefill mode).
enum GridMode : int { kGridPrefill = 0, kGridDecode = 1, kGridMixed = 2 };

// Kernel launchers (defined in the .hip files); they return hipError_t as int.
int launch_attention(const AttnParams& p, int grid, int head_dim, int kv_format, bool paged,
                     int mode, void* stream);
// fp8 "QKV-Prob" attention over every unit of the launch (fp8 cache, no splits)
int launch_attention_prob8(const AttnParams& p, int grid, int head_dim, void* stream);
int launch_append(const AppendParams& p, void* stream);
int launch_merge(const MergeParams& p, void* stream);
int launch_rope(const RopeParams& p, int head_dim, void* stream);

}  // namespace vpk
