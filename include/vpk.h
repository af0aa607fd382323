/*
 * vpk.h -- C ABI of libvpk: forward attention of packed variable-length queries
 * over a paged KV cache, with an in-place append of new keys/values, for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources are the public pull-request pages this library is
 * built from, cited by page title and section):
 *
 *   For every sequence b of a batch, with Lq = q_len, Lc = cached length,
 *   Ln = new length, Lk = Lc + Ln, S = page_size, g = Hq / Hkv:
 *
 *   1. append: new token j (0 <= j < Ln) is stored at logical position
 *      pos = Lc + j, i.e. page block_table[b][pos / S], slot pos % S, all kv
 *      heads; bf16 caches receive the bytes unchanged, fp8 caches receive
 *      e4m3fn(fp32(x) * fp32(1 / scale)), rounded to nearest even, saturated to
 *      +-448.  ("Add flash_attn_varlen_func_with_kvcache", Usage: the cache is
 *      updated in place and read through per-sequence lengths; Minor Changes:
 *      the cache length is its own parameter and the new tokens carry their own
 *      cumulative offsets.)
 *   2. attention: out[i, h] = sum_j softmax_j(scale * q_i . k_j) v_j over the
 *      keys j < Lk of the sequence, keys and values read from the cache after
 *      the append, kv head h / g, with j <= i + Lk - Lq when causal (the
 *      diagonal aligned to the end of the keys); lse[h, i] = ln sum_j
 *      exp(scale * q_i . k_j).  A query that sees no key gets out = 0 and
 *      lse = -inf.  ("Extend FlashAttention Prefill with KV cache",
 *      description: cached plus current KV, causal and non-causal; "Add KV
 *      cache for paged/non-paged attention", Description: one page table for
 *      K and V, batches that mix context and generation; "[Kernel][Triton][FP8]
 *      Adding fp8 and variable length sequence support to Triton FAv2 kernel",
 *      feature list: 8-bit KV cache, causal, grouped-query heads, variable
 *      lengths.)
 *
 * Layouts (all contiguous, row-major, element strides implied by the shape):
 *   q, out            [total_q, num_q_heads, head_dim]        bf16
 *   k_new, v_new      [total_knew, num_kv_heads, head_dim]    bf16
 *   k_cache, v_cache  [num_pages, page_size, num_kv_heads, head_dim]
 *                     bf16 or fp8 e4m3fn (kv_cache_dtype)
 *   block_table       [batch, max_pages_per_seq]              int32
 *   cu_seqlens_q      [batch + 1] int32, 0 = c[0] <= c[1] <= ... = total_q
 *   cu_seqlens_knew   [batch + 1] int32, likewise ending at total_knew
 *   cache_seqlens     [batch]     int32, cached length BEFORE the append
 *   lse               [num_q_heads, total_q]                  fp32, natural log
 *
 * Memory and ownership: every pointer is borrowed.  Device pointers (q, k_new,
 * v_new, caches, block_table, out, lse and the device index arrays) must stay
 * valid until the work enqueued on `stream` has run; the call returns as soon
 * as the work is enqueued.  Host pointers (dims, host mirrors, kv_scale) are
 * read before the call returns.  The caches are modified in place only at the
 * slots of the appended tokens.  cache_seqlens is never modified: the caller
 * advances it, as with the cache-length parameter of the flash-attention page.
 * Device buffers must be 16-byte aligned (lse: 4-byte).
 *
 * Workspace: split partials, the device error flag and (attn_varlen_paged_rope_fwd)
 * the turned copies of q and k_new live in a per-device, per-stream workspace
 * in device memory.  The caller provides it with vpk_set_workspace (sized by
 * vpk_workspace_bytes_upper_bound; the Python binding does this with a torch
 * tensor, so that PyTorch owns the device memory); a stream without one gets a
 * library-allocated workspace that grows as needed (the fallback).  The work
 * list of a direct call is written into a small ring of pinned host buffers
 * that the kernels read directly, or from a copy at the end of a caller's
 * workspace when it repeats the previous call's (option "plan_reuse").  Two calls that overlap in time on one
 * device must use the same stream or different streams, never the same stream
 * from two host threads at once.
 *
 * Errors: every entry point returns a vpk_status; nothing throws or aborts.
 * vpk_last_error() gives a message for the calling thread's last failure.
 * Argument errors are detected on the host from the dims and the host mirrors
 * before anything is enqueued.
 */
#ifndef VPK_H_
#define VPK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VPK_ABI_VERSION 1

typedef enum {
  VPK_SUCCESS = 0,
  VPK_ERROR_INVALID_VALUE = 1,   /* a shape, pointer, length or page id is wrong */
  VPK_ERROR_NOT_SUPPORTED = 2,   /* valid but not implemented (e.g. head_dim 96) */
  VPK_ERROR_CAPACITY = 3,        /* Lc + Ln exceeds max_pages_per_seq * page_size */
  VPK_ERROR_HIP = 4,             /* a HIP runtime call failed */
  VPK_ERROR_OUT_OF_MEMORY = 5    /* workspace allocation failed */
} vpk_status;

typedef enum {
  VPK_DTYPE_BF16 = 1,
  VPK_DTYPE_FP8_E4M3FN = 2       /* OCP e4m3fn, per-tensor scale */
} vpk_dtype;

/* Problem sizes.  kv_cache_dtype is ignored when there is no cache. */
typedef struct {
  int32_t batch;               /* B >= 0 */
  int32_t total_q;             /* Tq = cu_seqlens_q[B] */
  int32_t total_knew;          /* Tn = cu_seqlens_knew[B]; 0 without new K/V */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;            /* D: 64 or 128 */
  int32_t num_pages;           /* P: pages of each cache tensor; 0 without a cache */
  int32_t max_pages_per_seq;   /* row length of block_table */
  int32_t kv_cache_dtype;      /* vpk_dtype */
} vpk_dims;

/* Host copies of the index arrays (same contents as the device arrays).  The
 * work list is planned from these.  Any member may be NULL: the library then
 * copies the device array to the host with a blocking copy on `stream` (slow
 * path).  block_table, when given, lets the host reject page ids outside
 * [0, num_pages) for the slots that are read or written; without it the
 * kernels skip such pages and raise a device error flag that
 * vpk_device_error() returns: appends to such a page are dropped and its
 * slots read as zero keys and values (with a bf16 cache the new tokens
 * themselves are read from k_new / v_new, so only its cached slots read as
 * zero). */
typedef struct {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_knew;
  const int32_t* cache_seqlens;
  const int32_t* block_table;
} vpk_host_index;

/*
 * attn_varlen_paged_fwd -- the whole call: append the new K/V (if any) into
 * the cache (if any), then attention for every packed query row.
 *
 *   dims            sizes (host).
 *   q               device bf16 [Tq, Hq, D].
 *   cu_seqlens_q    device int32 [B + 1].
 *   k_new, v_new    device bf16 [Tn, Hkv, D], or both NULL (attend over the
 *                   cache only, as the flash-attention page's Usage section
 *                   allows).  With Tn == 0 they may be NULL while
 *                   cu_seqlens_knew is given (every sequence adds nothing).
 *   cu_seqlens_knew device int32 [B + 1]; NULL when there are no new tokens.
 *   k_cache,v_cache device [P, S, Hkv, D] in kv_cache_dtype, or both NULL: no
 *                   cache, attention runs over k_new/v_new of each sequence and
 *                   nothing is stored.  With a cache, new tokens are appended
 *                   first and attention reads every key from the cache.
 *   block_table     device int32 [B, max_pages_per_seq], shared by K and V;
 *                   entries beyond ceil(Lk / S) of a row are never read.
 *   cache_seqlens   device int32 [B] (NULL without a cache).
 *   page_size       S >= 1 tokens per page (ignored without a cache).
 *   causal          0 or 1.
 *   scale           softmax scale, finite and > 0.
 *   kv_scale        host float[2] = {k_scale, v_scale} > 0 for an fp8 cache:
 *                   stored code c means c * scale; NULL for bf16.
 *   out             device bf16 [Tq, Hq, D].
 *   lse             device fp32 [Hq, Tq], or NULL.
 *   host            host mirrors (see vpk_host_index), or NULL.
 *   stream          hipStream_t (NULL = default stream).
 *
 * Returns VPK_SUCCESS once all work is enqueued.  Split-KV, the persistent
 * work schedule and the merge pass are internal choices of the library.
 * A direct call plans on the host and may grow its workspace, so it cannot be
 * captured into a graph: on a capturing stream it returns
 * VPK_ERROR_NOT_SUPPORTED before anything is enqueued (prepared calls,
 * vpk_plan_create / vpk_plan_run, are the capturable form).  The same holds
 * for attn_varlen_paged_rope_fwd, attn_varlen_paged_list_fwd and
 * kv_cache_append.
 */
int32_t attn_varlen_paged_fwd(const vpk_dims* dims,
                              const void* q, const int32_t* cu_seqlens_q,
                              const void* k_new, const void* v_new,
                              const int32_t* cu_seqlens_knew,
                              void* k_cache, void* v_cache,
                              const int32_t* block_table, const int32_t* cache_seqlens,
                              int32_t page_size, int32_t causal, float scale,
                              const float* kv_scale,
                              void* out, float* lse,
                              const vpk_host_index* host, void* stream);

/*
 * attn_varlen_paged_fwd_noalloc -- attn_varlen_paged_fwd for callers that
 * cannot allocate memory (tight serving loops, harnesses that forbid device
 * allocation).  It allocates no device or pinned memory, creates no stream or
 * event and never synchronises: its work list and split partials go to a
 * fixed 64 MiB scratch array in device memory that the library's code object
 * holds on each device it runs on (until the process ends).  The work list is
 * copied there from pageable host memory with one hipMemcpyAsync on `stream`.
 *   Arguments and results as for attn_varlen_paged_fwd, except:
 *   host    required, with every index array the call uses (cu_seqlens_q,
 *           cu_seqlens_knew with new tokens, cache_seqlens and block_table
 *           with a cache): nothing is read back from the device, and page
 *           ids are range-checked on the host.
 *   The planner limits its key-range splits to what the scratch array holds;
 *   a call whose work list and unsplit needs exceed it returns
 *   VPK_ERROR_CAPACITY before anything is enqueued.  A mixed batch runs its
 *   two grids one after the other on `stream`.
 * Every call on a device shares that device's scratch array, which keeps the
 * last call's contents: calls that overlap in time on one device (two
 * streams, or two host threads) race and must not be issued; consecutive
 * calls on one stream are ordered.  Not during stream capture
 * (VPK_ERROR_NOT_SUPPORTED): the copy reads host memory.
 */
int32_t attn_varlen_paged_fwd_noalloc(const vpk_dims* dims,
                                      const void* q, const int32_t* cu_seqlens_q,
                                      const void* k_new, const void* v_new,
                                      const int32_t* cu_seqlens_knew,
                                      void* k_cache, void* v_cache,
                                      const int32_t* block_table, const int32_t* cache_seqlens,
                                      int32_t page_size, int32_t causal, float scale,
                                      const float* kv_scale,
                                      void* out, float* lse,
                                      const vpk_host_index* host, void* stream);

/*
 * Rotary position embedding applied by attn_varlen_paged_rope_fwd.  The
 * TransformerEngine KV-cache page ("Add KV cache for paged/non-paged
 * attention", Description) names RoPE for inference as the step that comes
 * with the cache path without defining it; the rotation here is the published
 * one (Su et al., "RoFormer", section 3.4): coordinates in pairs (a, b), pair
 * i of a row at position m turned by the angle m * theta_i:
 *   a' = a cos - b sin,  b' = a sin + b cos.
 *   cos, sin        device float32 [max_positions, rotary_dim / 2], 16-byte
 *                   aligned: entry [m, i] for position m, pair i (the caller's
 *                   angles; any base or scaling).  Borrowed, read only.
 *   max_positions   rows of the tables.
 *   rotary_dim      turned coordinates [0, rotary_dim): a multiple of 16 in
 *                   [16, head_dim]; later coordinates are copied.
 *   interleaved     0: pair i is (i, i + rotary_dim / 2); 1: pair i is (2i, 2i + 1).
 */
typedef struct {
  const float* cos;
  const float* sin;
  int32_t max_positions;
  int32_t rotary_dim;
  int32_t interleaved;
} vpk_rope;

/*
 * attn_varlen_paged_rope_fwd -- attn_varlen_paged_fwd with the query rows and
 * the new key rows turned by vpk_rope first (values are not turned).  New
 * token j of a sequence sits at position Lc + j (the slot it is appended to),
 * query row i at Lk - Lq + i (the key its end-aligned causal bound stops at),
 * so a decode row over a cache of Lk keys sits at Lk - 1.  The turned rows
 * are bf16: each product and the difference / sum rounded to float32, then
 * round to nearest even; the cache stores the turned keys.  q and k_new are
 * not modified: the attention kernels turn the query rows of prefill-mode
 * sequences as they load them (interleaved pairs, or half-split pairs with
 * rotary_dim a multiple of 32), an fp8 cache's append turns the new keys as
 * it quantises them, and the other rows (decode-mode query rows, other
 * rotary dims, the new keys of a bf16 cache or of a call without a cache)
 * are turned into copies in the workspace first.
 * Extra errors: VPK_ERROR_INVALID_VALUE when rope is NULL or its fields break
 * the rules above, when a sequence has more query rows than keys, or when a
 * position reaches max_positions.  Other arguments and errors as for
 * attn_varlen_paged_fwd.
 */
int32_t attn_varlen_paged_rope_fwd(const vpk_dims* dims,
                                   const void* q, const int32_t* cu_seqlens_q,
                                   const void* k_new, const void* v_new,
                                   const int32_t* cu_seqlens_knew,
                                   void* k_cache, void* v_cache,
                                   const int32_t* block_table, const int32_t* cache_seqlens,
                                   int32_t page_size, int32_t causal, float scale,
                                   const float* kv_scale, const vpk_rope* rope,
                                   void* out, float* lse,
                                   const vpk_host_index* host, void* stream);

/*
 * attn_varlen_paged_qkv_prob_fwd -- attn_varlen_paged_fwd (or, with `rope`,
 * attn_varlen_paged_rope_fwd) with the attention in fp8 "QKV-Prob" form: the
 * query rows, the keys and values and the softmax output are all fp8 e4m3fn,
 * and both products run on fp8 matrix cores.  The vLLM Triton FAv2 PR page
 * ("[Kernel][Triton][FP8] Adding fp8 and variable length sequence support to
 * Triton FAv2 kernel", feature list item 7 and the paragraph before its
 * LM EVAL tables) names such models: softmax(QK^T) is quantised to fp8
 * before the second product.  The page fixes no scales or rounding; here:
 *   query codes  qc = e4m3fn(fp32(q) * fp32(1 / q_scale)), the cache's rule
 *                (after rotary embedding when `rope` is given);
 *   scores       s_ij = scale * q_scale * k_scale * sum_d qc_id kc_jd, masked
 *                as in attn_varlen_paged_fwd;
 *   softmax      P_ij = exp(s_ij - lse_i), lse_i = ln sum_j exp(s_ij): the
 *                row's exact softmax over all its visible keys;
 *   P codes      pc_ij = e4m3fn(P_ij / p_scale), nearest, ties to even;
 *   output       out_i = p_scale * v_scale * sum_j pc_ij vc_j (bf16, round to
 *                nearest even), not renormalised; lse as above.
 * Each row's scores are formed twice (once for the row maximum and sum,
 * once for P and the second product) and no key range is split.  Sequences
 * of at most 8 packed rows (head_dim 128) keep their first-pass scores in
 * the workspace when it has room (vpk_qkv_prob_score_bytes; option
 * "keep_scores"), so their second pass reads the scores instead of the K
 * codes; the results are the same either way.
 *   kv_scale  host float[2] {k_scale, v_scale}, required (fp8 cache only).
 *   qp_scale  host float[2] {q_scale, p_scale}: q_scale finite and > 0;
 *             p_scale finite and >= 1/452 (P <= 1, so P / p_scale stays
 *             within the range the conversion rounds without saturating;
 *             1/448 maps P = 1 to the largest finite code).
 *   rope      vpk_rope as for attn_varlen_paged_rope_fwd, or NULL.
 * fp8 matrix-core sums are not exact float32 sums: on gfx950 they deviate by
 * up to about 2^-13 of the sum of the magnitudes of their terms, so a P code
 * whose value lies that close to a rounding boundary may take either
 * neighbour.
 * Extra errors: VPK_ERROR_INVALID_VALUE for a bf16 cache, no cache, or
 * scales that break the rules above; VPK_ERROR_NOT_SUPPORTED when a
 * sequence's keys span more than 1023 pages.  Otherwise as
 * attn_varlen_paged_fwd.
 */
int32_t attn_varlen_paged_qkv_prob_fwd(const vpk_dims* dims,
                                       const void* q, const int32_t* cu_seqlens_q,
                                       const void* k_new, const void* v_new,
                                       const int32_t* cu_seqlens_knew,
                                       void* k_cache, void* v_cache,
                                       const int32_t* block_table, const int32_t* cache_seqlens,
                                       int32_t page_size, int32_t causal, float scale,
                                       const float* kv_scale, const float* qp_scale, const vpk_rope* rope,
                                       void* out, float* lse,
                                       const vpk_host_index* host, void* stream);

/*
 * The page-list form of the same call.  The POD page's batch API describes
 * sequences by a page list in CSR form (an offsets array into one array of
 * page ids) and lets the query rows of a sequence sit anywhere in q/out (its
 * own start and length instead of cumulative offsets) ("[Refactor] Uniform
 * PoDAttention API with Horizontal Fusion SMs Schedule", Key Changes 1).
 */
typedef struct {
  const int32_t* q_start;          /* [B]: first row of sequence b in q / out and in lse's row axis */
  const int32_t* q_len;            /* [B]: Lq; rows of different sequences may not overlap */
  const int32_t* cu_seqlens_knew;  /* [B + 1], as for attn_varlen_paged_fwd; NULL without new K/V */
  const int32_t* cache_seqlens;    /* [B] length before the append; NULL without a cache */
  const int32_t* kv_indptr;        /* [B + 1] non-decreasing: sequence b's page ids are
                                      kv_indices[kv_indptr[b] .. kv_indptr[b + 1]); NULL without a cache */
  const int32_t* kv_indices;       /* host copy of kv_indices, or NULL (then page ids are not range-checked
                                      on the host; see vpk_host_index.block_table) */
} vpk_host_pages;

/*
 * attn_varlen_paged_list_fwd -- attn_varlen_paged_fwd with the page lists and
 * query rows of vpk_host_pages: every length and offset comes from `host`
 * (required), only kv_indices (device int32 [kv_indptr[B]]) is read on the
 * device.  dims->total_q is the row count of q / out / lse (rows no sequence
 * names are left untouched); dims->max_pages_per_seq is not used.  Results
 * are those of attn_varlen_paged_fwd for a block_table whose row b holds
 * sequence b's page list.  Errors as for attn_varlen_paged_fwd (overlapping
 * query rows: VPK_ERROR_INVALID_VALUE; a page list too short for Lc + Ln:
 * VPK_ERROR_CAPACITY).
 */
int32_t attn_varlen_paged_list_fwd(const vpk_dims* dims, const void* q, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, const int32_t* kv_indices, int32_t page_size,
                                   int32_t causal, float scale, const float* kv_scale, void* out, float* lse,
                                   const vpk_host_pages* host, void* stream);

/*
 * kv_cache_append -- step 1 alone: store k_new/v_new into the paged cache at
 * positions [Lc, Lc + Ln) of each sequence (same rules and arguments as above).
 * Idempotent: repeating it with the same arguments writes the same bytes.
 */
int32_t kv_cache_append(const vpk_dims* dims,
                        const void* k_new, const void* v_new,
                        const int32_t* cu_seqlens_knew,
                        void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        int32_t page_size, const float* kv_scale,
                        const vpk_host_index* host, void* stream);

/*
 * Prepared calls (plan once, run many times).  The work list of a call depends
 * only on the lengths (cu_seqlens_q, cu_seqlens_knew, cache_seqlens), the head
 * counts and the flags, so a caller that runs the same lengths repeatedly (a
 * layer stack of one decode step, a graph replayed every step) can plan once
 * and launch without host work.  vpk_plan_run allocates nothing, synchronises
 * nothing and records no event, so it can be captured into a HIP graph; the
 * flash-attention-style APIs on the pages either lack graph support or list it
 * per backend ("[Refactor] Uniform PoDAttention API with Horizontal Fusion SMs
 * Schedule", Limitations and Future Work; "Add KV cache for paged/non-paged
 * attention", the backend support list).
 */
typedef struct vpk_plan_s* vpk_plan;

/*
 * vpk_plan_create -- validate the lengths and build the work list of a call,
 * in device memory of the current device (with its own split-partial space,
 * error flag and zero rows).  Synchronous (one blocking upload); not for use
 * inside stream capture.
 *   dims        as for attn_varlen_paged_fwd (kv_cache_dtype fixes the cache
 *               format of every run).
 *   host        host copies of the index arrays; cu_seqlens_q always,
 *               cu_seqlens_knew with has_new, cache_seqlens with has_cache
 *               (block_table optional: when given, its page ids for the
 *               slots that will be read or written are range-checked here).
 *   has_new     1: runs pass k_new / v_new (appended first when has_cache).
 *   has_cache   1: runs pass a paged cache.
 *   page_size, causal  as for attn_varlen_paged_fwd.
 *   plan        receives the handle; the caller owns it (vpk_plan_destroy).
 * The host arrays are read before the call returns.  Errors as for
 * attn_varlen_paged_fwd; nothing is allocated on failure.
 */
int32_t vpk_plan_create(const vpk_dims* dims, const vpk_host_index* host, int32_t has_new,
                        int32_t has_cache, int32_t page_size, int32_t causal, vpk_plan* plan);

/*
 * vpk_plan_run -- enqueue the call a plan describes on `stream`: the same
 * steps and results as attn_varlen_paged_fwd with those lengths (append, then
 * attention, then the merge of split parts), with the device buffers given
 * here (same layouts and alignment rules).  The device index arrays are not
 * read: the lengths are the plan's, and block_table is read on the device
 * only.  When a plan has both prefill-mode and decode-mode work, the two grids
 * run one after the other on `stream`.  Runs of one plan share its partial
 * space: overlapping runs of the same plan (two streams at once) race.
 * kv_scale is read on the host at each call (a captured graph keeps the
 * values of the captured call; vpk_plan_run_device_scale reads them on the
 * device instead).
 */
int32_t vpk_plan_run(vpk_plan plan, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, const int32_t* block_table, float scale,
                     const float* kv_scale, void* out, float* lse, void* stream);

/*
 * vpk_plan_run_device_scale -- vpk_plan_run with the fp8 scales in device
 * memory: kv_scale_dev is a device float[2] = {k_scale, v_scale} (4-byte
 * aligned, borrowed) that the kernels read when they run, so a graph captured
 * around this call follows scales the caller updates between replays.  The
 * kernels derive the score factor and the reciprocals the way the host does
 * for vpk_plan_run (same bits for the same scales).  The values must be
 * finite and > 0 (they are not checked: a bad value gives bad results, never
 * an out-of-bounds access).  For a bf16 plan kv_scale_dev must be NULL.
 * Errors as for vpk_plan_run.
 */
int32_t vpk_plan_run_device_scale(vpk_plan plan, const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const int32_t* block_table, float scale,
                                  const float* kv_scale_dev, void* out, float* lse, void* stream);

/* Synchronise `stream` and return (and clear) the plan's device error flag
 * (bit 0: a page id outside [0, num_pages) was met on the device). */
int32_t vpk_plan_device_error(vpk_plan plan, void* stream, int32_t* flags);

/* Free a plan (NULL is accepted).  No run of it may still be pending. */
int32_t vpk_plan_destroy(vpk_plan plan);

/*
 * vpk_set_workspace -- give the direct calls on `stream` (of the current
 * device) caller-owned device memory for their workspace; ptr NULL goes back
 * to the library's own.  The flash-attention page's interface leaves every
 * buffer with the caller's tensors ("Add flash_attn_varlen_func_with_kvcache",
 * Usage); this is the same for the scratch memory.
 *   ptr     device memory, 256-byte aligned, at least 4608 bytes, borrowed:
 *           it must stay valid, and untouched by anything else, until the
 *           work of every call on `stream` that used it has run (replacing or
 *           freeing it in stream order after those calls is fine).
 *   bytes   its size.  A call needs at most
 *           vpk_workspace_bytes_upper_bound(dims, ...) bytes; with less the
 *           planner splits key ranges less (the results stay within the same
 *           tolerances), and a call whose unsplit needs do not fit returns
 *           VPK_ERROR_CAPACITY before anything is enqueued.
 * The first 512 bytes are cleared on `stream` (error flag and zero rows).
 * Not during stream capture (VPK_ERROR_NOT_SUPPORTED).
 */
int32_t vpk_set_workspace(void* stream, void* ptr, size_t bytes);

/*
 * vpk_workspace_bytes_upper_bound -- device bytes that suffice for the
 * workspace of any direct call with these sizes (any lengths, any split the
 * planner may choose): head, split partials (at most 2^17 rows of
 * (head_dim + 1) floats), the plan records, and with rope != 0 the turned
 * copies of q and k_new.  num_cus <= 0: those of the current device.
 * Host only; returns 0 for invalid dims.
 */
size_t vpk_workspace_bytes_upper_bound(const vpk_dims* dims, int32_t num_cus, int32_t rope);

/*
 * vpk_qkv_prob_score_bytes -- device bytes, beyond the bound above, with which
 * attn_varlen_paged_qkv_prob_fwd keeps the first-pass scores of its
 * decode-mode rows in the workspace (sequences of at most 8 packed rows,
 * q_len * num_q_heads / num_kv_heads, with head_dim 128): 128 bytes per row
 * and 32 keys of each kv head, a quarter or less of re-reading the K codes in
 * the second pass.  A workspace without this room gives the same results
 * (the second pass reads K again).  From the host arrays cu_seqlens_q,
 * cu_seqlens_knew and cache_seqlens of `host` (the latter two may be NULL:
 * no new tokens / no cache).  Host only; returns 0 for invalid arguments or
 * when no row qualifies.
 */
size_t vpk_qkv_prob_score_bytes(const vpk_dims* dims, const vpk_host_index* host);

/* Memory the library holds on its own: device bytes of its fallback
 * workspaces (streams without vpk_set_workspace) and pinned host bytes of its
 * plan buffers.  Prepared plans are not counted (each owns its buffer). */
int32_t vpk_library_memory(size_t* device_bytes, size_t* pinned_bytes);

/* Message describing the calling thread's last non-success status ("" if none). */
const char* vpk_last_error(void);

/* VPK_ABI_VERSION of the loaded library. */
int32_t vpk_abi_version(void);

/*
 * Tuning / test knobs (process-wide).  Names:
 *   "force_splits"     0 = planner decides; n >= 1 = split every work item's
 *                      key range into n parts (tests of the merge pass).
 *   "persistent"       -1 = planner decides (default; persistent grids), 0 = one
 *                      work item per workgroup,
 *                      1 = persistent grid with static per-workgroup queues.
 *   "split_min_keys"   smallest key range of a split part (default 256).
 *   "num_cus"          compute units assumed by the planner (0 = query device).
 *   "mixed_grid"       for a call with both prefill-mode items (more than 32
 *                      packed rows per kv head) and decode-mode items: 1 = one
 *                      launch of 512-thread workgroups, prefill tiles first;
 *                      0 = two grids (side by side for direct calls, one after
 *                      the other for prepared ones and the allocation-free
 *                      form); -1 (default) = two grids side by side for direct
 *                      calls, one launch where they would run one after the
 *                      other.  Plans built while it is 0 have no one-launch grid.
 *   "mixed_dec_parts"  decode-mode split size in such a call: parts of the
 *                      total decode work / (num_cus * this); default 1.
 *   "plan_upload"      0 = the kernels read a direct call's work list from
 *                      pinned host memory (default); 1 = it is copied into the
 *                      workspace on the call's stream first.
 *   "plan_reuse"       1 (default) = a direct call with a caller's workspace
 *                      whose work list has the same bytes as the previous
 *                      call's on its stream (same lengths, options and
 *                      workspace, as in every layer of a model step) has it
 *                      copied once, on the stream, to the end of that
 *                      workspace, and the calls after it read the copy
 *                      instead of pinned host memory; the copy is dropped
 *                      when a call brings another work list, when a call's
 *                      partials reach it, or when the workspace is replaced.
 *                      0 = always the pinned buffer.  Same results either way.
 *   "keep_scores"      QKV-Prob calls: 1 (default) = decode-mode rows keep
 *                      their first-pass scores in the workspace when it has
 *                      room (vpk_qkv_prob_score_bytes); 0 = the second pass
 *                      reads K again.  Same results either way.
 *   "plan_log"         1 = print one line per planned call on stderr: units
 *                      and workgroups of each launch ("q" marks persistent
 *                      queues), split tiles, partial rows, bytes of plan
 *                      records and device work memory; 0 = off; -1 (default)
 *                      = on when the environment variable VPK_LOG is set to
 *                      a value other than 0 (read at the first call).
 * Returns VPK_ERROR_INVALID_VALUE for an unknown name or value.
 */
int32_t vpk_set_option(const char* name, int64_t value);

/*
 * Kernel timing: when enabled, every launch of the library's kernels is
 * bracketed by HIP events recorded on the launch stream.  vpk_timing_read
 * synchronises those events and returns the summed milliseconds and the
 * launch count per kernel since the last reset.
 *   kernel: 0 = attention grid of prefill-mode items (sequences with more
 *               than 32 packed rows; may include the append of a bf16 cache),
 *           1 = append launched on its own (fp8 cache, persistent schedule,
 *               or kv_cache_append),
 *           2 = attention grid of decode-mode items (likewise),
 *           3 = LSE merge of split parts,
 *           4 = rotary embedding of the rows turned into copies before attention,
 *           5 = mixed attention grid (prefill-mode and decode-mode items of one
 *               call in one launch, option "mixed_grid"),
 *           6 = fp8 QKV-Prob attention grid (attn_varlen_paged_qkv_prob_fwd).
 */
int32_t vpk_timing_enable(int32_t enable);
int32_t vpk_timing_reset(void);
int32_t vpk_timing_read(int32_t kernel, double* total_ms, int64_t* launches);

/* Synchronise `stream` and return (and clear) the device error flag of its
 * workspace: bit 0 = a page id outside [0, num_pages) was met. */
int32_t vpk_device_error(void* stream, int32_t* flags);

/*
 * Planner introspection (host only, needs no GPU): build the work list the
 * attention launches would use and copy it out.  Each item is 8 int32:
 *   {seq, row0, nrows, kv_head, key_begin, key_end, part, queue}
 * where rows are packed (token * g + head-in-group) and part >= 0 marks a
 * split part whose result goes through the merge pass.  Items with more than
 * 32 rows come first (prefill-mode grid), then the others (decode-mode grid).
 * Each grid is either persistent (static per-workgroup queues) or runs one
 * workgroup per item: `queue` is the item's queue, numbered over the
 * persistent grids in launch order, or -1; *n_queues counts the queues.
 * `num_cus` as for the "num_cus" option (> 0 here).  Returns
 * VPK_ERROR_CAPACITY with *n_items set when `capacity` is too small.
 */
int32_t vpk_plan_debug(const vpk_dims* dims, const vpk_host_index* host,
                       int32_t has_cache, int32_t has_new, int32_t page_size,
                       int32_t causal, int32_t num_cus,
                       int32_t* items, int32_t capacity, int32_t* n_items,
                       int32_t* n_queues);

#ifdef __cplusplus
}
#endif

#endif /* VPK_H_ */
