// C ABI of libvpk: argument checks, host mirrors, planning, workspace and
// launches.  Nothing here throws across the boundary; every failure becomes a
// vpk_status plus a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "vpk.h"
#include "../vpk_internal.h"
#include "plan.h"

namespace {

using vpk::AppendParams;
using vpk::AttnParams;
using vpk::MergeGroup;
using vpk::MergeParams;
using vpk::Plan;
using vpk::PlanInput;
using vpk::SeqInfo;
using vpk::WorkItem;

thread_local std::string g_err;

int32_t fail(int32_t code, const std::string& msg) {
  g_err = msg;
  return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(VPK_ERROR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct Options {
  std::atomic<int64_t> force_splits{0};
  std::atomic<int64_t> persistent{-1};
  std::atomic<int64_t> split_min_keys{256};
  std::atomic<int64_t> num_cus{0};
  std::atomic<int64_t> plan_upload{0};
  std::atomic<int64_t> mixed_grid{-1};
  std::atomic<int64_t> mixed_dec_parts{1};
  std::atomic<int64_t> plan_log{-1};   // -1: VPK_LOG from the environment
  std::atomic<int64_t> keep_scores{1};
  std::atomic<int64_t> plan_reuse{1};
} g_opt;

// ------------------------------------------------------------------ timing

struct TimingRec {
  int kernel;
  hipEvent_t a, b;
};
std::mutex g_tmu;
std::atomic<bool> g_timing{false};
std::vector<TimingRec> g_tpending;
std::vector<hipEvent_t> g_tfree;
constexpr int kTimedKernels = 7;   // 0 prefill-mode attention grid, 1 append, 2 decode-mode attention grid, 3 merge,
                                   // 4 rotary embedding, 5 mixed attention grid, 6 fp8 QKV-Prob attention grid
double g_tms[kTimedKernels] = {0, 0, 0, 0, 0, 0, 0};
int64_t g_tcount[kTimedKernels] = {0, 0, 0, 0, 0, 0, 0};

hipEvent_t take_event() {
  if (!g_tfree.empty()) {
    hipEvent_t e = g_tfree.back();
    g_tfree.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct KernelTimer {
  int kernel;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  KernelTimer(int k, hipStream_t st) : kernel(k), s(st) {
    if (!g_timing.load()) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    a = take_event();
    b = take_event();
    if (a && b) (void)hipEventRecord(a, s);
  }
  ~KernelTimer() {
    if (!a || !b) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_tmu);
    g_tpending.push_back(TimingRec{kernel, a, b});
  }
};

// --------------------------------------------------------------- workspace

// new tokens stored by one workgroup of the standalone append kernel
constexpr int kAppendTokensStandalone = 8;

// workspace head: [0, 256) error flag, [256, 512) zeros (never written)
constexpr size_t kFlagBytes = 512;
constexpr size_t kZerosOffset = 256;

// Plans live in pinned host memory that the kernels read directly (each
// workgroup reads its unit and sequence records once): no copy, no copy
// stream, no cross-stream dependency on the critical path.  A ring of buffers
// lets the host plan ahead of the GPU; a buffer is reused once an event
// recorded behind the last kernel that read it has completed.  One event is
// recorded per kPlanCover calls (each record costs the stream a few
// microseconds): buffer k's use is covered by the event that the call with
// buffer k | (kPlanCover - 1) records after it.
constexpr int kPlanRing = 8;
constexpr int kPlanCover = 4;
static_assert(kPlanRing % kPlanCover == 0, "whole groups in the ring");

struct PlanBuf {
  char* host = nullptr;      // pinned, device-accessible
  size_t bytes = 0;
  hipEvent_t ev = nullptr;   // recorded after the kernels of the call that used this buffer (every kPlanCover-th)
  bool used = false;         // read by enqueued work that no recorded event covers yet
  int cover = -1;            // the buffer whose event covers this buffer's last use (-1: none pending)
};

// Split-partial rows one call may use at most, whatever its workspace (the
// planner scales its splits down to stay within it; the workloads measured
// here use at most a quarter of it).
constexpr int64_t kPartRowsCap = int64_t(1) << 17;

struct Workspace {
  int device = -1;
  // library-owned device memory (fallback): [flag | zeros][split partials, rope copies][plan records]
  char* dev = nullptr;
  size_t bytes = 0;
  size_t part_cap = 0;
  // caller-owned device memory (vpk_set_workspace), same layout; used instead of `dev` when set
  char* user = nullptr;
  size_t user_bytes = 0;
  PlanBuf plan[kPlanRing];
  int next = 0;
  // side stream for running the decode-mode grid next to the prefill-mode grid
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr;
  hipEvent_t ev_join = nullptr;
  // Plan reuse: the work list of the last direct call on this stream (its
  // bytes), and whether a copy of it sits at the end of the caller's
  // workspace, at offset rec_off
  std::vector<char> rec;
  int rec_state = 0;         // 0 none, 1 seen once (not copied), 2 copied
  size_t rec_off = 0;
  char* head() const { return user ? user : dev; }
  char* parts() const { return head() + kFlagBytes; }
};

int32_t ensure_aux(Workspace* w) {
  if (w->aux) return VPK_SUCCESS;
  hipError_t e = hipStreamCreateWithFlags(&w->aux, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags (side stream)");
  if ((e = hipEventCreateWithFlags(&w->ev_fork, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "hipEventCreate (fork)");
  if ((e = hipEventCreateWithFlags(&w->ev_join, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "hipEventCreate (join)");
  return VPK_SUCCESS;
}

std::mutex g_wmu;
std::map<std::pair<int, void*>, Workspace*> g_ws;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The bookkeeping of (current device, stream), created on first use.
int32_t find_workspace(hipStream_t stream, Workspace** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_wmu);
  Workspace*& w = g_ws[std::make_pair(dev, static_cast<void*>(stream))];
  if (!w) {
    w = new (std::nothrow) Workspace();
    if (!w) return fail(VPK_ERROR_OUT_OF_MEMORY, "workspace bookkeeping");
    w->device = dev;
  }
  *out = w;
  return VPK_SUCCESS;
}

// The workspace of (current device, stream) with `part_need` bytes after its
// head in device memory: the caller's (which must hold them) or the library's
// own, grown as needed.
int32_t get_workspace(hipStream_t stream, size_t part_need, Workspace** out) {
  Workspace* w = nullptr;
  int32_t st = find_workspace(stream, &w);
  if (st) return st;
  *out = w;
  if (w->user) {
    // a call whose partials reach the reused work list's copy overwrites it
    if (w->rec_state == 2 && kFlagBytes + part_need > w->rec_off) w->rec_state = 0;
    if (kFlagBytes + part_need > w->user_bytes)
      return fail(VPK_ERROR_CAPACITY, "the workspace set with vpk_set_workspace holds " + std::to_string(w->user_bytes) +
                                          " bytes, this call needs " + std::to_string(kFlagBytes + part_need) +
                                          " (see vpk_workspace_bytes_upper_bound)");
    return VPK_SUCCESS;
  }
  hipError_t e;
  std::lock_guard<std::mutex> lk(g_wmu);
  if (!w->dev || w->part_cap < part_need) {
    if (w->dev) {
      // everything that may still read the old buffer is on these streams
      if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize (workspace growth)");
      if (w->aux && (e = hipStreamSynchronize(w->aux)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize (side stream)");
      (void)hipFree(w->dev);
      w->dev = nullptr;
      w->bytes = 0;
    }
    const size_t qc = align_up(std::max(part_need + part_need / 2, w->part_cap), 4096);
    const size_t bytes = kFlagBytes + qc;
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return fail(VPK_ERROR_OUT_OF_MEMORY, std::string("hipMalloc workspace: ") + hipGetErrorString(e));
    e = hipMemset(p, 0, kFlagBytes);   // error flag and zero rows
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "hipMemset workspace head");
    }
    w->dev = static_cast<char*>(p);
    w->bytes = bytes;
    w->part_cap = qc;
  }
  *out = w;
  return VPK_SUCCESS;
}

// The next plan buffer with room for `bytes`, once the GPU is done with it.
int32_t take_plan_buffer(Workspace* w, size_t bytes, hipStream_t stream, int* index) {
  const int k = w->next;
  w->next = (w->next + 1) % kPlanRing;
  PlanBuf& pb = w->plan[k];
  hipError_t e;
  if (!pb.ev && (e = hipEventCreateWithFlags(&pb.ev, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "hipEventCreate (plan buffer)");
  if (pb.used) {
    // no event covers its last use (a call of its group failed before its
    // release): one recorded now covers everything enqueued so far
    if ((e = hipEventRecord(pb.ev, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord (plan buffer)");
    pb.used = false;
    pb.cover = k;
  }
  if (pb.cover >= 0) {
    e = hipEventSynchronize(w->plan[pb.cover].ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (plan buffer)");
    pb.cover = -1;
  }
  if (pb.bytes < bytes) {
    if (pb.host) (void)hipHostFree(pb.host);
    pb.host = nullptr;
    pb.bytes = 0;
    const size_t nb = align_up(std::max(bytes + bytes / 2, static_cast<size_t>(64) << 10), 4096);
    e = hipHostMalloc(reinterpret_cast<void**>(&pb.host), nb, hipHostMallocDefault);
    if (e != hipSuccess) return fail(VPK_ERROR_OUT_OF_MEMORY, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    pb.bytes = nb;
  }
  *index = k;
  return VPK_SUCCESS;
}

// Plan reuse (option plan_reuse): the kernels of a direct call read its
// work list (`bytes` bytes at R, in pinned host memory) over PCIe.  Every
// layer of a model step calls with the same lengths and so writes the same
// bytes: when they equal the previous call's on this stream, the list is
// copied once, on `stream`, to the end of the caller's workspace, and the
// calls after it read that copy (device memory) until a call brings other
// bytes or its partials reach the copy.  The first call with new bytes reads
// them from pinned memory as before, so calls whose lengths keep changing
// pay only the comparison on the host.
int32_t reuse_plan(Workspace* w, size_t bytes, size_t part_end, hipStream_t stream, char** R) {
  if (g_opt.plan_reuse.load() == 0 || !w->user) return VPK_SUCCESS;
  const size_t need = align_up(bytes, 256);
  if (kFlagBytes + part_end + need > w->user_bytes) {
    w->rec_state = 0;
    return VPK_SUCCESS;
  }
  const size_t off = (w->user_bytes - need) / 256 * 256;
  const bool same = w->rec_state > 0 && w->rec.size() == bytes && std::memcmp(w->rec.data(), *R, bytes) == 0;
  if (!same) {
    w->rec.assign(*R, *R + bytes);
    w->rec_state = 1;
    return VPK_SUCCESS;
  }
  if (w->rec_state == 1 || w->rec_off != off) {
    const hipError_t e = hipMemcpyAsync(w->user + off, *R, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (reused work list)");
    w->rec_state = 2;
    w->rec_off = off;
  }
  *R = w->user + off;
  return VPK_SUCCESS;
}

// Mark plan buffer k as read by everything enqueued on `stream` so far; the
// last buffer of each group of kPlanCover records the event that covers the
// group's uses.
int32_t release_plan_buffer(Workspace* w, hipStream_t stream, int k) {
  w->plan[k].used = true;
  if (k % kPlanCover != kPlanCover - 1) return VPK_SUCCESS;
  const hipError_t e = hipEventRecord(w->plan[k].ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (plan buffer)");
  for (int j = k - (kPlanCover - 1); j <= k; ++j)
    if (w->plan[j].used) {
      w->plan[j].used = false;
      w->plan[j].cover = k;
    }
  return VPK_SUCCESS;
}

// ---------------------------------------------------------- host mirrors

int32_t fetch_index(const int32_t* dev, size_t n, hipStream_t stream, std::vector<int32_t>& buf,
                    const int32_t** out) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(VPK_ERROR_NOT_SUPPORTED, "host mirrors are required during stream capture");
  buf.resize(n);
  if (n) {
    hipError_t e = hipMemcpyAsync(buf.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (index array to host)");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (index array to host)");
  }
  *out = buf.data();
  return VPK_SUCCESS;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Direct calls plan on the host and hand the kernels a plan buffer from a
// ring that the next calls reuse, and may grow their workspace: a graph
// captured around one would replay a later call's work list.  They refuse
// stream capture; prepared calls (vpk_plan_create / vpk_plan_run) are the
// capturable form.
int32_t refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(VPK_ERROR_NOT_SUPPORTED,
                "direct calls cannot be captured into a graph: use vpk_plan_create / vpk_plan_run");
  return VPK_SUCCESS;
}

struct Mirrors {
  const int32_t* cu_q = nullptr;
  const int32_t* cu_kn = nullptr;
  const int32_t* cache_lens = nullptr;
  const int32_t* block_table = nullptr;   // may stay null (no host check)
  // page-list form: each sequence's own query rows and page-id range
  const int32_t* q_start = nullptr;       // with q_len instead of cu_q
  const int32_t* q_len = nullptr;
  const int32_t* bt_row = nullptr;        // kv_indptr: first page-id index per sequence (B + 1 entries)
  std::vector<int32_t> b1, b2, b3;
};

struct Call {
  const vpk_dims* d;
  bool has_new, has_cache, fp8;
  int32_t page_size;
  const float* kv_scale;                  // host {k_scale, v_scale} (fp8)
  const float* kv_scale_dev = nullptr;    // or the same in device memory, read by the kernels
  const float* qp_scale = nullptr;        // fp8 QKV-Prob attention: host {q_scale, p_scale}
};

int32_t check_cu(const int32_t* cu, int32_t B, int32_t total, const char* name) {
  if (cu[0] != 0) return fail(VPK_ERROR_INVALID_VALUE, std::string(name) + "[0] must be 0");
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return fail(VPK_ERROR_INVALID_VALUE, std::string(name) + " must be non-decreasing");
  if (cu[B] != total)
    return fail(VPK_ERROR_INVALID_VALUE, std::string(name) + "[batch] must equal the total length");
  return VPK_SUCCESS;
}

// Shape/pointer checks that need no index contents.
int32_t check_dims(const Call& c) {
  const vpk_dims* d = c.d;
  if (!d) return fail(VPK_ERROR_INVALID_VALUE, "dims is NULL");
  if (d->batch < 0 || d->total_q < 0 || d->total_knew < 0)
    return fail(VPK_ERROR_INVALID_VALUE, "negative batch or length");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(VPK_ERROR_INVALID_VALUE, "head counts must be positive");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(VPK_ERROR_INVALID_VALUE, "num_q_heads must be a multiple of num_kv_heads");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(VPK_ERROR_NOT_SUPPORTED, "head_dim must be 64 or 128");
  if (static_cast<int64_t>(d->total_q) * d->num_q_heads > INT32_MAX ||
      static_cast<int64_t>(d->total_knew) * d->num_kv_heads > INT32_MAX)
    return fail(VPK_ERROR_NOT_SUPPORTED, "too many rows for 32-bit row indices");
  if (c.has_cache) {
    if (c.page_size < 1) return fail(VPK_ERROR_INVALID_VALUE, "page_size must be >= 1");
    if (d->num_pages < 1) return fail(VPK_ERROR_INVALID_VALUE, "num_pages must be >= 1 with a cache");
    if (d->max_pages_per_seq < 1) return fail(VPK_ERROR_INVALID_VALUE, "max_pages_per_seq must be >= 1");
    if (static_cast<int64_t>(d->num_pages) * c.page_size > INT32_MAX ||
        static_cast<int64_t>(d->max_pages_per_seq) * c.page_size > INT32_MAX)
      return fail(VPK_ERROR_NOT_SUPPORTED, "too many cache slots for 32-bit slot indices");
    if (d->kv_cache_dtype != VPK_DTYPE_BF16 && d->kv_cache_dtype != VPK_DTYPE_FP8_E4M3FN)
      return fail(VPK_ERROR_INVALID_VALUE, "kv_cache_dtype must be VPK_DTYPE_BF16 or VPK_DTYPE_FP8_E4M3FN");
    if (c.fp8) {
      if (!c.kv_scale) return fail(VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache");
      for (int i = 0; i < 2; ++i)
        if (!std::isfinite(c.kv_scale[i]) || !(c.kv_scale[i] > 0.f))
          return fail(VPK_ERROR_INVALID_VALUE, "kv_scale entries must be finite and > 0");
    }
  }
  return VPK_SUCCESS;
}

int32_t get_mirrors(const Call& c, const int32_t* cu_q_dev, const int32_t* cu_kn_dev,
                    const int32_t* cl_dev, const vpk_host_index* host, hipStream_t stream,
                    bool need_q, Mirrors& m) {
  const int32_t B = c.d->batch;
  int32_t st;
  if (need_q) {
    if (host && host->cu_seqlens_q) m.cu_q = host->cu_seqlens_q;
    else if ((st = fetch_index(cu_q_dev, B + 1, stream, m.b1, &m.cu_q)) != VPK_SUCCESS) return st;
  }
  if (c.has_new) {
    if (host && host->cu_seqlens_knew) m.cu_kn = host->cu_seqlens_knew;
    else if ((st = fetch_index(cu_kn_dev, B + 1, stream, m.b2, &m.cu_kn)) != VPK_SUCCESS) return st;
  }
  if (c.has_cache) {
    if (host && host->cache_seqlens) m.cache_lens = host->cache_seqlens;
    else if ((st = fetch_index(cl_dev, B, stream, m.b3, &m.cache_lens)) != VPK_SUCCESS) return st;
    if (host && host->block_table) m.block_table = host->block_table;
  }
  return VPK_SUCCESS;
}

// Length and page checks on the host mirrors.
int32_t check_contents(const Call& c, const Mirrors& m, bool need_q) {
  const vpk_dims* d = c.d;
  const int32_t B = d->batch;
  int32_t st;
  if (need_q && (st = check_cu(m.cu_q, B, d->total_q, "cu_seqlens_q")) != VPK_SUCCESS) return st;
  if (c.has_new && (st = check_cu(m.cu_kn, B, d->total_knew, "cu_seqlens_knew")) != VPK_SUCCESS) return st;
  if (c.has_cache) {
    for (int32_t b = 0; b < B; ++b) {
      const int64_t lc = m.cache_lens[b];
      if (lc < 0) return fail(VPK_ERROR_INVALID_VALUE, "cache_seqlens must be >= 0");
      const int64_t ln = c.has_new ? m.cu_kn[b + 1] - m.cu_kn[b] : 0;
      const int64_t lk = lc + ln;
      if (lk > static_cast<int64_t>(d->max_pages_per_seq) * c.page_size)
        return fail(VPK_ERROR_CAPACITY, "sequence " + std::to_string(b) + " needs " +
                                            std::to_string(lk) + " slots, block_table row holds " +
                                            std::to_string(static_cast<int64_t>(d->max_pages_per_seq) * c.page_size));
      if (m.block_table) {
        const int64_t np = (lk + c.page_size - 1) / c.page_size;
        const int32_t* row = m.block_table + static_cast<int64_t>(b) * d->max_pages_per_seq;
        for (int64_t i = 0; i < np; ++i)
          if (row[i] < 0 || row[i] >= d->num_pages)
            return fail(VPK_ERROR_INVALID_VALUE, "block_table[" + std::to_string(b) + "][" +
                                                     std::to_string(i) + "] = " + std::to_string(row[i]) +
                                                     " is outside [0, num_pages)");
      }
    }
  }
  return VPK_SUCCESS;
}

int32_t device_cus() {
  const int64_t forced = g_opt.num_cus.load();
  if (forced > 0) return static_cast<int32_t>(forced);
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

// fp8 cache, head_dim 128, new tokens, keys not turned: the decode-mode items
// may form and store their sequences' new token codes themselves (the group
// size g is returned; 0: the standalone append stores every new token)
int32_t dec_append_g(const Call& c, bool key_rope) {
  if (!c.fp8 || !c.has_cache || !c.has_new || c.qp_scale || key_rope || c.d->head_dim != 128) return 0;
  return c.d->num_q_heads / c.d->num_kv_heads;
}

void fill_plan_input(const Call& c, const Mirrors& m, int32_t causal, int32_t num_cus, PlanInput& in) {
  in.batch = c.d->batch;
  in.hq = c.d->num_q_heads;
  in.hkv = c.d->num_kv_heads;
  in.head_dim = c.d->head_dim;
  in.has_cache = c.has_cache;
  in.has_new = c.has_new;
  in.causal = causal != 0;
  in.page_size = c.has_cache ? c.page_size : 1;
  in.kv_bytes = c.fp8 ? 1 : 2;
  in.cu_q = m.cu_q;
  in.cu_kn = m.cu_kn;
  in.cache_lens = m.cache_lens;
  in.q_start = m.q_start;
  in.q_len = m.q_len;
  in.bt_row = m.bt_row;
  in.max_pages = c.d->max_pages_per_seq;
  in.num_cus = num_cus;
  in.force_splits = static_cast<int32_t>(g_opt.force_splits.load());
  in.persistent = static_cast<int32_t>(g_opt.persistent.load());
  in.split_min_keys = static_cast<int32_t>(g_opt.split_min_keys.load());
  in.max_part_rows = kPartRowsCap;
  in.mixed = g_opt.mixed_grid.load() != 0;
  in.mixed_dec_parts = static_cast<int32_t>(g_opt.mixed_dec_parts.load());
}

// ---- workspace sizes.  Bounds over every call with the sizes of `d` (any
//      lengths), for a workspace laid out as [head][split partials, rope
//      copies][plan records].

// most parts one tile is cut into: the split limit, or the parts a key range
// needs so that each fits the LDS page-id list (ceil(max_pages / 1023) + 1)
int64_t parts_per_tile_bound(const vpk_dims* d) {
  return std::max<int64_t>(vpk::kMaxSplits, d->max_pages_per_seq / (vpk::kMaxItemPages - 1) + 2);
}

size_t part_bytes_for(int64_t rows, int32_t D) {
  return align_up(sizeof(float) * static_cast<size_t>(D) * rows, 256) + align_up(sizeof(float) * rows, 256);
}

size_t rope_bytes_for(const vpk_dims* d) {
  return align_up(2 * static_cast<size_t>(d->total_q) * d->num_q_heads * d->head_dim, 256) +
         align_up(2 * static_cast<size_t>(d->total_knew) * d->num_kv_heads * d->head_dim, 256);
}

size_t plan_bytes_bound(const vpk_dims* d, int32_t num_cus, bool rope) {
  const int64_t B = d->batch, hkv = d->num_kv_heads, g = d->num_q_heads / d->num_kv_heads;
  const int64_t tiles = B + (static_cast<int64_t>(d->total_q) * g + vpk::kPrefillRows - 1) / vpk::kPrefillRows;
  const int64_t units = tiles * parts_per_tile_bound(d);
  const int64_t queue_starts = 2 * (2 * static_cast<int64_t>(std::max(num_cus, 1)) + 1);
  size_t b = sizeof(SeqInfo) * B + 2 * sizeof(int32_t) * static_cast<size_t>(d->total_knew) +
             sizeof(WorkItem) * units + sizeof(MergeGroup) * tiles * hkv + sizeof(int32_t) * queue_starts +
             sizeof(int32_t) * units * hkv;
  if (rope) b += sizeof(int32_t) * (static_cast<size_t>(d->total_q) + d->total_knew);
  return align_up(b + 8 * 64, 256);
}

int64_t part_rows_bound(const vpk_dims* d) {
  return std::min<int64_t>(kPartRowsCap,
                           parts_per_tile_bound(d) * static_cast<int64_t>(d->total_q) * d->num_q_heads);
}

// split-partial rows that fit a workspace of `bytes` next to everything else a call puts there
int64_t part_rows_fitting(size_t bytes, const vpk_dims* d, int32_t num_cus, bool rope, bool plan_inside) {
  const size_t fixed = kFlagBytes + 512 + (rope ? rope_bytes_for(d) : 0) +
                       (plan_inside ? plan_bytes_bound(d, num_cus, rope) : 0);
  if (bytes <= fixed) return 0;
  return static_cast<int64_t>((bytes - fixed) / (sizeof(float) * (static_cast<size_t>(d->head_dim) + 1)));
}

// Plan buffer layout (pinned host memory, offsets from its start):
//   [seqs][new tokens: sequence, position][units][merge groups][queue starts][queue work]
// Partials area (device memory): [part_o fp32 rows x D][part_lse fp32 rows]
struct Layout {
  size_t seqs, tok, items, groups, queues, work, qpos, kpos, plan_end, part_o, part_lse, rot_q, rot_k, scores,
      part_end;
};

// Rotary embedding (`rope` set): the positions of the query rows and new
// tokens go into the plan; turned copies of q (rows the attention kernels do
// not turn themselves) and of k_new (a call without a cache) go into device
// memory after the split partials.
struct RopeCopies {
  bool positions = false;
  bool q = false;
  bool k = false;
};

// QKV-Prob decode-mode units of at most this many rows keep their scores
// between the two passes (above it, storing and reloading them moves more
// bytes than reading the K codes again)
constexpr int32_t kKeepScoreRows = 8;

// Plan log: one line per planned call on stderr with the plan's shape --
// units and workgroups of each launch, split tiles, partial rows and the
// bytes of plan records and device work memory -- to see what the planner
// made of a batch without a profiler.  On with VPK_LOG=1 in the environment
// (read at the first call) or option "plan_log" = 1; option 0 turns it off.
bool plan_log_on() {
  static const bool env_on = [] {
    const char* v = std::getenv("VPK_LOG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
  }();
  const int64_t o = g_opt.plan_log.load();
  return o < 0 ? env_on : o != 0;
}

void log_plan(const char* entry, const Plan& p, const vpk_dims* d, size_t plan_bytes, size_t work_bytes) {
  if (!plan_log_on()) return;
  auto mode = [](const vpk::Launch& L) { return L.persistent ? "q" : ""; };
  std::fprintf(stderr,
               "vpk: %s batch=%d q_rows=%d new_rows=%d hq=%d hkv=%d D=%d | units pre=%d dec=%d | "
               "workgroups pre=%d%s dec=%d%s one=%d%s (q: persistent queues) | split tiles=%zu part_rows=%lld | "
               "plan_bytes=%zu device_work_bytes=%zu\n",
               entry, d->batch, d->total_q, d->total_knew, d->num_q_heads, d->num_kv_heads, d->head_dim,
               p.prefill.count, p.decode.count, p.prefill.grid, mode(p.prefill), p.decode.grid, mode(p.decode),
               p.mixed.grid, mode(p.mixed),
               p.groups.size() / std::max<size_t>(1, static_cast<size_t>(d->num_kv_heads)),
               static_cast<long long>(p.part_rows), plan_bytes, work_bytes);
  std::fflush(stderr);
}

Layout layout_for(const Plan& p, int32_t B, int32_t Tn, int32_t D, const vpk_dims* rope = nullptr,
                  RopeCopies rc = RopeCopies{}, size_t score_bytes = 0) {
  Layout L;
  L.seqs = 0;
  L.tok = align_up(L.seqs + sizeof(SeqInfo) * B, 64);
  L.items = align_up(L.tok + 2 * sizeof(int32_t) * static_cast<size_t>(Tn), 64);
  L.groups = align_up(L.items + sizeof(WorkItem) * p.items.size(), 64);
  L.queues = align_up(L.groups + sizeof(MergeGroup) * p.groups.size(), 64);
  L.work = align_up(L.queues + sizeof(int32_t) * p.queue_start.size(), 64);
  L.qpos = align_up(L.work + sizeof(int32_t) * p.queue_work.size(), 64);
  const size_t tq = rope ? static_cast<size_t>(rope->total_q) : 0, tn = rope ? static_cast<size_t>(Tn) : 0;
  L.kpos = align_up(L.qpos + sizeof(int32_t) * tq, 64);
  L.plan_end = align_up(L.kpos + sizeof(int32_t) * tn, 256);
  L.part_o = 0;
  L.part_lse = align_up(sizeof(float) * D * static_cast<size_t>(p.part_rows), 256);
  L.rot_q = align_up(L.part_lse + sizeof(float) * static_cast<size_t>(p.part_rows), 256);
  const size_t hq = rope ? static_cast<size_t>(rope->num_q_heads) : 0, hkv = rope ? static_cast<size_t>(rope->num_kv_heads) : 0;
  L.rot_k = align_up(L.rot_q + (rc.q ? 2 * tq * hq * D : 0), 256);
  L.scores = align_up(L.rot_k + (rc.k ? 2 * tn * hkv * D : 0), 256);
  L.part_end = align_up(L.scores + score_bytes, 256);
  return L;
}

// Serialise the plan records into `base` (L.plan_end bytes).  New token j of
// sequence b sits at logical position Lc + j: its record is the block_table
// index of that position's page id (the sequence's first index + pos / S)
// and the slot pos % S, so an append workgroup finds its tokens' slots with
// one read each.
// A decode-mode sequence (0 < q_len * g <= 32 packed rows) of a call whose
// decode-mode items store their own new tokens (dec_g > 0: the group size).
bool dec_stores_own(const SeqInfo& s, int32_t dec_g) {
  return dec_g > 0 && s.q_len > 0 && static_cast<int64_t>(s.q_len) * dec_g <= vpk::kWaveRows;
}

// The group size for a plan of decode-mode units only in which every
// sequence with new tokens is such a decode-mode sequence, else 0: the
// decode-mode items then store all new tokens and the standalone append is
// not launched (so its records need no change).  (Forming the codes in the item that reads them puts a
// dependent read of the new rows into that item's last block; on the mixed
// fp8 batch, whose prefill-mode tokens still need the append first, that
// cost more than it saved.)
int32_t dec_own_g(const Plan& p, int32_t dec_g) {
  if (dec_g <= 0 || p.num_pre_units > 0) return 0;
  for (const SeqInfo& s : p.seqs)
    if (s.new_len > 0 && !dec_stores_own(s, dec_g)) return 0;
  return dec_g;
}

void serialize_plan(const Plan& p, const Layout& L, const int32_t* cu_kn, int32_t B, int32_t page_size,
                    char* base) {
  if (B) std::memcpy(base + L.seqs, p.seqs.data(), sizeof(SeqInfo) * B);
  if (cu_kn) {
    int32_t* tok = reinterpret_cast<int32_t*>(base + L.tok);
    const int32_t S = std::max(1, page_size);
    for (int32_t b = 0; b < B; ++b)
      for (int32_t t = cu_kn[b]; t < cu_kn[b + 1]; ++t) {
        const int32_t pos = p.seqs[b].cache_len + (t - cu_kn[b]);
        tok[2 * t] = p.seqs[b].bt_row + pos / S;
        tok[2 * t + 1] = pos % S;
      }
  }
  if (!p.items.empty()) std::memcpy(base + L.items, p.items.data(), sizeof(WorkItem) * p.items.size());
  if (!p.groups.empty()) std::memcpy(base + L.groups, p.groups.data(), sizeof(MergeGroup) * p.groups.size());
  if (!p.queue_start.empty())
    std::memcpy(base + L.queues, p.queue_start.data(), sizeof(int32_t) * p.queue_start.size());
  if (!p.queue_work.empty())
    std::memcpy(base + L.work, p.queue_work.data(), sizeof(int32_t) * p.queue_work.size());
}

// Serialise the plan into the next pinned plan buffer; *index receives it.
int32_t write_plan(Workspace* w, const Plan& p, const Layout& L, const int32_t* cu_kn, int32_t B,
                   int32_t page_size, hipStream_t stream, int* index) {
  int32_t st = take_plan_buffer(w, L.plan_end, stream, index);
  if (st) return st;
  serialize_plan(p, L, cu_kn, B, page_size, w->plan[*index].host);
  return VPK_SUCCESS;
}

// Positions of the rows the rotary embedding turns: query row i of a sequence
// at Lk - Lq + i (the key its end-aligned causal bound stops at), new token j
// at Lc + j (the slot the append writes); rows no sequence names get -1.
// With `g` > 0 only the query rows of decode-mode sequences (q_len * g <= 32
// packed rows) get a position: the others are turned by the prefill-mode
// kernel as it loads them.
void write_rope_positions(const Plan& p, const Layout& L, int32_t B, int32_t Tq, char* base, int32_t g = 0) {
  int32_t* qpos = reinterpret_cast<int32_t*>(base + L.qpos);
  int32_t* kpos = reinterpret_cast<int32_t*>(base + L.kpos);
  std::fill(qpos, qpos + Tq, -1);
  for (int32_t b = 0; b < B; ++b) {
    const SeqInfo& q = p.seqs[b];
    if (g == 0 || static_cast<int64_t>(q.q_len) * g <= vpk::kWaveRows)
      for (int32_t i = 0; i < q.q_len; ++i) qpos[q.q_start + i] = q.kv_len - q.q_len + i;
    for (int32_t j = 0; j < q.new_len; ++j) kpos[q.kn_start + j] = q.cache_len + j;
  }
}

AppendParams append_params(const Call& c, char* head, char* R, const Layout& L,
                           const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_table) {
  const vpk_dims* d = c.d;
  AppendParams ap{};
  ap.k_new = static_cast<const uint16_t*>(k_new);
  ap.v_new = static_cast<const uint16_t*>(v_new);
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.block_table = block_table;
  ap.tok = reinterpret_cast<const int32_t*>(R + L.tok);
  ap.tokens_per_wg = kAppendTokensStandalone;
  ap.err_flag = reinterpret_cast<int32_t*>(head);
  ap.batch = d->batch;
  ap.total_knew = d->total_knew;
  ap.max_pages = d->max_pages_per_seq;
  ap.num_pages = d->num_pages;
  ap.page_size = c.page_size;
  ap.row_elems = d->num_kv_heads * d->head_dim;
  ap.fp8 = c.fp8 ? 1 : 0;
  ap.k_inv_scale = c.fp8 && c.kv_scale ? 1.0f / c.kv_scale[0] : 1.0f;
  ap.v_inv_scale = c.fp8 && c.kv_scale ? 1.0f / c.kv_scale[1] : 1.0f;
  ap.kv_scale_dev = c.fp8 ? c.kv_scale_dev : nullptr;
  return ap;
}

int32_t enqueue_append(const AppendParams& ap, hipStream_t stream) {
  KernelTimer tm(1, stream);
  const int rc = vpk::launch_append(ap, stream);
  if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "append launch");
  return VPK_SUCCESS;
}

int32_t check_ptr(const void* p, size_t a, const char* name) {
  if (!p) return fail(VPK_ERROR_INVALID_VALUE, std::string(name) + " is NULL");
  if (!aligned(p, a)) return fail(VPK_ERROR_INVALID_VALUE, std::string(name) + " is not " + std::to_string(a) + "-byte aligned");
  return VPK_SUCCESS;
}

// Pointer checks shared by a direct call and a prepared plan's run.
int32_t check_run_pointers(const Call& c, const void* q, const void* k_new, const void* v_new,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           float scale, const void* out, const float* lse) {
  const vpk_dims* dims = c.d;
  int32_t st;
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(VPK_ERROR_INVALID_VALUE, "scale must be finite and > 0");
  if (c.has_new && (dims->total_knew > 0 || k_new || v_new)) {
    if ((st = check_ptr(k_new, 16, "k_new")) || (st = check_ptr(v_new, 16, "v_new"))) return st;
  }
  if (!c.has_new && (k_new || v_new)) return fail(VPK_ERROR_INVALID_VALUE, "without new tokens k_new/v_new must be NULL");
  if (c.has_cache) {
    if ((st = check_ptr(k_cache, 16, "k_cache")) || (st = check_ptr(v_cache, 16, "v_cache"))) return st;
    if ((st = check_ptr(block_table, 4, "block_table"))) return st;
  } else if (k_cache || v_cache) {
    return fail(VPK_ERROR_INVALID_VALUE, "without a cache k_cache/v_cache must be NULL");
  }
  if (c.fp8 && c.kv_scale_dev) {
    if (c.kv_scale) return fail(VPK_ERROR_INVALID_VALUE, "give the fp8 scales on the host or on the device, not both");
    if ((st = check_ptr(c.kv_scale_dev, 4, "kv_scale_dev"))) return st;
  } else if (c.fp8) {
    if (!c.kv_scale) return fail(VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache");
    for (int i = 0; i < 2; ++i)
      if (!std::isfinite(c.kv_scale[i]) || !(c.kv_scale[i] > 0.f))
        return fail(VPK_ERROR_INVALID_VALUE, "kv_scale entries must be finite and > 0");
  } else if ((c.kv_scale || c.kv_scale_dev) && c.has_cache) {
    return fail(VPK_ERROR_INVALID_VALUE, "kv_scale must be NULL for a bf16 cache");
  }
  if (dims->total_q > 0) {
    if ((st = check_ptr(q, 16, "q")) || (st = check_ptr(out, 16, "out"))) return st;
    if (lse && !aligned(lse, 4)) return fail(VPK_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
  }
  return VPK_SUCCESS;
}

// Where a call's device-side data lives: the plan records (pinned host
// memory for a direct call, device memory for a prepared plan), the split
// partials, and the head with the error flag and the zero rows.
struct Bases {
  char* R;
  char* PA;
  char* head;
};

// Launch a planned call: the append (fp8 cache, or standalone), the attention
// grids, the merge.  With `side`, a call with both grids runs the decode-mode
// grid on the workspace's side stream next to the prefill-mode grid; without
// it the two grids run one after the other on `stream` (no events: nothing
// here allocates, synchronises or records on another stream, so the whole
// sequence can be captured into a graph).
// `rq`: query rows turned by the attention kernels as they load them; `rk`:
// new keys turned by the append (dim 0: no rotation); `q_dec`: if set, the
// decode-mode grid reads its query rows from there, already turned.
int32_t enqueue_all(const Call& c, const Plan& plan, const Layout& L, const Bases& bs, const void* q,
                    const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* block_table, int32_t causal, float scale, void* out, float* lse,
                    hipStream_t stream, Workspace* side, bool timed, const vpk::RopeArgs& rq = vpk::RopeArgs{},
                    const vpk::RopeArgs& rk = vpk::RopeArgs{}, const void* q_dec = nullptr) {
  const vpk_dims* dims = c.d;
  const float* kv_scale = c.kv_scale;
  const int32_t page_size = c.page_size;
  char* const R = bs.R;
  char* const PA = bs.PA;
  int32_t st;
  const int32_t dec_g = dec_own_g(plan, dec_append_g(c, rk.dim > 0));
  // tokens left to the standalone append (decode-mode items store their own)
  int64_t append_tokens = 0;
  if (c.has_cache && c.has_new)
    for (const SeqInfo& sq : plan.seqs)
      if (!dec_stores_own(sq, dec_g)) append_tokens += sq.new_len;
  const bool do_append = append_tokens > 0;
  AppendParams ap = append_params(c, bs.head, R, L, k_new, v_new, k_cache, v_cache, block_table);
  ap.rope = rk;
  ap.kpos = reinterpret_cast<const int32_t*>(R + L.kpos);
  ap.head_dim = dims->head_dim;
  // bf16 cache: attention reads the new tokens from k_new / v_new (the same
  // bytes the append stores), so the append can run inside an attention grid.
  // fp8 cache, or keys turned by the append: attention must see the stored
  // bytes, so the append runs first.
  const bool new_direct = do_append && !c.fp8 && rk.dim == 0;
  const bool run_pre = plan.prefill.grid > 0 || (c.qp_scale && plan.mixed.grid > 0);
  const bool run_dec = plan.decode.grid > 0;
  // both kinds of items: one launch when asked to, or (default) when the two
  // grids would otherwise run one after the other (no side stream: prepared
  // runs, graphs, the allocation-free form); side by side otherwise
  const int64_t mixed_mode = g_opt.mixed_grid.load();
  const bool run_mixed = run_pre && run_dec && plan.mixed.grid > 0 && (mixed_mode == 1 || (mixed_mode < 0 && !side));
  const bool fuse_append = new_direct && (run_pre || run_dec);
  if (do_append && !fuse_append) {
    if (timed) {
      if ((st = enqueue_append(ap, stream))) return st;
    } else {
      const int rc = vpk::launch_append(ap, stream);
      if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "append launch");
    }
  }
  // a8: LSE merge of split parts, after the grid that wrote them (the kernel
  // boundary makes the partials visible across the device without per-part
  // fences)
  auto merge = [&](hipStream_t s) -> int32_t {
    MergeParams mp{};
    mp.groups = reinterpret_cast<const MergeGroup*>(R + L.groups);
    mp.part_o = reinterpret_cast<const float*>(PA + L.part_o);
    mp.part_lse = reinterpret_cast<const float*>(PA + L.part_lse);
    mp.out = static_cast<uint16_t*>(out);
    mp.lse = lse;
    mp.num_groups = static_cast<int32_t>(plan.groups.size());
    mp.hq = dims->num_q_heads;
    mp.g = dims->num_q_heads / dims->num_kv_heads;
    mp.total_q = dims->total_q;
    mp.head_dim = dims->head_dim;
    int rc;
    if (timed) {
      KernelTimer tm(3, s);
      rc = vpk::launch_merge(mp, s);
    } else {
      rc = vpk::launch_merge(mp, s);
    }
    if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "merge launch");
    return VPK_SUCCESS;
  };
  bool merged = plan.groups.empty();
  if (run_pre || run_dec) {
    AttnParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = c.has_cache ? k_cache : k_new;
    p.v = c.has_cache ? v_cache : v_new;
    p.k_new = k_new;
    p.v_new = v_new;
    p.new_direct = new_direct ? 1 : 0;
    p.dec_append = dec_g > 0 ? 1 : 0;
    p.block_table = block_table;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.part_o = reinterpret_cast<float*>(PA + L.part_o);
    p.part_lse = reinterpret_cast<float*>(PA + L.part_lse);
    p.err_flag = reinterpret_cast<int32_t*>(bs.head);
    p.zeros = bs.head + kZerosOffset;
    p.max_pages = dims->max_pages_per_seq;
    p.num_pages = dims->num_pages;
    p.page_size = c.has_cache ? page_size : 1;
    p.page_shift = -1;
    if (c.has_cache && (page_size & (page_size - 1)) == 0) {
      int sh = 0;
      while ((1 << sh) < page_size) ++sh;
      p.page_shift = sh;
    }
    p.hq = dims->num_q_heads;
    p.hkv = dims->num_kv_heads;
    p.g = dims->num_q_heads / dims->num_kv_heads;
    p.total_q = dims->total_q;
    p.causal = causal;
    const double log2e = 1.4426950408889634;
    const bool host_scales = c.fp8 && kv_scale;
    p.scale_log2e = static_cast<double>(scale) * log2e;
    p.qk_scale_log2 = static_cast<float>(p.scale_log2e * (host_scales ? static_cast<double>(kv_scale[0]) : 1.0));
    p.v_scale = host_scales ? kv_scale[1] : 1.0f;
    p.kv_scale_dev = c.fp8 ? c.kv_scale_dev : nullptr;
    p.rope = rq;
    p.app = ap;
    const int fmt = c.fp8 ? vpk::kKvFp8 : vpk::kKvBf16;
    if (c.qp_scale) {
      // fp8 QKV-Prob: every unit in the one grid (the plan has no splits);
      // scores carry q_scale too, the output p_scale * v_scale
      const vpk::Launch& Lc = plan.mixed;
      if (Lc.grid <= 0) return VPK_SUCCESS;
      AttnParams a = p;
      a.num_pre_units = plan.num_pre_units;
      a.items = reinterpret_cast<const WorkItem*>(R + L.items) + Lc.first;
      a.queue_start = reinterpret_cast<const int32_t*>(R + L.queues) + Lc.queue_first;
      a.queue_work = reinterpret_cast<const int32_t*>(R + L.work) + Lc.work_first;
      a.persistent = Lc.persistent ? 1 : 0;
      a.num_items = Lc.count;
      a.attn_blocks = Lc.grid;
      a.qk_scale_log2 = static_cast<float>(p.scale_log2e * static_cast<double>(kv_scale[0]) *
                                           static_cast<double>(c.qp_scale[0]));
      a.v_scale = static_cast<float>(static_cast<double>(c.qp_scale[1]) * static_cast<double>(kv_scale[1]));
      a.kv_scale_dev = nullptr;
      a.q_inv_scale = 1.0f / c.qp_scale[0];
      a.scores = reinterpret_cast<float*>(PA + L.scores);
      a.p_log2 = static_cast<float>(std::log2(static_cast<double>(c.qp_scale[1])));
      a.rope = vpk::RopeArgs{};
      int rc;
      if (timed) {
        KernelTimer tm(6, stream);
        rc = vpk::launch_attention_prob8(a, Lc.grid, dims->head_dim, stream);
      } else {
        rc = vpk::launch_attention_prob8(a, Lc.grid, dims->head_dim, stream);
      }
      if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "attention launch (QKV-Prob)");
      return VPK_SUCCESS;
    }
    // `with_append`: this grid also runs one workgroup per new token
    auto launch = [&](const vpk::Launch& Lc, int mode, hipStream_t s, bool with_append) -> int32_t {
      const bool dec = mode == vpk::kGridDecode;
      AttnParams a = p;
      a.num_pre_units = mode == vpk::kGridPrefill ? Lc.count : mode == vpk::kGridMixed ? plan.num_pre_units : 0;
      a.items = reinterpret_cast<const WorkItem*>(R + L.items) + Lc.first;
      a.queue_start = reinterpret_cast<const int32_t*>(R + L.queues) + Lc.queue_first;
      a.queue_work = reinterpret_cast<const int32_t*>(R + L.work) + Lc.work_first;
      a.persistent = Lc.persistent ? 1 : 0;
      a.num_items = Lc.count;
      a.attn_blocks = Lc.grid;
      // new tokens in groups: 32 per 512-thread prefill workgroup, 16 per
      // 256-thread decode workgroup
      a.app.tokens_per_wg = dec ? 16 : 32;
      if (dec && q_dec) {
        // the decode-mode rows come already turned (a copy)
        a.q = static_cast<const uint16_t*>(q_dec);
        a.rope = vpk::RopeArgs{};
      }
      const int grid = Lc.grid + (with_append ? (dims->total_knew + a.app.tokens_per_wg - 1) / a.app.tokens_per_wg : 0);
      int rc;
      if (timed) {
        KernelTimer tm(mode == vpk::kGridMixed ? 5 : dec ? 2 : 0, s);
        rc = vpk::launch_attention(a, grid, dims->head_dim, fmt, c.has_cache, mode, s);
      } else {
        rc = vpk::launch_attention(a, grid, dims->head_dim, fmt, c.has_cache, mode, s);
      }
      if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "attention launch");
      return VPK_SUCCESS;
    };
    if (run_mixed) {
      // a9: prefill-mode tiles and decode-mode splits in one launch
      if ((st = launch(plan.mixed, vpk::kGridMixed, stream, fuse_append))) return st;
    } else if (run_pre && run_dec && side) {
      // both grids at once: the decode-mode grid (HBM-bound) on the side
      // stream next to the prefill-mode grid (MFMA-bound), joined at the end
      if ((st = ensure_aux(side))) return st;
      hipError_t e;
      if ((e = hipEventRecord(side->ev_fork, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord (fork)");
      if ((e = hipStreamWaitEvent(side->aux, side->ev_fork, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (fork)");
      if ((st = launch(plan.decode, vpk::kGridDecode, side->aux, fuse_append))) return st;
      // split parts of decode-mode tiles only: merged on the side stream
      // too, while the prefill-mode grid still runs
      if (!merged && std::all_of(plan.groups.begin(), plan.groups.end(), [](const MergeGroup& g) { return g.dec; })) {
        if ((st = merge(side->aux))) return st;
        merged = true;
      }
      if ((e = hipEventRecord(side->ev_join, side->aux)) != hipSuccess) return hip_fail(e, "hipEventRecord (join)");
      if ((st = launch(plan.prefill, vpk::kGridPrefill, stream, false))) return st;
      if ((e = hipStreamWaitEvent(stream, side->ev_join, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (join)");
    } else {
      // the new tokens ride with the first grid launched
      if (run_dec && (st = launch(plan.decode, vpk::kGridDecode, stream, fuse_append))) return st;
      if (run_pre && (st = launch(plan.prefill, vpk::kGridPrefill, stream, fuse_append && !run_dec))) return st;
    }
  }
  if (!merged && (st = merge(stream))) return st;
  return VPK_SUCCESS;
}

// Plan a validated call and enqueue it on `stream` (direct calls).
int32_t check_rope_args(const Call& c, const vpk_rope* rope) {
  int32_t st;
  const int32_t D = c.d->head_dim;
  if ((st = check_ptr(rope->cos, 16, "rope->cos")) || (st = check_ptr(rope->sin, 16, "rope->sin"))) return st;
  if (rope->rotary_dim < 16 || rope->rotary_dim > D || rope->rotary_dim % 16 != 0)
    return fail(VPK_ERROR_INVALID_VALUE, "rope->rotary_dim must be a multiple of 16 in [16, head_dim]");
  if (rope->interleaved != 0 && rope->interleaved != 1) return fail(VPK_ERROR_INVALID_VALUE, "rope->interleaved must be 0 or 1");
  if (rope->max_positions < 1) return fail(VPK_ERROR_INVALID_VALUE, "rope->max_positions must be >= 1");
  return VPK_SUCCESS;
}

// Every turned row needs a position in [0, max_positions): Lq <= Lk and Lk <= max_positions.
int32_t check_rope_positions(const PlanInput& in, const vpk_rope* rope) {
  for (int32_t b = 0; b < in.batch; ++b) {
    const int64_t q_len = in.q_start ? in.q_len[b] : in.cu_q[b + 1] - in.cu_q[b];
    const int64_t new_len = in.has_new ? in.cu_kn[b + 1] - in.cu_kn[b] : 0;
    const int64_t kv_len = ((in.has_cache && in.cache_lens) ? in.cache_lens[b] : 0) + new_len;
    if (q_len > kv_len)
      return fail(VPK_ERROR_INVALID_VALUE, "sequence " + std::to_string(b) + ": with rotary embedding a sequence needs "
                                           "no more query rows than keys (query row i sits at Lk - Lq + i)");
    if ((q_len > 0 || new_len > 0) && kv_len > rope->max_positions)
      return fail(VPK_ERROR_INVALID_VALUE, "sequence " + std::to_string(b) + " reaches position " +
                                               std::to_string(kv_len - 1) + ", past rope->max_positions");
  }
  return VPK_SUCCESS;
}

int32_t plan_and_enqueue(const Call& c, const Mirrors& m, int32_t causal, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, const int32_t* block_table, float scale,
                         void* out, float* lse, hipStream_t stream, const vpk_rope* rope = nullptr) {
  const vpk_dims* dims = c.d;
  const int32_t B = dims->batch;
  int32_t st;
  PlanInput in;
  fill_plan_input(c, m, causal, 0, in);
  if (c.qp_scale) {
    // QKV-Prob: one grid, whole key ranges (P needs each row's full sum)
    in.force_splits = 1;
    in.one_grid = true;
  }
  if (rope && (st = check_rope_positions(in, rope))) return st;
  if ((st = refuse_capture(stream))) return st;
  Workspace* w = nullptr;
  if ((st = find_workspace(stream, &w))) return st;
  // plan records: read by the kernels from the pinned plan buffer, or
  // uploaded into the workspace first (option "plan_upload")
  const bool upload = g_opt.plan_upload.load() != 0;
  const int32_t num_cus = device_cus();
  in.num_cus = num_cus;
  if (w->user)
    in.max_part_rows = std::min<int64_t>(in.max_part_rows,
                                         part_rows_fitting(w->user_bytes, dims, num_cus, rope != nullptr, upload));
  Plan plan;
  try {
    vpk::build_plan(in, plan);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host memory for the plan");
  }
  if (c.qp_scale && !plan.groups.empty())
    return fail(VPK_ERROR_NOT_SUPPORTED, "QKV-Prob attention: a sequence's keys span more than " +
                                             std::to_string(vpk::kMaxItemPages - 1) + " pages");
  // QKV-Prob: decode-mode units of at most kKeepScoreRows rows keep their
  // first-pass scores in the work memory (8 * rows bytes per key over both
  // passes, against re-reading 128-byte K rows); `part` / `part_stride` give
  // each (unit, kv head) its place in 128-byte units (one row of a 32-key block)
  size_t score_bytes = 0;
  if (c.qp_scale && dims->head_dim == 128 && g_opt.keep_scores.load() != 0) {
    int64_t units = 0;
    for (size_t i = static_cast<size_t>(plan.num_pre_units); i < plan.items.size(); ++i) {
      WorkItem& it = plan.items[i];
      if (it.nrows > kKeepScoreRows) continue;
      const int64_t nb = it.key_end > it.key_begin ? (it.key_end - it.key_begin + 31) / 32 : 0;
      const int64_t per_head = nb * it.nrows;
      if (units + per_head * dims->num_kv_heads > INT32_MAX) break;
      it.part = static_cast<int32_t>(units);
      it.part_stride = static_cast<int32_t>(per_head);
      units += per_head * dims->num_kv_heads;
    }
    score_bytes = static_cast<size_t>(units) * 128;
  }
  // Rotary embedding: the attention kernels turn the query rows as they load
  // them (interleaved pairs, or half-split pairs whose two chunks one lane
  // holds: rotary_dim a multiple of 32); with an fp8 cache the append, which
  // runs first anyway, turns the new keys as it quantises them; otherwise the
  // new keys are turned into a copy first (attention and the in-grid append
  // of a bf16 cache read it), and so are the query rows of other rotary dims.
  // Decode-mode rows are few and their items short, so turning them in the
  // kernel would put the angle loads on each item's critical path: they are
  // turned into the copy instead (measured on the paged decode batch: 146
  // against 136 us per step).
  RopeCopies rc;
  vpk::RopeArgs rq{}, rk{};
  bool q_dec_copy = false;
  if (rope) {
    rc.positions = true;
    const vpk::RopeArgs ra{rope->cos, rope->sin, rope->rotary_dim, rope->interleaved};
    // (the QKV-Prob grid reads turned copies of every query row)
    const bool fused_q = !c.qp_scale && (rope->interleaved != 0 || rope->rotary_dim % 32 == 0);
    q_dec_copy = fused_q && plan.decode.grid > 0 && !(plan.mixed.grid > 0 && g_opt.mixed_grid.load() == 1);
    rc.q = (!fused_q || q_dec_copy) && dims->total_q > 0;
    if (fused_q) rq = ra;
    if (c.has_cache && c.fp8) {
      if (c.has_new) rk = ra;
    } else {
      rc.k = k_new != nullptr && dims->total_knew > 0;
    }
  }
  Layout L = layout_for(plan, B, dims->total_knew, dims->head_dim, rope ? dims : nullptr, rc, score_bytes);
  if (score_bytes && w->user && kFlagBytes + L.part_end + (upload ? L.plan_end : 0) > w->user_bytes) {
    // the caller's workspace does not hold the scores: read K again instead
    for (size_t i = static_cast<size_t>(plan.num_pre_units); i < plan.items.size(); ++i) plan.items[i].part = -1;
    score_bytes = 0;
    L = layout_for(plan, B, dims->total_knew, dims->head_dim, rope ? dims : nullptr, rc, 0);
  }
  log_plan(c.qp_scale ? "qkv_prob" : "attention", plan, dims, L.plan_end, L.part_end);
  if ((st = get_workspace(stream, L.part_end + (upload ? L.plan_end : 0), &w))) return st;
  int region = 0;
  if ((st = write_plan(w, plan, L, m.cu_kn, B, c.page_size, stream, &region))) return st;
  char* R = w->plan[region].host;
  if (rope)
    write_rope_positions(plan, L, B, dims->total_q, R,
                         q_dec_copy && plan.prefill.grid > 0 ? dims->num_q_heads / dims->num_kv_heads : 0);
  if (upload) {
    char* const dR = w->parts() + L.part_end;
    const hipError_t e = hipMemcpyAsync(dR, R, L.plan_end, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan upload)");
    R = dR;
  } else if ((st = reuse_plan(w, L.plan_end, L.part_end, stream, &R))) {
    return st;
  }
  const Bases bases{R, w->parts(), w->head()};
  if (rc.q || rc.k) {
    // turned copies of q (rows the kernels do not turn) and of k_new (no
    // cache); everything after reads the copies
    vpk::RopeParams rp{};
    rp.q = static_cast<const uint16_t*>(q);
    rp.q_out = reinterpret_cast<uint16_t*>(bases.PA + L.rot_q);
    rp.qpos = reinterpret_cast<const int32_t*>(bases.R + L.qpos);
    rp.k = static_cast<const uint16_t*>(k_new);
    rp.k_out = reinterpret_cast<uint16_t*>(bases.PA + L.rot_k);
    rp.kpos = reinterpret_cast<const int32_t*>(bases.R + L.kpos);
    rp.cos = rope->cos;
    rp.sin = rope->sin;
    rp.q_rows = rc.q ? dims->total_q : 0;
    rp.k_rows = rc.k ? dims->total_knew : 0;
    if (q_dec_copy && plan.prefill.grid > 0) {
      // only the decode-mode rows are copied: the span of rows they occupy
      const int32_t g = dims->num_q_heads / dims->num_kv_heads;
      int32_t lo = dims->total_q, hi = 0;
      for (const SeqInfo& sq : plan.seqs)
        if (sq.q_len > 0 && static_cast<int64_t>(sq.q_len) * g <= vpk::kWaveRows) {
          lo = std::min(lo, sq.q_start);
          hi = std::max(hi, sq.q_start + sq.q_len);
        }
      const size_t off = static_cast<size_t>(std::min(lo, hi)) * dims->num_q_heads * dims->head_dim;
      rp.q += off;
      rp.q_out += off;
      rp.qpos += std::min(lo, hi);
      rp.q_rows = std::max(0, hi - lo);
    }
    rp.hq = dims->num_q_heads;
    rp.hkv = dims->num_kv_heads;
    rp.rot_dim = rope->rotary_dim;
    rp.interleaved = rope->interleaved;
    {
      KernelTimer tm(4, stream);
      const int rc = vpk::launch_rope(rp, dims->head_dim, stream);
      if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "rotary embedding launch");
    }
    if (rc.q && !q_dec_copy) q = rp.q_out;
    if (rc.k) k_new = rp.k_out;
  }
  const void* q_dec = q_dec_copy ? static_cast<const void*>(bases.PA + L.rot_q) : nullptr;
  if ((st = enqueue_all(c, plan, L, bases, q, k_new, v_new, k_cache, v_cache, block_table, causal, scale,
                        out, lse, stream, w, true, rq, rk, q_dec)))
    return st;
  return release_plan_buffer(w, stream, region);
}

// The allocation-free form of a direct call: the plan records go, behind a
// cleared head, into this device's static scratch array with one copy on
// `stream`, and the split partials after them; the planner limits its splits
// to what the array holds.  No device or pinned memory is allocated, no event
// or stream is created; host planning reuses this thread's buffers.  The
// source of the copy is pageable host memory, which the runtime has staged by
// the time the copy call returns.
int32_t plan_and_enqueue_noalloc(const Call& c, const Mirrors& m, int32_t causal, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache, const int32_t* block_table,
                                 float scale, void* out, float* lse, hipStream_t stream) {
  const vpk_dims* dims = c.d;
  const int32_t B = dims->batch;
  int32_t st;
  if ((st = refuse_capture(stream))) return st;
  void* sp = nullptr;
  const int rc = vpk::scratch_address(&sp);
  if (rc != 0) return hip_fail(static_cast<hipError_t>(rc), "hipGetSymbolAddress (scratch)");
  char* const base = static_cast<char*>(sp);
  const int32_t num_cus = device_cus();
  PlanInput in;
  fill_plan_input(c, m, causal, num_cus, in);
  in.max_part_rows = std::min<int64_t>(in.max_part_rows,
                                       part_rows_fitting(vpk::kScratchBytes, dims, num_cus, false, true));
  static thread_local Plan plan;
  try {
    vpk::build_plan(in, plan);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host memory for the plan");
  }
  const Layout L = layout_for(plan, B, dims->total_knew, dims->head_dim);
  log_plan("attention_noalloc", plan, dims, L.plan_end, L.part_end);
  const size_t need = kFlagBytes + L.plan_end + L.part_end;
  if (need > vpk::kScratchBytes)
    return fail(VPK_ERROR_CAPACITY, "the call needs " + std::to_string(need) + " bytes of scratch, the "
                                        "allocation-free entry point has " + std::to_string(vpk::kScratchBytes));
  // [head: error flag and zero rows][plan records][split partials]
  static thread_local std::vector<char> stage;
  stage.assign(kFlagBytes + L.plan_end, 0);
  serialize_plan(plan, L, m.cu_kn, B, c.page_size, stage.data() + kFlagBytes);
  const hipError_t e = hipMemcpyAsync(base, stage.data(), stage.size(), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan into scratch)");
  const Bases bases{base + kFlagBytes, base + kFlagBytes + L.plan_end, base};
  return enqueue_all(c, plan, L, bases, q, k_new, v_new, k_cache, v_cache, block_table, causal, scale, out, lse,
                     stream, nullptr, false);
}

int32_t attn_impl(const vpk_dims* dims, const void* q, const int32_t* cu_seqlens_q,
                  const void* k_new, const void* v_new, const int32_t* cu_seqlens_knew,
                  void* k_cache, void* v_cache, const int32_t* block_table,
                  const int32_t* cache_seqlens, int32_t page_size, int32_t causal, float scale,
                  const float* kv_scale, void* out, float* lse, const vpk_host_index* host,
                  void* stream_v, const vpk_rope* rope = nullptr, bool noalloc = false,
                  const float* qp_scale = nullptr, bool prob8 = false) {
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  if (!dims) return fail(VPK_ERROR_INVALID_VALUE, "dims is NULL");
  // new tokens are present when any of their arrays is given; with total_knew == 0
  // the token arrays may be NULL (a zero-size tensor has no storage)
  Call c{dims, k_new != nullptr || v_new != nullptr || cu_seqlens_knew != nullptr,
         k_cache != nullptr || v_cache != nullptr,
         dims->kv_cache_dtype == VPK_DTYPE_FP8_E4M3FN && (k_cache || v_cache), page_size, kv_scale};
  c.qp_scale = prob8 ? qp_scale : nullptr;
  int32_t st = check_dims(c);
  if (st != VPK_SUCCESS) return st;
  if (prob8) {
    if (!c.fp8 || !c.has_cache)
      return fail(VPK_ERROR_INVALID_VALUE, "QKV-Prob attention needs an fp8 (e4m3fn) cache");
    if (!qp_scale) return fail(VPK_ERROR_INVALID_VALUE, "qp_scale is NULL");
    if (!std::isfinite(qp_scale[0]) || !(qp_scale[0] > 0.f))
      return fail(VPK_ERROR_INVALID_VALUE, "q_scale must be finite and > 0");
    if (!std::isfinite(qp_scale[1]) || !(static_cast<double>(qp_scale[1]) >= 1.0 / 452.0))
      return fail(VPK_ERROR_INVALID_VALUE, "p_scale must be finite and >= 1/452");
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(VPK_ERROR_INVALID_VALUE, "k_new and v_new must both be given or both be NULL");
  if ((k_cache == nullptr) != (v_cache == nullptr)) return fail(VPK_ERROR_INVALID_VALUE, "k_cache and v_cache must both be given or both be NULL");
  if (!c.has_new && !c.has_cache) return fail(VPK_ERROR_INVALID_VALUE, "no keys: give k_new/v_new, a cache, or both");
  if (causal != 0 && causal != 1) return fail(VPK_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(VPK_ERROR_INVALID_VALUE, "scale must be finite and > 0");
  if (!c.has_new && dims->total_knew != 0) return fail(VPK_ERROR_INVALID_VALUE, "total_knew must be 0 without k_new");
  if (!c.has_cache && (dims->num_pages != 0)) return fail(VPK_ERROR_INVALID_VALUE, "num_pages must be 0 without a cache");
  if (!c.fp8 && kv_scale && c.has_cache) return fail(VPK_ERROR_INVALID_VALUE, "kv_scale must be NULL for a bf16 cache");
  const int32_t B = dims->batch;
  if (!cu_seqlens_q && !(host && host->cu_seqlens_q)) return fail(VPK_ERROR_INVALID_VALUE, "cu_seqlens_q is NULL");
  if (c.has_new) {
    if (!cu_seqlens_knew && !(host && host->cu_seqlens_knew))
      return fail(VPK_ERROR_INVALID_VALUE, "cu_seqlens_knew is NULL while k_new is given");
    if (dims->total_knew > 0 || k_new || v_new) {
      if ((st = check_ptr(k_new, 16, "k_new")) || (st = check_ptr(v_new, 16, "v_new"))) return st;
    }
  }
  if (c.has_cache) {
    if ((st = check_ptr(k_cache, 16, "k_cache")) || (st = check_ptr(v_cache, 16, "v_cache"))) return st;
    if ((st = check_ptr(block_table, 4, "block_table"))) return st;
    if ((st = check_ptr(cache_seqlens, 4, "cache_seqlens"))) return st;
  }
  if (dims->total_q > 0) {
    if ((st = check_ptr(q, 16, "q")) || (st = check_ptr(out, 16, "out"))) return st;
    if (lse && !aligned(lse, 4)) return fail(VPK_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
  }
  if (rope && (st = check_rope_args(c, rope))) return st;
  if (noalloc && !(host && host->cu_seqlens_q && (!c.has_new || host->cu_seqlens_knew) &&
                   (!c.has_cache || (host->cache_seqlens && host->block_table))))
    return fail(VPK_ERROR_INVALID_VALUE, "the allocation-free call needs host copies of every index array "
                                         "(cu_seqlens_q, and cu_seqlens_knew / cache_seqlens and block_table "
                                         "when there are new tokens / a cache)");
  if (B == 0) return VPK_SUCCESS;

  Mirrors m;
  if ((st = get_mirrors(c, cu_seqlens_q, cu_seqlens_knew, cache_seqlens, host, stream, true, m))) return st;
  if ((st = check_contents(c, m, true))) return st;
  if (noalloc)
    return plan_and_enqueue_noalloc(c, m, causal, q, k_new, v_new, k_cache, v_cache, block_table, scale, out, lse,
                                    stream);
  return plan_and_enqueue(c, m, causal, q, k_new, v_new, k_cache, v_cache, block_table, scale, out, lse, stream,
                          rope);
}

// The page-list form: each sequence's query rows [q_start, q_start + q_len)
// and page ids kv_indices[kv_indptr[b], kv_indptr[b + 1]); every index array
// is read from the host copies, kv_indices also on the device.
int32_t attn_list_impl(const vpk_dims* dims, const void* q, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const int32_t* kv_indices, int32_t page_size,
                       int32_t causal, float scale, const float* kv_scale, void* out, float* lse,
                       const vpk_host_pages* host, void* stream_v) {
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  if (!dims) return fail(VPK_ERROR_INVALID_VALUE, "dims is NULL");
  if (!host) return fail(VPK_ERROR_INVALID_VALUE, "host is NULL: the page-list form needs the host index arrays");
  const bool has_new = k_new != nullptr || v_new != nullptr || host->cu_seqlens_knew != nullptr;
  const bool has_cache = k_cache != nullptr || v_cache != nullptr;
  if (has_cache && (!host->cache_seqlens || !host->kv_indptr))
    return fail(VPK_ERROR_INVALID_VALUE, "cache_seqlens and kv_indptr are required with a cache");
  // the dense row length is not used here; the longest page list stands in for
  // it in the slot-index range check
  vpk_dims d = *dims;
  d.max_pages_per_seq = 0;
  if (has_cache) {
    if (dims->batch < 0) return fail(VPK_ERROR_INVALID_VALUE, "negative batch or length");
    for (int32_t b = 0; b < dims->batch; ++b) {
      const int64_t n = static_cast<int64_t>(host->kv_indptr[b + 1]) - host->kv_indptr[b];
      if (n < 0) return fail(VPK_ERROR_INVALID_VALUE, "kv_indptr must be non-decreasing");
      d.max_pages_per_seq = static_cast<int32_t>(std::max<int64_t>(d.max_pages_per_seq, n));
    }
    d.max_pages_per_seq = std::max(d.max_pages_per_seq, 1);
  }
  dims = &d;
  Call c{dims, has_new, has_cache, dims->kv_cache_dtype == VPK_DTYPE_FP8_E4M3FN && has_cache, page_size, kv_scale};
  int32_t st = check_dims(c);
  if (st != VPK_SUCCESS) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(VPK_ERROR_INVALID_VALUE, "k_new and v_new must both be given or both be NULL");
  if ((k_cache == nullptr) != (v_cache == nullptr)) return fail(VPK_ERROR_INVALID_VALUE, "k_cache and v_cache must both be given or both be NULL");
  if (!has_new && !has_cache) return fail(VPK_ERROR_INVALID_VALUE, "no keys: give k_new/v_new, a cache, or both");
  if (causal != 0 && causal != 1) return fail(VPK_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  if (!has_new && dims->total_knew != 0) return fail(VPK_ERROR_INVALID_VALUE, "total_knew must be 0 without k_new");
  if (!has_cache && dims->num_pages != 0) return fail(VPK_ERROR_INVALID_VALUE, "num_pages must be 0 without a cache");
  if ((st = check_run_pointers(c, q, k_new, v_new, k_cache, v_cache, kv_indices, scale, out, lse))) return st;
  const int32_t B = dims->batch;
  if (!host->q_start || !host->q_len) return fail(VPK_ERROR_INVALID_VALUE, "q_start and q_len are required");
  if (has_new && !host->cu_seqlens_knew) return fail(VPK_ERROR_INVALID_VALUE, "cu_seqlens_knew is NULL while k_new is given");
  if (B == 0) return VPK_SUCCESS;
  // query rows: inside [0, total_q), no two sequences sharing a row
  std::vector<std::pair<int32_t, int32_t>> spans;
  spans.reserve(B);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t a = host->q_start[b], n = host->q_len[b];
    if (a < 0 || n < 0 || a + n > dims->total_q)
      return fail(VPK_ERROR_INVALID_VALUE, "sequence " + std::to_string(b) + ": query rows outside [0, total_q)");
    if (n > 0) spans.emplace_back(static_cast<int32_t>(a), static_cast<int32_t>(a + n));
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return fail(VPK_ERROR_INVALID_VALUE, "two sequences share query rows");
  Mirrors m;
  m.q_start = host->q_start;
  m.q_len = host->q_len;
  m.cu_kn = has_new ? host->cu_seqlens_knew : nullptr;
  if (has_new && (st = check_cu(m.cu_kn, B, dims->total_knew, "cu_seqlens_knew")) != VPK_SUCCESS) return st;
  std::vector<int32_t> zero_rows;
  if (has_cache) {
    const int32_t* ip = host->kv_indptr;
    if (ip[0] < 0) return fail(VPK_ERROR_INVALID_VALUE, "kv_indptr[0] must be >= 0");
    for (int32_t b = 0; b < B; ++b) {
      const int64_t lc = host->cache_seqlens[b];
      if (lc < 0) return fail(VPK_ERROR_INVALID_VALUE, "cache_seqlens must be >= 0");
      const int64_t lk = lc + (has_new ? m.cu_kn[b + 1] - m.cu_kn[b] : 0);
      const int64_t cap = static_cast<int64_t>(ip[b + 1] - ip[b]) * page_size;
      if (lk > cap)
        return fail(VPK_ERROR_CAPACITY, "sequence " + std::to_string(b) + " needs " + std::to_string(lk) +
                                            " slots, its page list holds " + std::to_string(cap));
      if (host->kv_indices) {
        const int64_t np = (lk + page_size - 1) / page_size;
        for (int64_t i = 0; i < np; ++i) {
          const int32_t pg = host->kv_indices[ip[b] + i];
          if (pg < 0 || pg >= dims->num_pages)
            return fail(VPK_ERROR_INVALID_VALUE, "kv_indices[" + std::to_string(ip[b] + i) + "] = " +
                                                     std::to_string(pg) + " is outside [0, num_pages)");
        }
      }
    }
    m.cache_lens = host->cache_seqlens;
    m.bt_row = ip;
  } else {
    zero_rows.assign(B + 1, 0);
    m.bt_row = zero_rows.data();
  }
  return plan_and_enqueue(c, m, causal, q, k_new, v_new, k_cache, v_cache, kv_indices, scale, out, lse, stream);
}

int32_t append_impl(const vpk_dims* dims, const void* k_new, const void* v_new,
                    const int32_t* cu_seqlens_knew, void* k_cache, void* v_cache,
                    const int32_t* block_table, const int32_t* cache_seqlens, int32_t page_size,
                    const float* kv_scale, const vpk_host_index* host, void* stream_v) {
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  if (!dims) return fail(VPK_ERROR_INVALID_VALUE, "dims is NULL");
  Call c{dims, true, true, dims->kv_cache_dtype == VPK_DTYPE_FP8_E4M3FN, page_size, kv_scale};
  int32_t st = check_dims(c);
  if (st != VPK_SUCCESS) return st;
  if (!c.fp8 && kv_scale) return fail(VPK_ERROR_INVALID_VALUE, "kv_scale must be NULL for a bf16 cache");
  if (dims->total_knew == 0 && dims->batch >= 0) return VPK_SUCCESS;
  if ((st = check_ptr(k_new, 16, "k_new")) || (st = check_ptr(v_new, 16, "v_new"))) return st;
  if ((st = check_ptr(k_cache, 16, "k_cache")) || (st = check_ptr(v_cache, 16, "v_cache"))) return st;
  if ((st = check_ptr(block_table, 4, "block_table")) || (st = check_ptr(cache_seqlens, 4, "cache_seqlens"))) return st;
  if (!cu_seqlens_knew && !(host && host->cu_seqlens_knew)) return fail(VPK_ERROR_INVALID_VALUE, "cu_seqlens_knew is NULL");
  const int32_t B = dims->batch;
  if (B == 0 || dims->total_knew == 0) return VPK_SUCCESS;
  Mirrors m;
  if ((st = get_mirrors(c, nullptr, cu_seqlens_knew, cache_seqlens, host, stream, false, m))) return st;
  if ((st = check_contents(c, m, false))) return st;
  if ((st = refuse_capture(stream))) return st;
  Plan plan;
  plan.seqs.resize(B);
  for (int32_t b = 0; b < B; ++b) {
    SeqInfo s{};
    s.new_len = m.cu_kn[b + 1] - m.cu_kn[b];
    s.kn_start = m.cu_kn[b];
    s.cache_len = m.cache_lens[b];
    s.kv_len = s.cache_len + s.new_len;
    s.bt_row = static_cast<int32_t>(static_cast<int64_t>(b) * dims->max_pages_per_seq);
    plan.seqs[b] = s;
  }
  const Layout L = layout_for(plan, B, dims->total_knew, dims->head_dim);
  Workspace* w = nullptr;
  if ((st = get_workspace(stream, 0, &w))) return st;
  int region = 0;
  if ((st = write_plan(w, plan, L, m.cu_kn, B, c.page_size, stream, &region))) return st;
  if ((st = enqueue_append(append_params(c, w->head(), w->plan[region].host, L, k_new, v_new, k_cache,
                                         v_cache, block_table),
                           stream)))
    return st;
  return release_plan_buffer(w, stream, region);
}

}  // namespace

// A prepared call: the plan of one set of lengths, in device memory with its
// own error flag, zero rows and split partials.
struct vpk_plan_s {
  vpk_dims dims;
  bool has_new = false, has_cache = false, fp8 = false;
  int32_t page_size = 1, causal = 0;
  int device = -1;
  Plan plan;
  Layout L{};
  char* dev = nullptr;   // [head kFlagBytes][plan records L.plan_end][partials L.part_end]
};

namespace {

int32_t plan_create_impl(const vpk_dims* dims, const vpk_host_index* host, int32_t has_new,
                         int32_t has_cache, int32_t page_size, int32_t causal, vpk_plan* out) {
  if (!out) return fail(VPK_ERROR_INVALID_VALUE, "plan output pointer is NULL");
  *out = nullptr;
  if (!dims) return fail(VPK_ERROR_INVALID_VALUE, "dims is NULL");
  if ((has_new != 0 && has_new != 1) || (has_cache != 0 && has_cache != 1))
    return fail(VPK_ERROR_INVALID_VALUE, "has_new and has_cache must be 0 or 1");
  if (!has_new && !has_cache) return fail(VPK_ERROR_INVALID_VALUE, "no keys: a plan needs new tokens, a cache, or both");
  if (causal != 0 && causal != 1) return fail(VPK_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  const bool fp8 = has_cache && dims->kv_cache_dtype == VPK_DTYPE_FP8_E4M3FN;
  static const float kAnyScale[2] = {1.f, 1.f};   // the scales come with each run
  Call c{dims, has_new != 0, has_cache != 0, fp8, page_size, fp8 ? kAnyScale : nullptr};
  int32_t st = check_dims(c);
  if (st != VPK_SUCCESS) return st;
  if (!has_new && dims->total_knew != 0) return fail(VPK_ERROR_INVALID_VALUE, "total_knew must be 0 without new tokens");
  if (!has_cache && dims->num_pages != 0) return fail(VPK_ERROR_INVALID_VALUE, "num_pages must be 0 without a cache");
  if (!host || !host->cu_seqlens_q || (has_new && !host->cu_seqlens_knew) || (has_cache && !host->cache_seqlens))
    return fail(VPK_ERROR_INVALID_VALUE, "a plan needs the host index arrays (cu_seqlens_q, and cu_seqlens_knew / "
                                         "cache_seqlens when there are new tokens / a cache)");
  Mirrors m;
  if ((st = get_mirrors(c, nullptr, nullptr, nullptr, host, nullptr, true, m))) return st;
  if ((st = check_contents(c, m, true))) return st;

  vpk_plan_s* pl = new (std::nothrow) vpk_plan_s();
  if (!pl) return fail(VPK_ERROR_OUT_OF_MEMORY, "plan bookkeeping");
  pl->dims = *dims;
  pl->has_new = has_new != 0;
  pl->has_cache = has_cache != 0;
  pl->fp8 = fp8;
  pl->page_size = has_cache ? page_size : 1;
  pl->causal = causal;
  const int32_t B = dims->batch;
  PlanInput in;
  fill_plan_input(c, m, causal, device_cus(), in);
  try {
    vpk::build_plan(in, pl->plan);
  } catch (const std::bad_alloc&) {
    delete pl;
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host memory for the plan");
  }
  pl->L = layout_for(pl->plan, B, dims->total_knew, dims->head_dim);
  log_plan("plan_create", pl->plan, dims, pl->L.plan_end, pl->L.part_end);
  hipError_t e = hipGetDevice(&pl->device);
  if (e != hipSuccess) {
    delete pl;
    return hip_fail(e, "hipGetDevice");
  }
  const size_t bytes = kFlagBytes + pl->L.plan_end + pl->L.part_end;
  void* d = nullptr;
  if ((e = hipMalloc(&d, bytes)) != hipSuccess) {
    delete pl;
    return fail(VPK_ERROR_OUT_OF_MEMORY, std::string("hipMalloc plan: ") + hipGetErrorString(e));
  }
  pl->dev = static_cast<char*>(d);
  std::vector<char> rec(pl->L.plan_end + kFlagBytes, 0);   // head (flag, zeros) then the records
  serialize_plan(pl->plan, pl->L, m.cu_kn, B, pl->page_size, rec.data() + kFlagBytes);
  if ((e = hipMemcpy(pl->dev, rec.data(), rec.size(), hipMemcpyHostToDevice)) != hipSuccess) {
    (void)hipFree(pl->dev);
    delete pl;
    return hip_fail(e, "hipMemcpy plan");
  }
  *out = pl;
  return VPK_SUCCESS;
}

int32_t plan_run_impl(vpk_plan pl, const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* block_table, float scale, const float* kv_scale,
                      void* out, float* lse, void* stream_v, const float* kv_scale_dev = nullptr) {
  if (!pl) return fail(VPK_ERROR_INVALID_VALUE, "plan is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != pl->device) return fail(VPK_ERROR_INVALID_VALUE, "the plan was created on another device");
  Call c{&pl->dims, pl->has_new, pl->has_cache, pl->fp8, pl->page_size, kv_scale, kv_scale_dev};
  int32_t st = check_run_pointers(c, q, k_new, v_new, k_cache, v_cache, block_table, scale, out, lse);
  if (st) return st;
  if (pl->dims.batch == 0) return VPK_SUCCESS;
  const Bases bases{pl->dev + kFlagBytes, pl->dev + kFlagBytes + pl->L.plan_end, pl->dev};
  return enqueue_all(c, pl->plan, pl->L, bases, q, k_new, v_new, k_cache, v_cache, block_table, pl->causal,
                     scale, out, lse, static_cast<hipStream_t>(stream_v), nullptr, false);
}

}  // namespace

extern "C" {

int32_t vpk_plan_create(const vpk_dims* dims, const vpk_host_index* host, int32_t has_new, int32_t has_cache,
                        int32_t page_size, int32_t causal, vpk_plan* plan) {
  try {
    g_err.clear();
    return plan_create_impl(dims, host, has_new, has_cache, page_size, causal, plan);
  } catch (...) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host exception while planning");
  }
}

int32_t vpk_plan_run_device_scale(vpk_plan plan, const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const int32_t* block_table, float scale,
                                  const float* kv_scale_dev, void* out, float* lse, void* stream) {
  try {
    g_err.clear();
    if (plan && plan->fp8 && !kv_scale_dev) return fail(VPK_ERROR_INVALID_VALUE, "kv_scale_dev is NULL for an fp8 plan");
    return plan_run_impl(plan, q, k_new, v_new, k_cache, v_cache, block_table, scale, nullptr, out, lse, stream,
                         kv_scale_dev);
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t vpk_plan_run(vpk_plan plan, const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, const int32_t* block_table, float scale, const float* kv_scale, void* out,
                     float* lse, void* stream) {
  try {
    g_err.clear();
    return plan_run_impl(plan, q, k_new, v_new, k_cache, v_cache, block_table, scale, kv_scale, out, lse,
                         stream);
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t vpk_plan_device_error(vpk_plan plan, void* stream, int32_t* flags) {
  g_err.clear();
  if (!plan) return fail(VPK_ERROR_INVALID_VALUE, "plan is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t v = 0;
  if ((e = hipMemcpy(&v, plan->dev, sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy (flag)");
  if (v != 0) {
    const int32_t zero = 0;
    if ((e = hipMemcpy(plan->dev, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy (flag reset)");
  }
  if (flags) *flags = v;
  return VPK_SUCCESS;
}

int32_t vpk_plan_destroy(vpk_plan plan) {
  g_err.clear();
  if (!plan) return VPK_SUCCESS;
  hipError_t e = hipSuccess;
  if (plan->dev) e = hipFree(plan->dev);
  delete plan;
  if (e != hipSuccess) return hip_fail(e, "hipFree plan");
  return VPK_SUCCESS;
}

int32_t attn_varlen_paged_fwd(const vpk_dims* dims, const void* q, const int32_t* cu_seqlens_q,
                              const void* k_new, const void* v_new, const int32_t* cu_seqlens_knew,
                              void* k_cache, void* v_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int32_t page_size, int32_t causal,
                              float scale, const float* kv_scale, void* out, float* lse,
                              const vpk_host_index* host, void* stream) {
  try {
    g_err.clear();
    return attn_impl(dims, q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache,
                     block_table, cache_seqlens, page_size, causal, scale, kv_scale, out, lse,
                     host, stream);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t attn_varlen_paged_fwd_noalloc(const vpk_dims* dims, const void* q, const int32_t* cu_seqlens_q,
                                      const void* k_new, const void* v_new, const int32_t* cu_seqlens_knew,
                                      void* k_cache, void* v_cache, const int32_t* block_table,
                                      const int32_t* cache_seqlens, int32_t page_size, int32_t causal,
                                      float scale, const float* kv_scale, void* out, float* lse,
                                      const vpk_host_index* host, void* stream) {
  try {
    g_err.clear();
    return attn_impl(dims, q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache,
                     block_table, cache_seqlens, page_size, causal, scale, kv_scale, out, lse,
                     host, stream, nullptr, true);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t attn_varlen_paged_rope_fwd(const vpk_dims* dims, const void* q, const int32_t* cu_seqlens_q,
                                   const void* k_new, const void* v_new, const int32_t* cu_seqlens_knew,
                                   void* k_cache, void* v_cache, const int32_t* block_table,
                                   const int32_t* cache_seqlens, int32_t page_size, int32_t causal,
                                   float scale, const float* kv_scale, const vpk_rope* rope, void* out,
                                   float* lse, const vpk_host_index* host, void* stream) {
  try {
    g_err.clear();
    if (!rope) return fail(VPK_ERROR_INVALID_VALUE, "rope is NULL");
    return attn_impl(dims, q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache,
                     block_table, cache_seqlens, page_size, causal, scale, kv_scale, out, lse,
                     host, stream, rope);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t attn_varlen_paged_qkv_prob_fwd(const vpk_dims* dims, const void* q, const int32_t* cu_seqlens_q,
                                       const void* k_new, const void* v_new, const int32_t* cu_seqlens_knew,
                                       void* k_cache, void* v_cache, const int32_t* block_table,
                                       const int32_t* cache_seqlens, int32_t page_size, int32_t causal, float scale,
                                       const float* kv_scale, const float* qp_scale, const vpk_rope* rope, void* out,
                                       float* lse, const vpk_host_index* host, void* stream) {
  try {
    g_err.clear();
    return attn_impl(dims, q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                     cache_seqlens, page_size, causal, scale, kv_scale, out, lse, host, stream, rope, false, qp_scale,
                     true);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t attn_varlen_paged_list_fwd(const vpk_dims* dims, const void* q, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, const int32_t* kv_indices, int32_t page_size,
                                   int32_t causal, float scale, const float* kv_scale, void* out, float* lse,
                                   const vpk_host_pages* host, void* stream) {
  try {
    g_err.clear();
    return attn_list_impl(dims, q, k_new, v_new, k_cache, v_cache, kv_indices, page_size, causal, scale,
                          kv_scale, out, lse, host, stream);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t kv_cache_append(const vpk_dims* dims, const void* k_new, const void* v_new,
                        const int32_t* cu_seqlens_knew, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        int32_t page_size, const float* kv_scale, const vpk_host_index* host,
                        void* stream) {
  try {
    g_err.clear();
    return append_impl(dims, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                       cache_seqlens, page_size, kv_scale, host, stream);
  } catch (const std::bad_alloc&) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(VPK_ERROR_INVALID_VALUE, "unexpected host exception");
  }
}

int32_t vpk_set_workspace(void* stream_v, void* ptr, size_t bytes) {
  try {
    g_err.clear();
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    if (ptr && !aligned(ptr, 256)) return fail(VPK_ERROR_INVALID_VALUE, "the workspace must be 256-byte aligned");
    if (ptr && bytes < kFlagBytes + 4096)
      return fail(VPK_ERROR_INVALID_VALUE, "the workspace must hold at least " + std::to_string(kFlagBytes + 4096) +
                                               " bytes");
    int32_t st = refuse_capture(stream);
    if (st) return st;
    Workspace* w = nullptr;
    if ((st = find_workspace(stream, &w))) return st;
    if (ptr) {
      // a clear error flag and zero rows, in stream order before any call that uses them
      const hipError_t e = hipMemsetAsync(ptr, 0, kFlagBytes, stream);
      if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync (workspace head)");
    }
    std::lock_guard<std::mutex> lk(g_wmu);
    w->user = static_cast<char*>(ptr);
    w->user_bytes = ptr ? bytes : 0;
    w->rec_state = 0;   // no copy of a work list in the new buffer
    return VPK_SUCCESS;
  } catch (...) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host exception in vpk_set_workspace");
  }
}

int32_t vpk_library_memory(size_t* device_bytes, size_t* pinned_bytes) {
  size_t d = 0, h = 0;
  {
    std::lock_guard<std::mutex> lk(g_wmu);
    for (const auto& kv : g_ws) {
      const Workspace* w = kv.second;
      if (!w) continue;
      d += w->dev ? w->bytes : 0;
      for (const PlanBuf& pb : w->plan) h += pb.bytes;
    }
  }
  if (device_bytes) *device_bytes = d;
  if (pinned_bytes) *pinned_bytes = h;
  return VPK_SUCCESS;
}

size_t vpk_qkv_prob_score_bytes(const vpk_dims* dims, const vpk_host_index* host) {
  if (!dims || !host || !host->cu_seqlens_q || dims->batch < 0 || dims->num_kv_heads <= 0 ||
      dims->num_q_heads <= 0 || dims->num_q_heads % dims->num_kv_heads != 0 || dims->head_dim != 128)
    return 0;
  const int64_t g = dims->num_q_heads / dims->num_kv_heads;
  int64_t units = 0;
  for (int32_t b = 0; b < dims->batch; ++b) {
    const int64_t rows = (static_cast<int64_t>(host->cu_seqlens_q[b + 1]) - host->cu_seqlens_q[b]) * g;
    if (rows <= 0 || rows > kKeepScoreRows) continue;
    int64_t kv = host->cache_seqlens ? std::max<int32_t>(host->cache_seqlens[b], 0) : 0;
    if (host->cu_seqlens_knew) kv += std::max<int64_t>(0, static_cast<int64_t>(host->cu_seqlens_knew[b + 1]) -
                                                            host->cu_seqlens_knew[b]);
    units += (kv + 31) / 32 * rows;
  }
  if (units == 0) return 0;
  return static_cast<size_t>(units) * dims->num_kv_heads * 128 + 256;
}

size_t vpk_workspace_bytes_upper_bound(const vpk_dims* dims, int32_t num_cus, int32_t rope) {
  if (!dims || dims->batch < 0 || dims->total_q < 0 || dims->total_knew < 0 || dims->num_kv_heads <= 0 ||
      dims->num_q_heads <= 0 || dims->head_dim <= 0 || dims->num_q_heads % dims->num_kv_heads != 0)
    return 0;
  if (num_cus <= 0) num_cus = device_cus();
  return kFlagBytes + part_bytes_for(part_rows_bound(dims), dims->head_dim) +
         (rope ? rope_bytes_for(dims) : 0) + plan_bytes_bound(dims, num_cus, rope != 0);
}

const char* vpk_last_error(void) { return g_err.c_str(); }

int32_t vpk_abi_version(void) { return VPK_ABI_VERSION; }

int32_t vpk_set_option(const char* name, int64_t value) {
  if (!name) return fail(VPK_ERROR_INVALID_VALUE, "option name is NULL");
  const std::string n(name);
  if (n == "force_splits") {
    if (value < 0 || value > vpk::kMaxSplits) return fail(VPK_ERROR_INVALID_VALUE, "force_splits out of range");
    g_opt.force_splits = value;
  } else if (n == "persistent") {
    if (value < -1 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "persistent must be -1, 0 or 1");
    g_opt.persistent = value;
  } else if (n == "split_min_keys") {
    if (value < 1 || value > (1 << 24)) return fail(VPK_ERROR_INVALID_VALUE, "split_min_keys out of range");
    g_opt.split_min_keys = value;
  } else if (n == "plan_upload") {
    if (value < 0 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "plan_upload must be 0 or 1");
    g_opt.plan_upload = value;
  } else if (n == "mixed_dec_parts") {
    if (value < 1 || value > 64) return fail(VPK_ERROR_INVALID_VALUE, "mixed_dec_parts must be in [1, 64]");
    g_opt.mixed_dec_parts = value;
  } else if (n == "mixed_grid") {
    if (value < -1 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "mixed_grid must be -1, 0 or 1");
    g_opt.mixed_grid = value;
  } else if (n == "plan_reuse") {
    if (value < 0 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "plan_reuse must be 0 or 1");
    g_opt.plan_reuse = value;
  } else if (n == "keep_scores") {
    if (value < 0 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "keep_scores must be 0 or 1");
    g_opt.keep_scores = value;
  } else if (n == "plan_log") {
    if (value < -1 || value > 1) return fail(VPK_ERROR_INVALID_VALUE, "plan_log must be -1, 0 or 1");
    g_opt.plan_log = value;
  } else if (n == "num_cus") {
    if (value < 0 || value > 4096) return fail(VPK_ERROR_INVALID_VALUE, "num_cus out of range");
    g_opt.num_cus = value;
  } else {
    return fail(VPK_ERROR_INVALID_VALUE, "unknown option " + n);
  }
  return VPK_SUCCESS;
}

int32_t vpk_timing_enable(int32_t enable) {
  g_timing = enable != 0;
  return VPK_SUCCESS;
}

int32_t vpk_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (const TimingRec& r : g_tpending) {
    (void)hipEventSynchronize(r.b);
    g_tfree.push_back(r.a);
    g_tfree.push_back(r.b);
  }
  g_tpending.clear();
  for (int i = 0; i < kTimedKernels; ++i) {
    g_tms[i] = 0;
    g_tcount[i] = 0;
  }
  return VPK_SUCCESS;
}

int32_t vpk_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= kTimedKernels) return fail(VPK_ERROR_INVALID_VALUE, "kernel id must be 0..6");
  std::lock_guard<std::mutex> lk(g_tmu);
  for (const TimingRec& r : g_tpending) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (timing)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    g_tms[r.kernel] += ms;
    g_tcount[r.kernel] += 1;
    g_tfree.push_back(r.a);
    g_tfree.push_back(r.b);
  }
  g_tpending.clear();
  if (total_ms) *total_ms = g_tms[kernel];
  if (launches) *launches = g_tcount[kernel];
  return VPK_SUCCESS;
}

int32_t vpk_device_error(void* stream_v, int32_t* flags) {
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  if (!flags) return fail(VPK_ERROR_INVALID_VALUE, "flags is NULL");
  *flags = 0;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
  Workspace* w = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_wmu);
    auto it = g_ws.find(std::make_pair(dev, stream_v));
    if (it == g_ws.end() || !it->second->head()) return VPK_SUCCESS;
    w = it->second;
  }
  int32_t v = 0;
  if ((e = hipMemcpy(&v, w->head(), sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy flag");
  if ((e = hipMemset(w->head(), 0, sizeof(v))) != hipSuccess) return hip_fail(e, "hipMemset flag");
  *flags = v;
  return VPK_SUCCESS;
}

int32_t vpk_plan_debug(const vpk_dims* dims, const vpk_host_index* host, int32_t has_cache,
                       int32_t has_new, int32_t page_size, int32_t causal, int32_t num_cus,
                       int32_t* items, int32_t capacity, int32_t* n_items, int32_t* n_queues) {
  try {
    g_err.clear();
    if (!dims || !host || !host->cu_seqlens_q) return fail(VPK_ERROR_INVALID_VALUE, "dims and host->cu_seqlens_q are required");
    if (num_cus <= 0) return fail(VPK_ERROR_INVALID_VALUE, "num_cus must be > 0");
    Call c{dims, has_new != 0, has_cache != 0, has_cache && dims->kv_cache_dtype == VPK_DTYPE_FP8_E4M3FN,
           page_size, nullptr};
    const float one[2] = {1.f, 1.f};
    if (c.fp8) c.kv_scale = one;
    int32_t st = check_dims(c);
    if (st) return st;
    if (c.has_new && !host->cu_seqlens_knew) return fail(VPK_ERROR_INVALID_VALUE, "host->cu_seqlens_knew is required");
    if (c.has_cache && !host->cache_seqlens) return fail(VPK_ERROR_INVALID_VALUE, "host->cache_seqlens is required");
    Mirrors m;
    m.cu_q = host->cu_seqlens_q;
    m.cu_kn = host->cu_seqlens_knew;
    m.cache_lens = host->cache_seqlens;
    m.block_table = host->block_table;
    if ((st = check_contents(c, m, true))) return st;
    PlanInput in;
    fill_plan_input(c, m, causal, num_cus, in);
    Plan plan;
    vpk::build_plan(in, plan);
    // expand units to (unit, kv head) items in launch order
    const int32_t hkv = dims->num_kv_heads;
    const int32_t n = static_cast<int32_t>(plan.items.size()) * hkv;
    if (n_items) *n_items = n;
    if (n_queues)
      *n_queues = (plan.prefill.persistent ? plan.prefill.grid : 0) + (plan.decode.persistent ? plan.decode.grid : 0);
    if (n > capacity) return fail(VPK_ERROR_CAPACITY, "items buffer too small");
    int32_t k = 0;
    int32_t qoff = 0;
    for (const vpk::Launch* Lc : {&plan.prefill, &plan.decode}) {
      auto emit = [&](int32_t work, int32_t queue) {
        const int32_t u = work / hkv, h = work % hkv;
        const WorkItem& it = plan.items[Lc->first + u];
        int32_t* o = items + 8 * (k++);
        o[0] = it.seq; o[1] = it.row0; o[2] = it.nrows; o[3] = h;
        o[4] = it.key_begin; o[5] = it.key_end;
        o[6] = it.part < 0 ? -1 : it.part + h * it.part_stride;
        o[7] = queue;
      };
      if (!Lc->persistent) {
        for (int32_t wk = 0; wk < Lc->count * hkv; ++wk) emit(wk, -1);
      } else {
        for (int32_t q = 0; q < Lc->grid; ++q)
          for (int32_t e = plan.queue_start[Lc->queue_first + q]; e < plan.queue_start[Lc->queue_first + q + 1]; ++e)
            emit(plan.queue_work[Lc->work_first + e], qoff + q);
        qoff += Lc->grid;
      }
    }
    return VPK_SUCCESS;
  } catch (...) {
    return fail(VPK_ERROR_OUT_OF_MEMORY, "host exception in planner");
  }
}

}  // extern "C"
