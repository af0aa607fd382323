// Attention over a paged KV cache for packed variable-length queries, gfx950.
//
// One workgroup (4 wavefronts, 256 threads) processes one work item at a time:
// up to 128 packed query rows of one sequence under one kv head, against the
// keys [key_begin, key_end) of that sequence.  Rows are (token, query head)
// pairs packed token-major, so the g query heads that share a kv head
// (grouped-query attention, vLLM Triton FAv2 PR page, feature list) all use
// each K/V tile staged in LDS.
//
// Per 64-key block (a2..a6):
//   a2  K and V rows of the block are gathered through the item's page ids
//       (one page table for K and V: TransformerEngine KV-cache PR page,
//       Description).  bf16 rows go straight from HBM to LDS with
//       global_load_lds (16 bytes per lane, no registers); fp8 e4m3fn rows go
//       through registers and are widened to bf16 exactly on the way.  Both K
//       and V are stored row-major with the 16-byte chunks of each row
//       XOR-swizzled, and rows past the item's keys are loaded from a zero
//       region.  The next block is in flight while the current one computes.
//   a3  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//       column and 32 of the block's 64 keys, the other 32 sit in lane ^ 32.
//   a4  keys beyond the item's end, or (causal) beyond token + Lk - Lq, get
//       -inf; only blocks that cross that bound are masked.
//   a5  online softmax in base 2 on the raw scores: row max over registers
//       plus one permlane32 swap, p = 2^(s c - m c) with one fma, running
//       sum per lane, output rescaled only when some row's max moved.
//   a6  O^T += V^T P^T on the same MFMA; the V^T operand comes from
//       ds_read_b64_tr_b16 transposed LDS reads of the row-major V tile, P is
//       rounded to bf16 in registers.
//   a7  out = O / l (bf16) and lse = m c ln 2 + ln l, or for a split part the
//       fp32 normalised partial and its lse for the merge pass.
// Items of at most 32 rows (decode) instead split their keys over the four
// waves, each with its own 32-key half stage, and merge the four partial
// states through LDS at the end.
//
// The online softmax and the split of the key range into parts merged by LSE
// follow the FlashAttention-2 design the pages build on ("Add
// flash_attn_varlen_func_with_kvcache", Limitation and the discussion of
// split-KV for decoding); the tiling, the transposed S layout and the LDS
// layout are this library's own for CDNA4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../vpk_internal.h"
#include "append_dev.h"

namespace vpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazyLog2 = 8.f;   // log2 of the largest unnormalised p kept before rescaling

template <int D>
struct Cfg {
  static constexpr int CHUNKS = D / 8;          // 16-byte chunks of a bf16 row
  static constexpr int TILE = kBlockN * D;      // bf16 elements of a 64-key K (or V) tile
  static constexpr int STAGE = 2 * TILE;        // K tile then V tile
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dim
  static constexpr int DBLK = D / 32;           // 32-wide output blocks over the head dim
  // XOR swizzle of the chunk index by row.  The K operand reads take one
  // chunk of 16 consecutive rows per 16 lanes; the transposed V reads take
  // chunks 0..3 (of one 64-byte column group) of 4 consecutive rows per 32
  // lanes.  Both hit every LDS bank once when the swizzle is a bijection on
  // any 16 aligned rows and puts the 4 rows of an aligned quad into different
  // 64-byte bank groups (bits 2-3 of the chunk for 256-byte rows; for
  // 128-byte rows, two rows share a 256-byte bank line, so the rows of one
  // parity must differ in bit 2).
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (CHUNKS == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // element offset of chunk c of row r inside a tile
  __device__ static __forceinline__ int at(int r, int c) { return r * D + ((c ^ swz(r)) << 3); }
};

// Four e4m3fn codes (one dword) -> four bf16 values (two dwords), exactly:
// v_cvt_pk_f32_fp8 widens OCP e4m3fn to fp32 on gfx950, and every e4m3fn value
// is a bf16 value, so keeping the upper half of each fp32 loses nothing.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);   // bytes 0, 1
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);    // bytes 2, 3
  lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float wave_pair_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float wave_pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte global -> LDS copy; `lds` is the wave's destination base, lane l's
// bytes land at lds + 16 * l.
__device__ __forceinline__ void dma16(const void* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds), 16, 0, 0);
}

template <int D, int FMT, bool PAGED, bool DEC>
struct Kernel {
  using C = Cfg<D>;
  static constexpr int ESIZE = FMT == kKvFp8 ? 1 : 2;   // bytes per stored element
  static constexpr int RPI = 64 / C::CHUNKS;            // rows per DMA instruction (bf16)
  // fp8 register path: 16-code chunks per row and per-thread work of a block
  static constexpr int F8CH = D / 16;
  static constexpr int F8PASS = kBlockN * F8CH / kThreads;
  static_assert(FMT != kKvFp8 || F8PASS >= 1, "fp8 load split");
  static_assert(FMT != kKvFp8 || F8PASS * 64 == 16 * F8CH, "a wave moves 16 fp8 rows per call");
  // the decode combine area is [4][32][D] fp32 outputs plus [4][32] maxima and
  // [4][32] sums: the two stages hold the outputs, this tail the rest
  static constexpr int kCombineExtra = 2 * kWaves * kWaveRows * 2;   // bf16 elements
  static_assert(kWaves * kWaveRows * D * 4 <= 2 * C::STAGE * 2, "combine area fits the stages");

  struct Item {
    const char* kb;      // K base (bytes) at this item's kv head: cache, or the new tokens without a cache
    const char* vb;      // V base (bytes)
    const char* knb;     // new-token K rows read directly (bf16 cache, new_direct)
    const char* vnb;
    const int32_t* pids;
    uint32_t row_bytes;  // bytes between consecutive token rows of kb / vb
    uint32_t new_row_bytes;
    int first_page;
    int kn_start;
    int cache_len;
    int kvh;
    int kend;
    bool new_direct;
  };

  // Sources of key `key`'s K and V rows for the item's kv head; false when the
  // key is past the item's end (tested only with CHECK) or its page id is
  // unusable.  Token row indices fit 32 bits (the host rejects caches with
  // 2^32 or more slots), so each address is one 32x32->64-bit multiply-add.
  template <bool CHECK>
  __device__ static __forceinline__ bool row_src(const AttnParams& p, const Item& it, int key,
                                                 const char*& kp, const char*& vp) {
    if (CHECK && key >= it.kend) return false;
    if constexpr (PAGED) {
      if (FMT == kKvBf16 && it.new_direct && key >= it.cache_len) {
        // a new token: same bf16 bytes as the slot the append fills
        const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(it.kn_start + key - it.cache_len)) *
                             it.new_row_bytes;
        kp = it.knb + off;
        vp = it.vnb + off;
        return true;
      }
      uint32_t pi, slot;
      if (p.page_shift >= 0) {
        pi = static_cast<uint32_t>(key) >> p.page_shift;
        slot = static_cast<uint32_t>(key) & (p.page_size - 1);
      } else {
        pi = static_cast<uint32_t>(key) / static_cast<uint32_t>(p.page_size);
        slot = static_cast<uint32_t>(key) - pi * p.page_size;
      }
      const int page = it.pids[pi - it.first_page];
      if (page < 0) return false;
      const uint64_t off =
          static_cast<uint64_t>(static_cast<uint32_t>(page) * static_cast<uint32_t>(p.page_size) + slot) *
          it.row_bytes;
      kp = it.kb + off;
      vp = it.vb + off;
      return true;
    } else {
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(it.kn_start + key)) * it.row_bytes;
      kp = it.kb + off;
      vp = it.vb + off;
      return true;
    }
  }

  // ---- bf16: DMA `nrows` tile rows starting at `row0` (row r holds key
  //      kbase + r) into the K and V tiles; the calling wave issues nrows / RPI
  //      copies of each.
  template <bool CHECK>
  __device__ static __forceinline__ void dma_rows(const AttnParams& p, const Item& it,
                                                  uint16_t* ktile, uint16_t* vtile, int kbase,
                                                  int row0, int nrows, int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
#pragma unroll
    for (int i = 0; i < nrows / RPI; ++i) {
      const int r = row0 + i * RPI + lane / C::CHUNKS;
      const int c = (lane % C::CHUNKS) ^ C::swz(r);          // global chunk for this LDS slot
      const char *kp, *vp;
      const bool ok = row_src<CHECK>(p, it, kbase + r, kp, vp);
      dma16(ok ? kp + c * 16 : zeros, ktile + (row0 + i * RPI) * D);
      dma16(ok ? vp + c * 16 : zeros, vtile + (row0 + i * RPI) * D);
    }
  }

  // ---- fp8: rows through registers, widened to bf16 when stored
  struct F8Regs {
    u32x4 k[F8PASS];
    u32x4 v[F8PASS];
  };

  // rows [row0, row0 + nrows) of the tile, `nthreads` threads with index `tid`
  __device__ static __forceinline__ void f8_load(const AttnParams& p, const Item& it, F8Regs& r,
                                                 int kbase, int row0, int nrows, int tid,
                                                 int nthreads) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < F8PASS; ++i) {
      const int idx = tid + i * nthreads;
      const int row = row0 + idx / F8CH;
      const int c = idx % F8CH;
      const char *kp = it.kb, *vp = it.vb;
      const bool ok = row < row0 + nrows && row_src<true>(p, it, kbase + row, kp, vp);
      const u32x4 kv = *reinterpret_cast<const u32x4*>(ok ? kp + c * 16 : it.kb);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(ok ? vp + c * 16 : it.vb);
      r.k[i] = ok ? kv : z;
      r.v[i] = ok ? vv : z;
    }
  }

  __device__ static __forceinline__ void f8_store_one(const u32x4& x, uint16_t* tile, int row, int c) {
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) e4m3x4_to_bf16x4(x[q], w[2 * q], w[2 * q + 1]);
    const u32x4 lo = {w[0], w[1], w[2], w[3]};
    const u32x4 hi = {w[4], w[5], w[6], w[7]};
    *reinterpret_cast<u32x4*>(tile + C::at(row, 2 * c)) = lo;
    *reinterpret_cast<u32x4*>(tile + C::at(row, 2 * c + 1)) = hi;
  }

  __device__ static __forceinline__ void f8_store(const F8Regs& r, uint16_t* ktile, uint16_t* vtile,
                                                  int row0, int nrows, int tid, int nthreads) {
#pragma unroll
    for (int i = 0; i < F8PASS; ++i) {
      const int idx = tid + i * nthreads;
      const int row = row0 + idx / F8CH;
      const int c = idx % F8CH;
      if (row < row0 + nrows) {
        f8_store_one(r.k[i], ktile, row, c);
        f8_store_one(r.v[i], vtile, row, c);
      }
    }
  }

  // ---- a3..a6 for this wave's 32 query rows over keys [kbase, kbase + 32 NH)
  //      held in tile rows [trow0, trow0 + 32 NH).  MASK: some key of the block
  //      lies beyond `lim` (the item's end, or the causal bound of the row).
  template <int NH, bool MASK>
  __device__ static __forceinline__ void compute(const uint16_t* ktile, const uint16_t* vtile,
                                                 int trow0, const bf16x8 (&qf)[C::KSTEPS],
                                                 f32x16 (&o)[C::DBLK], float& m_run, float& l_run,
                                                 int kbase, int lim, float c, int lr, int lg) {
    // Operand fragments are read from LDS one round ahead of the MFMAs that
    // use them (two rounds per phase), so each read's latency hides behind
    // MFMA or softmax work while the live registers stay within budget.
    constexpr int KH = C::KSTEPS / 2;                    // k-steps per K round
    // a3: S^T = K Q^T, NH independent 32-key accumulators interleaved
    f32x16 acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
    bf16x8 kf[2][NH][KH];
#pragma unroll
    for (int s = 0; s < KH; ++s)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        kf[0][h][s] = *reinterpret_cast<const bf16x8*>(ktile + C::at(trow0 + h * 32 + lr, 2 * s + lg));
#pragma unroll
    for (int s = 0; s < KH; ++s)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        kf[1][h][s] =
            *reinterpret_cast<const bf16x8*>(ktile + C::at(trow0 + h * 32 + lr, 2 * (s + KH) + lg));
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[rnd][h][s], qf[rnd * KH + s], acc[h], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // V^T fragments for a6.  Key step j covers tile rows 16j..16j+15; lane
    // (lr, lg) feeds keys 16j + 4lg + e and 16j + 8 + 4lg + e (e = 0..3) for
    // head-dim element lr of the output block, which two transposed reads
    // deliver: in each quarter wave the 16 lanes address 8 bytes (4 head-dim
    // elements) of 4 consecutive V rows, and lane i receives element i of each
    // of those 4 rows.
    const int vrow = lg * 4 + ((lr & 15) >> 2);          // row this lane addresses
    const int vd = (lr & 16) + 4 * (lr & 3);             // first head-dim element it addresses
    auto vread = [&](int j, int d) {
      const int dd = d * 32 + vd;
      const int r1 = trow0 + j * 16 + vrow;
      const uint16_t* a1 = vtile + C::at(r1, dd >> 3) + (dd & 4);
      const uint16_t* a2 = vtile + C::at(r1 + 8, dd >> 3) + (dd & 4);
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
      const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int JH = NH;                               // key steps per V round
    bf16x8 vf[2][JH][C::DBLK];
#pragma unroll
    for (int j = 0; j < JH; ++j)
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d) vf[0][j][d] = vread(j, d);
    __builtin_amdgcn_sched_barrier(0);

    // a4: mask; running max of the raw scores (scale > 0 keeps the order)
    if constexpr (MASK) {
      const int rel = lim - kbase - lg * 4;   // last visible key, relative to this lane's first
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (h * 32 + (i >> 2) * 8 + (i & 3) > rel) acc[h][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[h][i]);
    mx = wave_pair_max(mx);

    // a5: p = 2^(c s - c m), one fma per score.  The reference max m moves
    // only when the block's max exceeds it by more than 2^kLazyLog2 in p:
    // until then p stays below 2^kLazyLog2 (fine for fp32 sums and for bf16
    // P), and O and l need no rescaling.  The result after the final division
    // by l is the same softmax.
    const bool grow = mx * c > m_run * c + kLazyLog2;
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;
    const float neg_mc = m_new == -INFINITY ? 0.f : -m_new * c;
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pf[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[h][i], c, neg_mc));
        psum += pv;
        pf[h][i >> 3][i & 7] = static_cast<__bf16>(pv);
      }
    l_run = l_run * alpha + psum;
    if (__any(grow)) {
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    __builtin_amdgcn_sched_barrier(0);

    // a6: O^T += V^T P^T, second V round read ahead of the first round's MFMAs
#pragma unroll
    for (int j = 0; j < JH; ++j)
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d) vf[1][j][d] = vread(JH + j, d);
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int j = 0; j < JH; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) {
          const int jj = rnd * JH + j;
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[rnd][j][d], pf[jj >> 1][jj & 1], o[d], 0, 0, 0);
        }
  }

  __device__ static __forceinline__ void load_q(const AttnParams& p, const SeqInfo& sq, int kvh,
                                                int prow, bool row_ok, int lg,
                                                bf16x8 (&qf)[C::KSTEPS], int& token, int& qh) {
    token = prow / p.g;
    qh = kvh * p.g + (prow - token * p.g);
    const uint16_t* qrow = p.q + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qrow + s * 16 + lg * 8);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // a7: 4 consecutive head-dim values (from d0) of tile row r, to out / lse or
  // to the split partials
  __device__ static __forceinline__ void store4(const AttnParams& p, const WorkItem& item,
                                                const SeqInfo& sq, int r, int token, int qh, int d0,
                                                float x0, float x1, float x2, float x3, float lse_v,
                                                bool write_lse) {
    if (item.part < 0) {
      uint16_t* orow = p.out + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D + d0;
      u32x2 w2;
      w2[0] = f32_to_bf16_rne(x0) | (static_cast<uint32_t>(f32_to_bf16_rne(x1)) << 16);
      w2[1] = f32_to_bf16_rne(x2) | (static_cast<uint32_t>(f32_to_bf16_rne(x3)) << 16);
      *reinterpret_cast<u32x2*>(orow) = w2;
      if (write_lse && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + sq.q_start + token] = lse_v;
    } else {
      *reinterpret_cast<float4*>(p.part_o + static_cast<int64_t>(item.part + r) * D + d0) =
          make_float4(x0, x1, x2, x3);
      if (write_lse) p.part_lse[item.part + r] = lse_v;
    }
  }

  // ------------------------------------------------------------- prefill
  __device__ static void prefill_item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq,
                                      const Item& it, uint16_t* smem, float c, int wave, int lr,
                                      int lg, int t) {
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int nblk = it.kend > kbeg ? (it.kend - kbeg + kBlockN - 1) / kBlockN : 0;
    uint16_t* const st0 = smem;
    uint16_t* const st1 = smem + C::STAGE;

    // stage the first block (each wave copies 16 of the 64 rows)
    F8Regs fr;
    if (nblk > 0) {
      if constexpr (FMT == kKvFp8) {
        f8_load(p, it, fr, kbeg, 0, kBlockN, t, kThreads);
      } else {
        dma_rows<true>(p, it, st0, st0 + C::TILE, kbeg, wave * 16, 16, lane);
      }
    }

    const int wrow = wave * kWaveRows + lr;
    const bool row_ok = wrow < item.nrows;
    const bool wave_active = wave * kWaveRows < item.nrows;
    bf16x8 qf[C::KSTEPS];
    int token, qh;
    load_q(p, sq, it.kvh, item.row0 + wrow, row_ok, lg, qf, token, qh);

    const int shift = sq.kv_len - sq.q_len;
    int lim = it.kend - 1;
    if (p.causal) lim = min(lim, token + shift);
    int tile_lim = it.kend - 1;
    if (p.causal) tile_lim = min(tile_lim, item.row0 / p.g + shift);

    f32x16 o[C::DBLK];
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    if (nblk > 0) {
      if constexpr (FMT == kKvFp8) {
        f8_store(fr, st0, st0 + C::TILE, 0, kBlockN, t, kThreads);
        if (nblk > 1) f8_load(p, it, fr, kbeg + kBlockN, 0, kBlockN, t, kThreads);
      } else {
        wait_vmem();
      }
      __syncthreads();
    }
    // one block: stage block n + 1 while block n is computed
    auto step = [&](int n, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      uint16_t* const cur = (n & 1) ? st1 : st0;
      uint16_t* const nxt = (n & 1) ? st0 : st1;
      const int kbase = kbeg + n * kBlockN;
      if constexpr (FMT != kKvFp8) {
        if (n + 1 < nblk) {
          if (kbase + 2 * kBlockN <= it.kend)
            dma_rows<false>(p, it, nxt, nxt + C::TILE, kbase + kBlockN, wave * 16, 16, lane);
          else
            dma_rows<true>(p, it, nxt, nxt + C::TILE, kbase + kBlockN, wave * 16, 16, lane);
        }
      }
      if (wave_active) compute<2, MASK>(cur, cur + C::TILE, 0, qf, o, m_run, l_run, kbase, lim, c, lr, lg);
      if constexpr (FMT == kKvFp8) {
        if (n + 1 < nblk) {
          f8_store(fr, nxt, nxt + C::TILE, 0, kBlockN, t, kThreads);
          if (n + 2 < nblk) f8_load(p, it, fr, kbase + 2 * kBlockN, 0, kBlockN, t, kThreads);
        }
      } else {
        wait_vmem();
      }
      __syncthreads();   // stage `cur` is free, stage `nxt` is complete
    };
    // blocks entirely at or below the tile's smallest key bound need no mask
    const int n_full = min(nblk, max(0, (tile_lim - kbeg + 1) / kBlockN));
    int n = 0;
    for (; n < n_full; ++n) step(n, std::false_type{});
    for (; n < nblk; ++n) step(n, std::true_type{});

    if (wave_active) {
      const float l_tot = wave_pair_sum(l_run);
      const bool live = l_tot > 0.f;
      const float inv = live ? p.v_scale / l_tot : 0.f;
      const float lse_v = live ? m_run * c * kLn2 + __logf(l_tot) : -INFINITY;
      if (row_ok) {
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            store4(p, item, sq, wrow, token, qh, d * 32 + i4 * 8 + lg * 4, o[d][i4 * 4 + 0] * inv,
                   o[d][i4 * 4 + 1] * inv, o[d][i4 * 4 + 2] * inv, o[d][i4 * 4 + 3] * inv, lse_v,
                   lg == 0 && d == 0 && i4 == 0);
      }
    }
  }

  // -------------------------------------------------------------- decode
  // Items with at most 32 packed rows (decode steps: q_len * g rows) would
  // leave three of four waves without rows, so the waves split the keys
  // instead: wave w takes the 32-key blocks w, w + 4, ... of the item, staged
  // in its own half of an LDS stage (no workgroup barrier in the loop), and
  // keeps its own running max / sum / output; the four partial states are
  // merged through LDS at the end, the same LSE merge the split pass uses.
  __device__ static void decode_item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq,
                                     const Item& it, uint16_t* smem, float c, int wave, int lr,
                                     int lg, int t) {
    constexpr int DK = 32;
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int nb = it.kend > kbeg ? (it.kend - kbeg + DK - 1) / DK : 0;
    uint16_t* const ktile = smem + (wave >> 1) * C::STAGE;
    uint16_t* const vtile = ktile + C::TILE;
    const int trow0 = (wave & 1) * DK;

    const bool row_ok = lr < item.nrows;
    bf16x8 qf[C::KSTEPS];
    int token, qh;
    load_q(p, sq, it.kvh, item.row0 + lr, row_ok, lg, qf, token, qh);
    const int shift = sq.kv_len - sq.q_len;
    int lim = it.kend - 1;
    if (p.causal) lim = min(lim, token + shift);
    int tile_lim = it.kend - 1;
    if (p.causal) tile_lim = min(tile_lim, item.row0 / p.g + shift);

    f32x16 o[C::DBLK];
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    auto step = [&](int j, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int kbase = kbeg + j * DK;
      wait_lds();   // this wave's reads of its previous block are complete
      if constexpr (FMT == kKvFp8) {
        // one wave moves its 32 rows in two halves of 16 (the per-thread
        // register set is sized for 64 rows over 256 threads)
#pragma unroll
        for (int hr = 0; hr < DK; hr += 16) {
          F8Regs fr;
          f8_load(p, it, fr, kbase - trow0, trow0 + hr, 16, lane, 64);
          f8_store(fr, ktile, vtile, trow0 + hr, 16, lane, 64);
        }
        wait_lds();
      } else {
        if (kbase + DK <= it.kend)
          dma_rows<false>(p, it, ktile, vtile, kbase - trow0, trow0, DK, lane);
        else
          dma_rows<true>(p, it, ktile, vtile, kbase - trow0, trow0, DK, lane);
        wait_vmem();
      }
      compute<1, MASK>(ktile, vtile, trow0, qf, o, m_run, l_run, kbase, lim, c, lr, lg);
    };
    // this wave's blocks j = wave, wave + 4, ...: unmasked while at or below
    // the item's smallest key bound
    const int nb_full = min(nb, max(0, (tile_lim - kbeg + 1) / DK));
    int j = wave;
    for (; j < nb_full; j += kWaves) step(j, std::false_type{});
    for (; j < nb; j += kWaves) step(j, std::true_type{});

    // ---- combine the four waves' states through LDS
    __syncthreads();                     // every wave is done with its stage
    float* const so = reinterpret_cast<float*>(smem);              // [4][32][D]
    float* const sm = so + kWaves * kWaveRows * D;                 // [4][32]
    float* const sl = sm + kWaves * kWaveRows;                     // [4][32]
    const float l_tot = wave_pair_sum(l_run);
    if (row_ok) {
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = d * 32 + i4 * 8 + lg * 4;
          *reinterpret_cast<float4*>(so + (wave * kWaveRows + lr) * D + d0) =
              make_float4(o[d][i4 * 4 + 0], o[d][i4 * 4 + 1], o[d][i4 * 4 + 2], o[d][i4 * 4 + 3]);
        }
      if (lg == 0) {
        sm[wave * kWaveRows + lr] = m_run;
        sl[wave * kWaveRows + lr] = l_tot;
      }
    }
    __syncthreads();
    const int per_row = D / 4;
    for (int idx = t; idx < item.nrows * per_row; idx += kThreads) {
      const int r = idx / per_row;
      const int d0 = (idx - r * per_row) * 4;
      float mw[kWaves];
      float mmax = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = sm[w * kWaveRows + r];
        mmax = fmaxf(mmax, mw[w]);
      }
      float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
      float lsum = 0.f;
      if (mmax != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float wt = __builtin_amdgcn_exp2f((mw[w] - mmax) * c);
          const float4 f = *reinterpret_cast<const float4*>(so + (w * kWaveRows + r) * D + d0);
          lsum += wt * sl[w * kWaveRows + r];
          acc4.x += wt * f.x;
          acc4.y += wt * f.y;
          acc4.z += wt * f.z;
          acc4.w += wt * f.w;
        }
      }
      const bool live = lsum > 0.f;
      const float inv = live ? p.v_scale / lsum : 0.f;
      const float lse_v = live ? mmax * c * kLn2 + __logf(lsum) : -INFINITY;
      const int pr = item.row0 + r;
      const int tok = pr / p.g;
      const int h = it.kvh * p.g + (pr - tok * p.g);
      store4(p, item, sq, r, tok, h, d0, acc4.x * inv, acc4.y * inv, acc4.z * inv, acc4.w * inv,
             lse_v, d0 == 0);
    }
  }

  __device__ static void run(const AttnParams& p) {
    // two K/V stages (the block being computed and the block being staged);
    // decode items use them as four per-wave half stages, then as the area
    // where the waves combine their partial softmax states
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * C::STAGE + (DEC ? kCombineExtra : 0)];
    __shared__ int32_t pids[PAGED ? kMaxItemPages : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;   // query column of this lane
    const int lg = lane >> 5;   // lane half
    const float c = p.qk_scale_log2;

    // workgroups past the attention part of the grid store new tokens
    if (static_cast<int>(blockIdx.x) >= p.attn_blocks) {
      append_token(p.app, blockIdx.x - p.attn_blocks, t, kThreads);
      return;
    }

    int w_idx = blockIdx.x, w_end = blockIdx.x + 1;
    if (p.persistent) {
      w_idx = p.queue_start[blockIdx.x];
      w_end = p.queue_start[blockIdx.x + 1];
    }

    for (; w_idx < w_end; ++w_idx) {
      // work = unit * hkv + kv head
      const int work = p.persistent ? p.queue_work[w_idx] : w_idx;
      const int unit = work / p.hkv;
      const int kvh = work - unit * p.hkv;
      WorkItem item = p.items[unit];
      if (item.part >= 0) item.part += kvh * item.part_stride;
      const SeqInfo sq = p.seqs[item.seq];
      Item it;
      it.row_bytes = static_cast<uint32_t>(p.hkv) * (D * ESIZE);
      it.new_row_bytes = static_cast<uint32_t>(p.hkv) * (D * 2);
      it.kb = static_cast<const char*>(p.k) + kvh * (D * ESIZE);
      it.vb = static_cast<const char*>(p.v) + kvh * (D * ESIZE);
      it.knb = static_cast<const char*>(p.k_new) + kvh * (D * 2);
      it.vnb = static_cast<const char*>(p.v_new) + kvh * (D * 2);
      it.pids = pids;
      it.first_page = 0;
      it.kn_start = sq.kn_start;
      it.cache_len = sq.cache_len;
      it.kvh = kvh;
      it.kend = item.key_end;
      it.new_direct = p.new_direct != 0;

      // ---- page ids of the item's key range -> LDS
      if constexpr (PAGED) {
        if (item.key_end > item.key_begin) {
          it.first_page = item.key_begin / p.page_size;
          const int last_page = (item.key_end - 1) / p.page_size;
          const int32_t* bt = p.block_table + static_cast<int64_t>(item.seq) * p.max_pages;
          for (int i = t; i <= last_page - it.first_page; i += kThreads) {
            int pg = bt[it.first_page + i];
            if (pg < 0 || pg >= p.num_pages) {
              atomicOr(p.err_flag, 1);
              pg = -1;
            }
            pids[i] = pg;
          }
          __syncthreads();
        }
      }

      if constexpr (DEC)
        decode_item(p, item, sq, it, smem, c, wave, lr, lg, t);
      else
        prefill_item(p, item, sq, it, smem, c, wave, lr, lg, t);
      __syncthreads();   // LDS (stages, page ids, combine area) free for the next item
    }
  }
};

// One kernel per item mode: prefill-mode items (more than 32 rows) and
// decode-mode items each get the full register budget of two waves per SIMD.
template <int D, int FMT, bool PAGED, bool DEC>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const AttnParams p) {
  Kernel<D, FMT, PAGED, DEC>::run(p);
}

template <int D, int FMT, bool PAGED>
int launch_t(const AttnParams& p, int grid, bool decode, hipStream_t s) {
  if (decode)
    hipLaunchKernelGGL((attn_fwd_kernel<D, FMT, PAGED, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, FMT, PAGED, false>), dim3(grid), dim3(kThreads), 0, s, p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_attention(const AttnParams& p, int grid, int head_dim, int kv_format, bool paged,
                     bool decode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) {
    if (!paged) return launch_t<128, kKvBf16, false>(p, grid, decode, s);
    if (kv_format == kKvFp8) return launch_t<128, kKvFp8, true>(p, grid, decode, s);
    return launch_t<128, kKvBf16, true>(p, grid, decode, s);
  }
  if (head_dim == 64) {
    if (!paged) return launch_t<64, kKvBf16, false>(p, grid, decode, s);
    if (kv_format == kKvFp8) return launch_t<64, kKvFp8, true>(p, grid, decode, s);
    return launch_t<64, kKvBf16, true>(p, grid, decode, s);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

}  // namespace vpk
