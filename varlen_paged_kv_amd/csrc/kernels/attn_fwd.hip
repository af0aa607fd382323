// Attention over a paged KV cache for packed variable-length queries, gfx950.
//
// Rows are (token, query head) pairs packed token-major, so the g query heads
// that share a kv head (grouped-query attention, vLLM Triton FAv2 PR page,
// feature list) all use each K/V tile staged in LDS.  A work item is a tile of
// packed rows of one sequence under one kv head, against the keys
// [key_begin, key_end) of that sequence.  Two kernels serve the two kinds of
// items:
//
// Prefill mode (items of up to 256 rows; 8 wavefronts of 32 rows, one
// workgroup per CU).  Per 64-key block:
//   a2  K and V rows of the block are gathered through the item's page ids
//       (one page table for K and V: TransformerEngine KV-cache PR page,
//       Description).  bf16 rows go straight from HBM to LDS with
//       global_load_lds (16 bytes per lane, no registers); fp8 e4m3fn rows go
//       through registers and are widened to bf16 exactly on the way.  Tiles
//       are row-major with the 16-byte chunks of each row XOR-swizzled; rows
//       past the item's keys are loaded from a zero region.  Blocks rotate
//       through a four-stage ring, staged up to three blocks ahead.
//   a3  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//       column and 32 of the block's 64 keys, the other 32 sit in lane ^ 32.
//   a4  keys beyond the item's end, or (causal) beyond token + Lk - Lq, get
//       -inf; only blocks that cross the bound of some row of a wave are
//       masked, and blocks no row of a wave can see are skipped by that wave.
//   a5  online softmax in base 2 on the raw scores: row max over registers
//       plus one permlane32 swap, p = 2^(s c - m c) with one fma, running
//       sum per lane; the reference max only moves when the block max
//       exceeds it by 2^8 in p, so O is rarely rescaled.
//   a6  O^T += V^T P^T on the same MFMA; the V^T operand comes from
//       ds_read_b64_tr_b16 transposed LDS reads of the row-major V tile, P is
//       rounded to bf16 in registers.
//   a7  out = O / l (bf16) and lse = m c ln 2 + ln l, or for a split part the
//       fp32 normalised partial and its lse for the merge pass.
// Decode mode (items of at most 32 rows: a decode step's q_len * g rows).  The
// four waves of a 256-thread workgroup split the item's 32-key blocks, each
// with its own LDS half stage, and merge their partial states through LDS at
// the end, the same LSE merge the split pass uses.
//
// The online softmax and the split of the key range into parts merged by LSE
// follow the FlashAttention-2 design the pages build on ("Add
// flash_attn_varlen_func_with_kvcache", Limitation and the discussion of
// split-KV for decoding); the tiling, the transposed S layout, the LDS layout
// and the pipelining are this library's own for CDNA4.
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
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
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
// gfx950's v_cvt_scalef32_pk_bf16_fp8 widens two OCP e4m3fn codes straight to
// two bf16 values times a scale; with the scale 1 nothing is rounded, since
// every e4m3fn value is a bf16 value (one instruction per two codes).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));   // bytes 0, 1
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));    // bytes 2, 3
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

// wait until at most n (0..8) vector-memory instructions of this wave are in
// flight; larger n waits for at most 8
__device__ __forceinline__ void wait_vmem_upto(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
  }
}

// a ^ b computed where it is used: the compiler cannot hoist it out of a
// loop (hoisted lane-dependent addresses would not fit the register budget,
// and their spill reloads would wait for all vector memory)
__device__ __forceinline__ int xor_here(int a, int b) {
  int r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// 16-byte global -> LDS copy; `lds` is the wave's destination base (uniform),
// lane l's bytes land at lds + 16 * l.  ASYNC: issued as inline assembly, so
// the compiler does not treat the copy as an LDS store that every later LDS
// read must wait for (it would wait for all copies in flight, including the
// ones staged blocks ahead); completion is then ordered only by the explicit
// vmcnt waits and barriers of the caller.  Loads complete in issue order, so
// the compiler's own vmcnt waits for its loads stay correct with these in the
// queue.  M0 holds the LDS base; one wait state separates its write from the
// copy.  Without ASYNC the compiler's builtin is used and orders the copy
// itself.
template <bool ASYNC>
__device__ __forceinline__ void dma16(const void* g, uint16_t* lds) {
  if constexpr (!ASYNC) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds), 16, 0, 0);
    return;
  }
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(lds))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(base)
               : "memory", "m0");
}

// The same copy from a uniform 64-bit base plus a per-lane 32-bit byte offset
// (the global_load saddr form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16_base(const char* base, uint32_t off, uint16_t* lds) {
  const uint32_t lb = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(lds))));
  // (readfirstlane yields an int: each half goes through uint32_t so that it
  // is zero-extended)
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t bs = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(bs), "s"(lb)
               : "memory", "m0");
}

// ---------------------------------------------------------------- shared parts
template <int D, int FMT, bool PAGED>
struct Src {
  using C = Cfg<D>;
  static constexpr int ESIZE = FMT == kKvFp8 ? 1 : 2;   // bytes per stored element
  static constexpr int RPI = 64 / C::CHUNKS;            // rows per DMA instruction (bf16)
  static constexpr int F8CH = D / 16;                   // 16-code chunks of an fp8 row

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
  // 2^31 or more slots), so each address is one 32x32->64-bit multiply-add.
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

  // ---- bf16: DMA tile rows [row0, row0 + nrows) (row r holds key kbase + r)
  //      of K (V_ROWS false) or V into `tile`; the calling wave issues
  //      nrows / RPI copies.
  template <bool CHECK, bool V_ROWS, bool ASYNC = false>
  __device__ static __forceinline__ void dma_tile(const AttnParams& p, const Item& it, uint16_t* tile,
                                                  int kbase, int row0, int nrows, int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
#pragma unroll
    for (int i = 0; i < nrows / RPI; ++i) {
      const int r = row0 + i * RPI + lane / C::CHUNKS;
      const int c = (lane % C::CHUNKS) ^ C::swz(r);          // global chunk for this LDS slot
      const char *kp, *vp;
      const bool ok = row_src<CHECK>(p, it, kbase + r, kp, vp);
      dma16<ASYNC>(ok ? (V_ROWS ? vp : kp) + c * 16 : zeros, tile + (row0 + i * RPI) * D);
    }
  }

  // ---- bf16: when keys [key0, key0 + n) are all before the item's end and
  //      their rows are consecutive in one source (one page, the new tokens,
  //      or the unpaged K/V), the row of key0 and the row stride; all values
  //      uniform over the wave.
  __device__ static __forceinline__ bool rows_contig(const AttnParams& p, const Item& it, int key0, int n,
                                                     const char*& k0, const char*& v0, uint32_t& stride) {
    key0 = __builtin_amdgcn_readfirstlane(key0);
    if (key0 + n > it.kend) return false;
    if constexpr (PAGED) {
      if (FMT == kKvBf16 && it.new_direct && key0 + n > it.cache_len) {
        if (key0 < it.cache_len) return false;
        const uint64_t off =
            static_cast<uint64_t>(static_cast<uint32_t>(it.kn_start + key0 - it.cache_len)) * it.new_row_bytes;
        k0 = it.knb + off;
        v0 = it.vnb + off;
        stride = it.new_row_bytes;
        return true;
      }
      uint32_t pi, pl, slot;
      if (p.page_shift >= 0) {
        pi = static_cast<uint32_t>(key0) >> p.page_shift;
        pl = static_cast<uint32_t>(key0 + n - 1) >> p.page_shift;
        slot = static_cast<uint32_t>(key0) & (p.page_size - 1);
      } else {
        pi = static_cast<uint32_t>(key0) / static_cast<uint32_t>(p.page_size);
        pl = static_cast<uint32_t>(key0 + n - 1) / static_cast<uint32_t>(p.page_size);
        slot = static_cast<uint32_t>(key0) - pi * p.page_size;
      }
      if (pi != pl) return false;
      const int page = __builtin_amdgcn_readfirstlane(it.pids[pi - it.first_page]);
      if (page < 0) return false;
      const uint64_t off =
          static_cast<uint64_t>(static_cast<uint32_t>(page) * static_cast<uint32_t>(p.page_size) + slot) *
          it.row_bytes;
      k0 = it.kb + off;
      v0 = it.vb + off;
    } else {
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(it.kn_start + key0)) * it.row_bytes;
      k0 = it.kb + off;
      v0 = it.vb + off;
    }
    stride = it.row_bytes;
    return true;
  }

  // tile rows [row0, row0 + nrows) from consecutive source rows at `src`
  // (row r + row0 at src + r * stride); the calling wave issues nrows / RPI
  // copies
  __device__ static __forceinline__ void dma_rows(const char* src, uint32_t stride, uint16_t* tile, int row0,
                                                  int nrows, int lane) {
#pragma unroll
    for (int i = 0; i < nrows / RPI; ++i) {
      const int rr = i * RPI + lane / C::CHUNKS;
      const int c = (lane % C::CHUNKS) ^ C::swz(row0 + rr);
      dma16_base(src, static_cast<uint32_t>(rr) * stride + c * 16, tile + (row0 + i * RPI) * D);
    }
  }

  // ---- fp8: rows through registers, widened to bf16 when stored.  `n`
  //      threads of index `tid` move rows [row0, row0 + nrows) of one tile;
  //      each thread holds up to NPASS 16-code chunks.
  template <int NPASS>
  struct F8Regs {
    u32x4 x[NPASS];
  };

  template <int NPASS, bool V_ROWS>
  __device__ static __forceinline__ void f8_load(const AttnParams& p, const Item& it, F8Regs<NPASS>& r,
                                                 int kbase, int row0, int nrows, int tid, int n) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int idx = tid + i * n;
      const int row = row0 + idx / F8CH;
      const int c = idx % F8CH;
      const char *kp = it.kb, *vp = it.vb;
      const bool ok = row < row0 + nrows && row_src<true>(p, it, kbase + row, kp, vp);
      const char* src = V_ROWS ? vp : kp;
      const u32x4 x = *reinterpret_cast<const u32x4*>(ok ? src + c * 16 : (V_ROWS ? it.vb : it.kb));
      r.x[i] = ok ? x : z;
    }
  }

  template <int NPASS>
  __device__ static __forceinline__ void f8_store(const F8Regs<NPASS>& r, uint16_t* tile, int row0,
                                                  int nrows, int tid, int n) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int idx = tid + i * n;
      const int row = row0 + idx / F8CH;
      const int c = idx % F8CH;
      if (row < row0 + nrows) {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) e4m3x4_to_bf16x4(r.x[i][q], w[2 * q], w[2 * q + 1]);
        const u32x4 lo = {w[0], w[1], w[2], w[3]};
        const u32x4 hi = {w[4], w[5], w[6], w[7]};
        *reinterpret_cast<u32x4*>(tile + C::at(row, 2 * c)) = lo;
        *reinterpret_cast<u32x4*>(tile + C::at(row, 2 * c + 1)) = hi;
      }
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

  // Rotary embedding of this lane's query chunks (chunk 2 s + lg at k-step s)
  // at position `pos` = Lk - Lq + token (the key the row's end-aligned causal
  // bound stops at).  The angles are loaded first (rope_load, issued with the
  // Q loads and the first staging copies, so one memory round trip covers
  // them all) and applied once they have arrived (rope_apply).  The caller
  // turns only rotary dims that are multiples of 32 in the half-split
  // pairing, so that both chunks of a pair (c and c + dim / 16, k-steps s and
  // s + dim / 32) sit in one lane; interleaved pairs sit inside one chunk.
  // Angle slots: interleaved, a[s] = {cos, sin} of k-step s's 4 pairs;
  // half-split, a[s] = cos and a[s + KSTEPS / 2] = sin of the 8 pairs whose
  // first chunk is at k-step s.
  struct QAngles {
    float4 a[C::KSTEPS][2];
  };
  __device__ static __forceinline__ void rope_load(const RopeArgs& r, int pos, int lg, QAngles& g) {
    const int half = r.dim >> 1;
    const float* cr = r.cos + static_cast<int64_t>(pos) * half;
    const float* sr = r.sin + static_cast<int64_t>(pos) * half;
    if (r.interleaved) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const int d0 = 16 * s + 8 * lg;
        if (d0 < r.dim) {
          g.a[s][0] = *reinterpret_cast<const float4*>(cr + (d0 >> 1));
          g.a[s][1] = *reinterpret_cast<const float4*>(sr + (d0 >> 1));
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < C::KSTEPS / 2; ++s) {
      if (16 * s < half) {
        const int i0 = 16 * s + 8 * lg;
        g.a[s][0] = *reinterpret_cast<const float4*>(cr + i0);
        g.a[s][1] = *reinterpret_cast<const float4*>(cr + i0 + 4);
        g.a[s + C::KSTEPS / 2][0] = *reinterpret_cast<const float4*>(sr + i0);
        g.a[s + C::KSTEPS / 2][1] = *reinterpret_cast<const float4*>(sr + i0 + 4);
      }
    }
  }
  __device__ static __forceinline__ void rope_apply(const RopeArgs& r, int lg, const QAngles& g,
                                                    bf16x8 (&qf)[C::KSTEPS]) {
    using namespace rope_detail;
    if (r.interleaved) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        if (16 * s + 8 * lg < r.dim) {
          const float cs[4] = {g.a[s][0].x, g.a[s][0].y, g.a[s][0].z, g.a[s][0].w};
          const float sn[4] = {g.a[s][1].x, g.a[s][1].y, g.a[s][1].z, g.a[s][1].w};
          u32x4 x = __builtin_bit_cast(u32x4, qf[s]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint16_t ra, rb;
            turn(bf16_lo(x[q]), bf16_hi(x[q]), cs[q], sn[q], ra, rb);
            x[q] = ra | (static_cast<uint32_t>(rb) << 16);
          }
          qf[s] = __builtin_bit_cast(bf16x8, x);
        }
      }
      return;
    }
    switch (r.dim >> 5) {
      case 1: rope_pairs<1>(g, qf); break;
      case 2: rope_pairs<2>(g, qf); break;
      case 3: if constexpr (C::KSTEPS >= 6) rope_pairs<3>(g, qf); break;
      case 4: if constexpr (C::KSTEPS >= 8) rope_pairs<4>(g, qf); break;
      default: break;
    }
  }
  template <int DS>
  __device__ static __forceinline__ void rope_pairs(const QAngles& g, bf16x8 (&qf)[C::KSTEPS]) {
    using namespace rope_detail;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const float4 c0 = g.a[s][0], c1 = g.a[s][1];
      const float4 s0 = g.a[s + C::KSTEPS / 2][0], s1 = g.a[s + C::KSTEPS / 2][1];
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      u32x4 a = __builtin_bit_cast(u32x4, qf[s]);
      u32x4 b = __builtin_bit_cast(u32x4, qf[s + DS]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t a0, b0, a1, b1;
        turn(bf16_lo(a[q]), bf16_lo(b[q]), cs[2 * q], sn[2 * q], a0, b0);
        turn(bf16_hi(a[q]), bf16_hi(b[q]), cs[2 * q + 1], sn[2 * q + 1], a1, b1);
        a[q] = a0 | (static_cast<uint32_t>(a1) << 16);
        b[q] = b0 | (static_cast<uint32_t>(b1) << 16);
      }
      qf[s] = __builtin_bit_cast(bf16x8, a);
      qf[s + DS] = __builtin_bit_cast(bf16x8, b);
    }
  }

  // a7: 4 consecutive head-dim values (from d0) of tile row r, to out / lse or
  // to the split partials
  __device__ static __forceinline__ void store4(const AttnParams& p, int part, int q_start, int r, int token,
                                                int qh, int d0, float x0, float x1, float x2, float x3,
                                                float lse_v, bool write_lse) {
    if (part < 0) {
      uint16_t* orow = p.out + (static_cast<int64_t>(q_start + token) * p.hq + qh) * D + d0;
      u32x2 w2;
      w2[0] = f32_to_bf16_rne(x0) | (static_cast<uint32_t>(f32_to_bf16_rne(x1)) << 16);
      w2[1] = f32_to_bf16_rne(x2) | (static_cast<uint32_t>(f32_to_bf16_rne(x3)) << 16);
      *reinterpret_cast<u32x2*>(orow) = w2;
      if (write_lse && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + q_start + token] = lse_v;
    } else {
      *reinterpret_cast<float4*>(p.part_o + static_cast<int64_t>(part + r) * D + d0) =
          make_float4(x0, x1, x2, x3);
      if (write_lse) p.part_lse[part + r] = lse_v;
    }
  }

  // a7 for a whole row pair of lanes: output block d (32 head-dim values) of
  // this lane's row, from the O^T accumulator layout, where lane half lg
  // holds values 8 i + 4 lg + (0..3), i = 0..3.  Two permlane32 swaps per 16
  // values give lane half 0 the values 16 k + (0..7) and lane half 1 the
  // values 16 k + 8 + (0..7), so each row is written as contiguous 16-byte
  // pieces (half as many store instructions as 8-byte stores).
  __device__ static __forceinline__ void store_out_block(const AttnParams& p, int q_start, int token, int qh,
                                                         int d, const f32x16& od, float inv, int lg,
                                                         bool row_ok) {
    uint16_t* orow = p.out + (static_cast<int64_t>(q_start + token) * p.hq + qh) * D + d * 32 + lg * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t x[2], y[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        x[e] = f32_to_bf16_rne(od[8 * k + 2 * e] * inv) |
               (static_cast<uint32_t>(f32_to_bf16_rne(od[8 * k + 2 * e + 1] * inv)) << 16);
        y[e] = f32_to_bf16_rne(od[8 * k + 4 + 2 * e] * inv) |
               (static_cast<uint32_t>(f32_to_bf16_rne(od[8 * k + 4 + 2 * e + 1] * inv)) << 16);
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // vdst x: upper lanes receive y of the lower lanes; src y: lower
        // lanes receive x of the upper lanes
        const auto s = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
        w[e] = s[0];
        w[2 + e] = s[1];
      }
      if (row_ok) *reinterpret_cast<u32x4*>(orow + 16 * k) = w;
    }
  }

  // Work-queue entries of a workgroup, read from the plan once per chunk of
  // the queue into LDS (the plan lives in pinned host memory, so each read
  // crosses PCIe: one round trip per chunk instead of one per item).
  struct QEntry {
    WorkItem item;       // with its sequence's facts in item.s
    int32_t kvh;
    int32_t dec;         // decode-mode item (unit at or past p.num_pre_units)
    int32_t pad[2];
  };
  static constexpr int kQueueChunk = 48;

  // Entries [w0, w0 + n) of the grid's work list (the workgroup's queue when
  // persistent) -> q[0, n), by `nt` threads; the caller synchronises.
  __device__ static __forceinline__ void load_queue(const AttnParams& p, int w0, int n, QEntry* q, int t,
                                                    int nt) {
    for (int i = t; i < n; i += nt) {
      // work = unit * hkv + kv head
      const int work = p.persistent ? p.queue_work[w0 + i] : w0 + i;
      const int unit = work / p.hkv;
      const int kvh = work - unit * p.hkv;
      WorkItem item = p.items[unit];
      if (item.part >= 0) item.part += kvh * item.part_stride;
      q[i].item = item;
      q[i].kvh = kvh;
      q[i].dec = unit >= p.num_pre_units ? 1 : 0;
    }
  }

  // Sources of an entry's keys and values; with a cache, its page ids are
  // staged in `pids` (LDS) by all `nt` threads.
  __device__ static __forceinline__ void setup_item(const AttnParams& p, const QEntry& e, int32_t* pids, int t,
                                                    int nt, Item& it) {
    // every field is the same for all lanes: keep them in scalar registers
    const int kvh = __builtin_amdgcn_readfirstlane(e.kvh);
    it.row_bytes = static_cast<uint32_t>(p.hkv) * (D * ESIZE);
    it.new_row_bytes = static_cast<uint32_t>(p.hkv) * (D * 2);
    it.kb = static_cast<const char*>(p.k) + kvh * (D * ESIZE);
    it.vb = static_cast<const char*>(p.v) + kvh * (D * ESIZE);
    it.knb = static_cast<const char*>(p.k_new) + kvh * (D * 2);
    it.vnb = static_cast<const char*>(p.v_new) + kvh * (D * 2);
    it.pids = pids;
    it.first_page = 0;
    it.kn_start = __builtin_amdgcn_readfirstlane(e.item.s.kn_start);
    it.cache_len = __builtin_amdgcn_readfirstlane(e.item.s.cache_len);
    it.kvh = kvh;
    it.kend = __builtin_amdgcn_readfirstlane(e.item.key_end);
    it.new_direct = p.new_direct != 0;
    // page ids of the item's key range -> LDS
    if constexpr (PAGED) {
      if (e.item.key_end > e.item.key_begin) {
        it.first_page = __builtin_amdgcn_readfirstlane(e.item.key_begin / p.page_size);
        const int last_page = (e.item.key_end - 1) / p.page_size;
        const int32_t* bt = p.block_table + e.item.s.bt_row;
        for (int i = t; i <= last_page - it.first_page; i += nt) {
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
  }

  // The workgroup's items: [blockIdx, blockIdx + 1) of the grid, or its queue
  // when persistent; `body(entry, item)` runs each, all threads together.
  // FILTER 0 / 1: only the prefill-mode / decode-mode entries (-1: all).
  template <int FILTER = -1, typename Body>
  __device__ static __forceinline__ void for_each_item(const AttnParams& p, QEntry* qbuf, int32_t* pids, int t,
                                                       int nt, Body&& body) {
    int w0 = blockIdx.x, w_end = blockIdx.x + 1;
    if (p.persistent) {
      w0 = p.queue_start[blockIdx.x];
      w_end = p.queue_start[blockIdx.x + 1];
    }
    for (; w0 < w_end; w0 += kQueueChunk) {
      const int n = min(kQueueChunk, w_end - w0);
      load_queue(p, w0, n, qbuf, t, nt);
      __syncthreads();
      for (int k = 0; k < n; ++k) {
        const QEntry& e = qbuf[k];
        if constexpr (FILTER >= 0) {
          if (__builtin_amdgcn_readfirstlane(e.dec) != FILTER) continue;
        }
        Item it;
        setup_item(p, e, pids, t, nt, it);
        body(e, it);
        __syncthreads();   // LDS (stages, page ids) free for the next item
      }
    }
  }

  // a4 + a5 on a 32-query x 32 NH-key score block `acc` (S^T layout): mask,
  // running max with the lazy reference, p = 2^(c s - c m) rounded to bf16
  // into pf, running sum, and the O rescale when some row's reference moved.
  template <int NH, bool MASK>
  __device__ static __forceinline__ void softmax(f32x16 (&acc)[NH], bf16x8 (&pf)[NH][2],
                                                 f32x16 (&o)[C::DBLK], float& m_run, float& l_run,
                                                 int kbase, int lim, float c, int lg) {
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
    // The reference max m moves only when the block's max exceeds it by more
    // than 2^kLazyLog2 in p: until then p stays below 2^kLazyLog2 (fine for
    // fp32 sums and for bf16 P), and O and l need no rescaling.  The result
    // after the final division by l is the same softmax.
    const bool grow = mx * c > m_run * c + kLazyLog2;
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;
    const float neg_mc = m_new == -INFINITY ? 0.f : -m_new * c;
    m_run = m_new;
    float psum = 0.f;
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
  }

  // V^T operand fragment of key step j (tile rows trow0 + 16j .. + 15) and
  // output block d.  Lane (lr, lg) feeds keys 16j + 4lg + e and 16j + 8 + 4lg
  // + e (e = 0..3) for head-dim element lr of block d, which two transposed
  // reads deliver: in each quarter wave the 16 lanes address 8 bytes (4
  // head-dim elements) of 4 consecutive V rows, and lane i receives element i
  // of each of those 4 rows.  This key order matches the P^T operand built
  // from the S^T accumulator layout.
  __device__ static __forceinline__ bf16x8 vread(const uint16_t* vtile, int trow0, int j, int d, int lr,
                                                 int lg) {
    const int vrow = lg * 4 + ((lr & 15) >> 2);          // row this lane addresses
    const int vd = (lr & 16) + 4 * (lr & 3);             // first head-dim element it addresses
    const int dd = d * 32 + vd;
    const int r1 = trow0 + j * 16 + vrow;
    const uint16_t* a1 = vtile + C::at(r1, dd >> 3) + (dd & 4);
    const uint16_t* a2 = vtile + C::at(r1 + 8, dd >> 3) + (dd & 4);
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // K operand fragment: key row r of the tile, head-dim chunk pair k-step s
  __device__ static __forceinline__ bf16x8 kread(const uint16_t* ktile, int r, int s, int lg) {
    return *reinterpret_cast<const bf16x8*>(ktile + C::at(r, 2 * s + lg));
  }

  // ---- a3 alone: S^T of this wave's 32 query rows against tile rows
  //      [trow0, trow0 + 32 NH) into acc; all K fragments are read first.
  template <int NH>
  __device__ static __forceinline__ void qk(const uint16_t* ktile, int trow0, const bf16x8 (&qf)[C::KSTEPS],
                                            f32x16 (&acc)[NH], int lr, int lg) {
    constexpr int KH = C::KSTEPS / 2;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
    bf16x8 kf[2][NH][KH];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h) kf[rnd][h][s] = kread(ktile, trow0 + h * 32 + lr, rnd * KH + s, lg);
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[rnd][h][s], qf[rnd * KH + s], acc[h], 0, 0, 0);
  }

  // ---- a6 alone: O^T += V^T P^T over tile rows [trow0, trow0 + 32 NH); the
  //      second round of V fragments is read while the first round's MFMAs run
  template <int NH>
  __device__ static __forceinline__ void pv(const uint16_t* vtile, int trow0, const bf16x8 (&pf)[NH][2],
                                            f32x16 (&o)[C::DBLK], int lr, int lg) {
    constexpr int JH = NH;
    bf16x8 vf[2][JH][C::DBLK];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int j = 0; j < JH; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) vf[rnd][j][d] = vread(vtile, trow0, rnd * JH + j, d, lr, lg);
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

  // ---- a3 and a6 as above for tile rows from 0, with the LDS addresses
  //      formed where they are used.  The swizzle only XORs the chunk index,
  //      so the address of k-step s is the k-step 0 address XOR 32 s bytes,
  //      and that of V output block d the block 0 address XOR 64 d bytes;
  //      rows 32 (K) or 16 (V) further on are plain immediate offsets.  The
  //      XORs run next to their reads, so no per-step address stays live
  //      across the key loop.
  __device__ static __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(p)));
  }
  template <typename T>
  __device__ static __forceinline__ T lds_read(uint32_t a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>(static_cast<uintptr_t>(a));
  }
  template <int NH>
  __device__ static __forceinline__ void qk0(const uint16_t* ktile, const bf16x8 (&qf)[C::KSTEPS],
                                             f32x16 (&acc)[NH], int lr, int lg) {
    constexpr int KH = C::KSTEPS / 2;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
    const uint32_t a0 = lds_addr(ktile + C::at(lr, lg));
    bf16x8 kf[2][NH][KH];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s) {
        const int ks = rnd * KH + s;
        const uint32_t a = ks ? static_cast<uint32_t>(xor_here(static_cast<int>(a0), 32 * ks)) : a0;
#pragma unroll
        for (int h = 0; h < NH; ++h) kf[rnd][h][s] = lds_read<bf16x8>(a + h * 32 * D * 2);
      }
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[rnd][h][s], qf[rnd * KH + s], acc[h], 0, 0, 0);
  }
  template <int NH>
  __device__ static __forceinline__ void pv0(const uint16_t* vtile, const bf16x8 (&pf)[NH][2],
                                             f32x16 (&o)[C::DBLK], int lr, int lg) {
    constexpr int JH = NH;
    const int vrow = lg * 4 + ((lr & 15) >> 2);
    const int vd = (lr & 16) + 4 * (lr & 3);
    const uint32_t b1 = lds_addr(vtile + C::at(vrow, vd >> 3) + (vd & 4));
    const uint32_t b2 = lds_addr(vtile + C::at(vrow + 8, vd >> 3) + (vd & 4));
    uint32_t a1[C::DBLK], a2[C::DBLK];
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d) {
      a1[d] = d ? static_cast<uint32_t>(xor_here(static_cast<int>(b1), 64 * d)) : b1;
      a2[d] = d ? static_cast<uint32_t>(xor_here(static_cast<int>(b2), 64 * d)) : b2;
    }
    bf16x8 vf[2][JH][C::DBLK];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int j = 0; j < JH; ++j)
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d) {
          const uint32_t off = (rnd * JH + j) * 16 * D * 2;
          const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<lds_i16x4*>(static_cast<uintptr_t>(a1[d] + off)));
          const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<lds_i16x4*>(static_cast<uintptr_t>(a2[d] + off)));
          vf[rnd][j][d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7));
        }
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

  // ---- fp8 cache, decode mode: raw e4m3fn code rows in LDS, widened when
  //      the MFMA fragments are read.  A wave's 16 KB region (32 bf16 rows of
  //      K and of V) holds 64 code rows of 128 bytes (head_dim 128) of K and
  //      of V, so a wave keeps 64 keys in flight instead of the 32 it could
  //      hold widened.  Chunk c (16 bytes) of code row r sits at c ^ f8swz(r):
  //      the transposed V reads of a 16-lane group take chunks c and c ^ 1 of
  //      rows {0..3, 8..11} (+ 4 or + 16 j), which then fall into distinct
  //      bank groups.
  static constexpr int F8ROW = D;   // bytes of a code row
  __device__ static __forceinline__ int f8swz(int r) {
    return (((r >> 1) & 1) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 2);
  }
  // rows [0, 64) of a region <- keys [kbase, kbase + 64) of K (V_ROWS false)
  // or V; rows past the item's end or on an unusable page read zeros; the
  // calling wave issues 8 copies of 8 rows
  template <bool V_ROWS>
  __device__ static __forceinline__ void dma_raw8(const AttnParams& p, const Item& it, uint8_t* region, int kbase,
                                                  int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ f8swz(r);
      const char *kp, *vp;
      const bool ok = row_src<true>(p, it, kbase + r, kp, vp);
      dma16<true>(ok ? (V_ROWS ? vp : kp) + c * 16 : zeros, reinterpret_cast<uint16_t*>(region + i * 8 * F8ROW));
    }
  }
  // New tokens among keys [kbase, kbase + 64) of an fp8 decode-mode block
  // (AttnParams::dec_append): after the block's copies have landed, each lane
  // replaces the 16 codes its copy brought for such a row (the slot the
  // append would fill, not yet written) by the codes of k_new / v_new under
  // the append's encoder, in LDS and in the cache.  Rows on an unusable page
  // keep the zeros their copy read, as with the standalone append.
  __device__ static __forceinline__ void dec_new8(const AttnParams& p, const Item& it, uint8_t* rk, uint8_t* rv,
                                                  int kbase, int lane) {
    using append_detail::enc2;
    if (kbase + 64 <= it.cache_len) return;
    float k_inv = p.app.k_inv_scale, v_inv = p.app.v_inv_scale;
    if (p.app.kv_scale_dev) {
      k_inv = 1.0f / p.app.kv_scale_dev[0];
      v_inv = 1.0f / p.app.kv_scale_dev[1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int key = kbase + r;
      if (key < it.cache_len || key >= it.kend) continue;
      const int c = (lane & 7) ^ f8swz(r);
      const uint32_t pi = static_cast<uint32_t>(key) / static_cast<uint32_t>(p.page_size);
      const int page = it.pids[pi - it.first_page];
      if (page < 0) continue;
      const int64_t tok = it.kn_start + key - it.cache_len;
      const char* ks = it.knb + tok * it.new_row_bytes + c * 32;
      const char* vs = it.vnb + tok * it.new_row_bytes + c * 32;
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(ks), k1 = *reinterpret_cast<const u32x4*>(ks + 16);
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(vs), v1 = *reinterpret_cast<const u32x4*>(vs + 16);
      u32x4 kc, vc;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        kc[e] = enc2(k0[2 * e], k_inv) | (enc2(k0[2 * e + 1], k_inv) << 16);
        kc[2 + e] = enc2(k1[2 * e], k_inv) | (enc2(k1[2 * e + 1], k_inv) << 16);
        vc[e] = enc2(v0[2 * e], v_inv) | (enc2(v0[2 * e + 1], v_inv) << 16);
        vc[2 + e] = enc2(v1[2 * e], v_inv) | (enc2(v1[2 * e + 1], v_inv) << 16);
      }
      // the LDS slot this lane's copy of row r filled
      *reinterpret_cast<u32x4*>(rk + i * 8 * F8ROW + lane * 16) = kc;
      *reinterpret_cast<u32x4*>(rv + i * 8 * F8ROW + lane * 16) = vc;
      const uint32_t slot = static_cast<uint32_t>(key) - pi * static_cast<uint32_t>(p.page_size);
      const int64_t off = (static_cast<int64_t>(page) * p.page_size + slot) * p.app.row_elems +
                          static_cast<int64_t>(it.kvh) * D + c * 16;
      *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.app.k_cache) + off) = kc;
      *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.app.v_cache) + off) = vc;
    }
    wait_lds();   // the rows' codes are in LDS before the block is read
  }
  __device__ static __forceinline__ bf16x8 widen8(uint32_t c0, uint32_t c1) {
    u32x4 w;
    uint32_t a, b, x, y;
    e4m3x4_to_bf16x4(c0, a, b);
    e4m3x4_to_bf16x4(c1, x, y);
    w[0] = a;
    w[1] = b;
    w[2] = x;
    w[3] = y;
    return __builtin_bit_cast(bf16x8, w);
  }
  // K operand of k-step s for code row r: head-dim values 16 s + 8 lg + (0..7)
  __device__ static __forceinline__ bf16x8 kread8(const uint8_t* rk, int r, int s, int lg) {
    const u32x2 v =
        *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
            static_cast<uintptr_t>(lds_addr(reinterpret_cast<const uint16_t*>(rk + r * F8ROW + ((s ^ f8swz(r)) << 4) + lg * 8))));
    return widen8(v[0], v[1]);
  }
  // V^T operand of key step j and output block d: keys 16 j + 4 lg + e and
  // 16 j + 8 + 4 lg + e (e = 0..3) of head-dim value 32 d + lr, the key order
  // of the P^T operand.  A 16-lane group addresses 8 code rows (lanes 2q and
  // 2q + 1 the two halves of row q's 16-byte chunk); ds_read_b64_tr_b8 then
  // gives lane i byte i of each of the 8 rows, in row order.
  __device__ static __forceinline__ bf16x8 vread8(const uint8_t* rv, int j, int d, int lr, int lg) {
    const int i = lr & 15;
    const int q = i >> 1;
    const int row = 16 * j + 4 * lg + (q & 3) + 8 * (q >> 2);
    const int chunk = 2 * d + (lr >> 4);
    const uint8_t* a = rv + row * F8ROW + ((chunk ^ f8swz(row)) << 4) + 8 * (i & 1);
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        reinterpret_cast<lds_i32x2*>(static_cast<uintptr_t>(lds_addr(reinterpret_cast<const uint16_t*>(a)))));
    return widen8(static_cast<uint32_t>(x[0]), static_cast<uint32_t>(x[1]));
  }
  // a3..a6 over the 32 keys held in code rows [hrow0, hrow0 + 32) of the
  // regions rk / rv (keys kbase ..), as compute<1, MASK> does for bf16 tiles
  template <bool MASK>
  __device__ static __forceinline__ void compute8(const uint8_t* rk, const uint8_t* rv, int hrow0,
                                                  const bf16x8 (&qf)[C::KSTEPS], f32x16 (&o)[C::DBLK],
                                                  float& m_run, float& l_run, int kbase, int lim, float c, int lr,
                                                  int lg) {
    constexpr int KH = C::KSTEPS / 2;
    f32x16 acc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = 0.f;
    bf16x8 kf[2][KH];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s) kf[rnd][s] = kread8(rk, hrow0 + lr, rnd * KH + s, lg);
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[rnd][s], qf[rnd * KH + s], acc[0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* const rvh = rv + hrow0 * F8ROW;
    bf16x8 vf[2][C::DBLK];
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d) vf[0][d] = vread8(rvh, 0, d, lr, lg);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pf[1][2];
    softmax<1, MASK>(acc, pf, o, m_run, l_run, kbase, lim, c, lg);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < C::DBLK; ++d) vf[1][d] = vread8(rvh, 1, d, lr, lg);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[jj][d], pf[0][jj], o[d], 0, 0, 0);
  }

  // ---- a3..a6 for this wave's 32 query rows over keys [kbase, kbase + 32 NH)
  //      held in tile rows [trow0, trow0 + 32 NH).  MASK: some key of the block
  //      lies beyond `lim` (the item's end, or the causal bound of the row).
  //      Operand fragments are read from LDS one round ahead of the MFMAs that
  //      use them (two rounds per phase), so each read's latency hides behind
  //      MFMA or softmax work while the live registers stay within budget.
  template <int NH, bool MASK>
  __device__ static __forceinline__ void compute(const uint16_t* ktile, const uint16_t* vtile,
                                                 int trow0, const bf16x8 (&qf)[C::KSTEPS],
                                                 f32x16 (&o)[C::DBLK], float& m_run, float& l_run,
                                                 int kbase, int lim, float c, int lr, int lg) {
    constexpr int KH = C::KSTEPS / 2;                    // k-steps per K round
    // a3: S^T = K Q^T, NH independent 32-key accumulators interleaved
    f32x16 acc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
    bf16x8 kf[2][NH][KH];
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h) kf[rnd][h][s] = kread(ktile, trow0 + h * 32 + lr, rnd * KH + s, lg);
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd)
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[rnd][h][s], qf[rnd * KH + s], acc[h], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // first V round, read while the softmax runs
    constexpr int JH = NH;                               // key steps per V round
    bf16x8 vf[2][JH][C::DBLK];
#pragma unroll
    for (int j = 0; j < JH; ++j)
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d) vf[0][j][d] = vread(vtile, trow0, j, d, lr, lg);
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 pf[NH][2];
    softmax<NH, MASK>(acc, pf, o, m_run, l_run, kbase, lim, c, lg);
    __builtin_amdgcn_sched_barrier(0);

    // a6: O^T += V^T P^T, second V round read ahead of the first round's MFMAs
#pragma unroll
    for (int j = 0; j < JH; ++j)
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d) vf[1][j][d] = vread(vtile, trow0, JH + j, d, lr, lg);
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
};

// ------------------------------------------------------------------ decode mode
// The score factor (scale * log2 e, times k_scale for fp8) and the output
// factor (v_scale for fp8): by value, or, when the call passes the fp8 scales
// in device memory, derived from them here the way the host derives them (a
// double product rounded once to float), so both give the same bits.
__device__ __forceinline__ void scales(const AttnParams& p, float& qk, float& vs) {
  qk = p.qk_scale_log2;
  vs = p.v_scale;
  if (p.kv_scale_dev) {
    qk = static_cast<float>(p.scale_log2e * static_cast<double>(p.kv_scale_dev[0]));
    vs = p.kv_scale_dev[1];
  }
}

// NWV: waves of the workgroup (4 in the decode-mode grid; 8 when a decode-mode
// item runs in the 512-thread workgroup of the mixed grid)
// DECAPP: the item forms and stores the new tokens its fp8 blocks hold
// (AttnParams::dec_append; head_dim 128, keys not turned)
template <int D, int FMT, bool PAGED, bool ROPE, int NWV = kWaves, bool DECAPP = false>
struct Decode : Src<D, FMT, PAGED> {
  using B = Src<D, FMT, PAGED>;
  using C = Cfg<D>;
  using Item = typename B::Item;
  static constexpr int kWaves = NWV;
  static constexpr int NT = kWaves * 64;
  static constexpr int DK = 32;                     // keys per wave block
  static constexpr int F8PASS = (DK * B::F8CH + 63) / 64;   // per lane, one wave moving 32 rows
  // the combine area is [4][32][D] fp32 outputs plus [4][32] maxima and
  // [4][32] sums: the two stages hold the outputs, this tail the rest
  static constexpr int kStages = kWaves / 2;        // each wave uses half a stage
  // Row stride (fp32) of the combine area: padded by 16 bytes, so that a
  // wave's 32 rows written at one head-dim offset fall into different banks
  // (with a stride of D floats they all hit the same ones)
  static constexpr int kCombStride = D + 4;
  // the combine area, [waves][32][kCombStride] fp32 outputs plus [waves][32]
  // maxima and sums, over the stages and past them: its size past the stages
  // (bf16 elements)
  static constexpr int kCombineExtra =
      (kWaves * kWaveRows * (kCombStride + 2) * 4 - kStages * C::STAGE * 2) / 2;
  static_assert(kCombineExtra > 0, "combine area extends past the stages");

  // Items with at most 32 packed rows (decode steps: q_len * g rows) would
  // leave three of four waves without rows, so the waves split the keys
  // instead: wave w takes the 32-key blocks w, w + 4, ... of the item, staged
  // in its own half of an LDS stage (no workgroup barrier in the loop), and
  // keeps its own running max / sum / output; the four partial states are
  // merged through LDS at the end.
  __device__ static __forceinline__ void item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq, const Item& it,
                              uint16_t* smem, float c, float v_scale, int wave, int lr, int lg, int t) {
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int nb = it.kend > kbeg ? (it.kend - kbeg + DK - 1) / DK : 0;
    const int part = __builtin_amdgcn_readfirstlane(item.part);
    const int q_start = __builtin_amdgcn_readfirstlane(sq.q_start);
    const int row0 = __builtin_amdgcn_readfirstlane(item.row0);
    uint16_t* const ktile = smem + (wave >> 1) * C::STAGE;
    uint16_t* const vtile = ktile + C::TILE;
    const int trow0 = (wave & 1) * DK;

    const bool row_ok = lr < item.nrows;
    bf16x8 qf[C::KSTEPS];
    int token, qh;
    B::load_q(p, sq, it.kvh, item.row0 + lr, row_ok, lg, qf, token, qh);
    if constexpr (ROPE) {
      // angles loaded beside Q, applied once both have arrived
      typename B::QAngles qa;
      if (row_ok) B::rope_load(p.rope, sq.kv_len - sq.q_len + token, lg, qa);
      if (row_ok) B::rope_apply(p.rope, lg, qa, qf);
    }
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
        typename B::template F8Regs<F8PASS> fk, fv;
        B::template f8_load<F8PASS, false>(p, it, fk, kbase - trow0, trow0, DK, lane, 64);
        B::template f8_load<F8PASS, true>(p, it, fv, kbase - trow0, trow0, DK, lane, 64);
        B::template f8_store<F8PASS>(fk, ktile, trow0, DK, lane, 64);
        B::template f8_store<F8PASS>(fv, vtile, trow0, DK, lane, 64);
        wait_lds();
      } else {
        const char *k0, *v0, *k1, *v1;
        uint32_t st0, st1;
        if (B::rows_contig(p, it, kbase, DK / 2, k0, v0, st0) &&
            B::rows_contig(p, it, kbase + DK / 2, DK / 2, k1, v1, st1)) {
          B::dma_rows(k0, st0, ktile, trow0, DK / 2, lane);
          B::dma_rows(k1, st1, ktile, trow0 + DK / 2, DK / 2, lane);
          B::dma_rows(v0, st0, vtile, trow0, DK / 2, lane);
          B::dma_rows(v1, st1, vtile, trow0 + DK / 2, DK / 2, lane);
        } else if (kbase + DK <= it.kend) {
          B::template dma_tile<false, false>(p, it, ktile, kbase - trow0, trow0, DK, lane);
          B::template dma_tile<false, true>(p, it, vtile, kbase - trow0, trow0, DK, lane);
        } else {
          B::template dma_tile<true, false>(p, it, ktile, kbase - trow0, trow0, DK, lane);
          B::template dma_tile<true, true>(p, it, vtile, kbase - trow0, trow0, DK, lane);
        }
        wait_vmem();
      }
      B::template compute<1, MASK>(ktile, vtile, trow0, qf, o, m_run, l_run, kbase, lim, c, lr, lg);
    };
    // this wave's blocks j = wave, wave + 4, ...: unmasked while at or below
    // the item's smallest key bound
    const int nb_full = min(nb, max(0, (tile_lim - kbeg + 1) / DK));
    if constexpr (FMT == kKvFp8 && D == 128) {
      // fp8 codes staged raw: wave w takes the 64-key blocks w, w + 4, ...
      // (two 32-key halves each) in its own region
      uint8_t* const rk = reinterpret_cast<uint8_t*>(ktile + trow0 * D);
      uint8_t* const rv = reinterpret_cast<uint8_t*>(vtile + trow0 * D);
      const int nb64 = (nb + 1) / 2;
      for (int jb = wave; jb < nb64; jb += kWaves) {
        const int kbase = kbeg + jb * 2 * DK;
        wait_lds();   // this wave's reads of its previous block are complete
        B::template dma_raw8<false>(p, it, rk, kbase, lane);
        B::template dma_raw8<true>(p, it, rv, kbase, lane);
        wait_vmem();
        if constexpr (DECAPP && !ROPE) B::dec_new8(p, it, rk, rv, kbase, lane);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int j32 = 2 * jb + hh;
          if (j32 < nb_full)
            B::template compute8<false>(rk, rv, hh * DK, qf, o, m_run, l_run, kbase + hh * DK, lim, c, lr, lg);
          else if (j32 < nb)
            B::template compute8<true>(rk, rv, hh * DK, qf, o, m_run, l_run, kbase + hh * DK, lim, c, lr, lg);
        }
      }
    } else {
      int j = wave;
      for (; j < nb_full; j += kWaves) step(j, std::false_type{});
      for (; j < nb; j += kWaves) step(j, std::true_type{});
    }

    // ---- combine the four waves' states through LDS
    __syncthreads();                     // every wave is done with its stage
    float* const so = reinterpret_cast<float*>(smem);              // [waves][32][D]
    float* const sm = so + kWaves * kWaveRows * kCombStride;       // [waves][32]
    float* const sl = sm + kWaves * kWaveRows;                     // [waves][32]
    const float l_tot = wave_pair_sum(l_run);
    if (row_ok) {
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = d * 32 + i4 * 8 + lg * 4;
          *reinterpret_cast<float4*>(so + (wave * kWaveRows + lr) * kCombStride + d0) =
              make_float4(o[d][i4 * 4 + 0], o[d][i4 * 4 + 1], o[d][i4 * 4 + 2], o[d][i4 * 4 + 3]);
        }
      if (lg == 0) {
        sm[wave * kWaveRows + lr] = m_run;
        sl[wave * kWaveRows + lr] = l_tot;
      }
    }
    __syncthreads();
    const int per_row = D / 4;
    for (int idx = t; idx < item.nrows * per_row; idx += NT) {
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
          const float4 f = *reinterpret_cast<const float4*>(so + (w * kWaveRows + r) * kCombStride + d0);
          lsum += wt * sl[w * kWaveRows + r];
          acc4.x += wt * f.x;
          acc4.y += wt * f.y;
          acc4.z += wt * f.z;
          acc4.w += wt * f.w;
        }
      }
      const bool live = lsum > 0.f;
      const float inv = live ? v_scale / lsum : 0.f;
      const float lse_v = live ? mmax * c * kLn2 + __logf(lsum) : -INFINITY;
      const int pr = row0 + r;
      const int tok = pr / p.g;
      const int h = it.kvh * p.g + (pr - tok * p.g);
      B::store4(p, part, q_start, r, tok, h, d0, acc4.x * inv, acc4.y * inv, acc4.z * inv, acc4.w * inv,
                lse_v, d0 == 0);
    }
  }

  __device__ static __forceinline__ void run(const AttnParams& p) {
    // two K/V stages used as four per-wave half stages, then as the area
    // where the waves combine their partial softmax states
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kStages * C::STAGE + kCombineExtra];
    __shared__ int32_t pids[PAGED ? kMaxItemPages : 1];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;   // query column of this lane
    const int lg = lane >> 5;   // lane half
    // workgroups past the attention part of the grid store new tokens
    if (static_cast<int>(blockIdx.x) >= p.attn_blocks) {
      append_tokens(p.app, blockIdx.x - p.attn_blocks, t, NT, reinterpret_cast<int64_t*>(smem));
      return;
    }
    float qk, vs;
    scales(p, qk, vs);
    __shared__ typename B::QEntry qbuf[B::kQueueChunk];
    B::for_each_item(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      item(p, e.item, e.item.s, it, smem, qk, vs, wave, lr, lg, t);
    });
  }
};

// ----------------------------------------------------------------- prefill mode
template <int D, int FMT, bool PAGED, bool ROPE>
struct Prefill : Src<D, FMT, PAGED> {
  using B = Src<D, FMT, PAGED>;
  using C = Cfg<D>;
  using Item = typename B::Item;
  static constexpr int NW = kPrefillWaves;
  static constexpr int NT = NW * 64;
  static constexpr int NS = 4;                        // ring stages (K and V of one block each)
  static constexpr int WROWS = kBlockN / NW;          // tile rows each wave stages
  static constexpr int DMA_PER_TILE = WROWS / B::RPI; // bf16 copies per wave and tile
  static_assert(WROWS % B::RPI == 0, "whole DMA rows per wave");
  static_assert(2 * DMA_PER_TILE <= 4, "in-flight copies of one block fit wait_vmem_upto");
  static constexpr int KSTEPS = C::KSTEPS;
  static constexpr int DBLK = C::DBLK;
  static constexpr int F8PASS = (kBlockN * B::F8CH + NT - 1) / NT;

  __device__ static __forceinline__ void item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq, const Item& it,
                              uint16_t* smem, int* lims, float c, float v_scale, int wave, int lr, int lg, int t) {
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int nblk = it.kend > kbeg ? (it.kend - kbeg + kBlockN - 1) / kBlockN : 0;
    const int part = __builtin_amdgcn_readfirstlane(item.part);
    const int q_start = __builtin_amdgcn_readfirstlane(sq.q_start);

    // ---- staging of block j into stage j mod NS: this wave's WROWS rows of K
    //      and V (bf16), or the block through registers (fp8)
    // fp8 cache, head_dim 128: three bf16 stages and two raw-code areas in
    // the same LDS (below); otherwise four bf16 stages
    constexpr bool RAW8 = FMT == kKvFp8 && D == 128;
    auto stage_of = [&](int j) {
      if constexpr (RAW8) return smem + (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(j)) % 3u) * C::STAGE;
      else return smem + (j & (NS - 1)) * C::STAGE;
    };
    auto stage_dma = [&](int j) {
      const int kbase = kbeg + j * kBlockN;
      uint16_t* const kt = stage_of(j);
      const char *k0, *v0;
      uint32_t stride;
      if (B::rows_contig(p, it, kbase + wave * WROWS, WROWS, k0, v0, stride)) {
        B::dma_rows(k0, stride, kt, wave * WROWS, WROWS, lane);
        B::dma_rows(v0, stride, kt + C::TILE, wave * WROWS, WROWS, lane);
      } else if (kbase + kBlockN <= it.kend) {
        B::template dma_tile<false, false, true>(p, it, kt, kbase, wave * WROWS, WROWS, lane);
        B::template dma_tile<false, true, true>(p, it, kt + C::TILE, kbase, wave * WROWS, WROWS, lane);
      } else {
        B::template dma_tile<true, false, true>(p, it, kt, kbase, wave * WROWS, WROWS, lane);
        B::template dma_tile<true, true, true>(p, it, kt + C::TILE, kbase, wave * WROWS, WROWS, lane);
      }
    };
    using F8 = typename B::template F8Regs<F8PASS>;
    F8 fk, fv;
    auto f8_load = [&](int j) {
      B::template f8_load<F8PASS, false>(p, it, fk, kbeg + j * kBlockN, 0, kBlockN, t, NT);
      B::template f8_load<F8PASS, true>(p, it, fv, kbeg + j * kBlockN, 0, kBlockN, t, NT);
    };
    auto f8_store = [&](int j) {
      B::template f8_store<F8PASS>(fk, stage_of(j), 0, kBlockN, t, NT);
      B::template f8_store<F8PASS>(fv, stage_of(j) + C::TILE, 0, kBlockN, t, NT);
    };
    // RAW8: block j's codes (64 rows of 128 bytes of K, then of V) go by DMA
    // into raw area j mod 2, each wave its own 8 rows (one copy per tile);
    // the same wave later widens those rows into bf16 stage j mod 3.  Lane l
    // moves chunk l mod 8 (16 codes) of row 8 wave + l / 8 both times, so it
    // reads back only what its own copy wrote.
    uint8_t* const raw0 = reinterpret_cast<uint8_t*>(smem + 3 * C::STAGE);
    auto raw_of = [&](int j) { return raw0 + (j & 1) * (2 * kBlockN * D); };
    auto raw_dma = [&](int j) {
      const int r = wave * 8 + (lane >> 3);
      const char *kp, *vp;
      const bool ok = B::template row_src<true>(p, it, kbeg + j * kBlockN + r, kp, vp);
      const char* zeros = static_cast<const char*>(p.zeros);
      const int off = (lane & 7) * 16;
      uint8_t* const a = raw_of(j) + wave * 8 * D;
      dma16<true>(ok ? kp + off : zeros, reinterpret_cast<uint16_t*>(a));
      dma16<true>(ok ? vp + off : zeros, reinterpret_cast<uint16_t*>(a + kBlockN * D));
    };
    auto raw_convert = [&](int j) {
      const int r = wave * 8 + (lane >> 3);
      const int cc = lane & 7;
      const uint8_t* const a = raw_of(j) + r * D + cc * 16;
      uint16_t* const st = stage_of(j);
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const u32x4 codes = *reinterpret_cast<const u32x4*>(a + kv * kBlockN * D);
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) e4m3x4_to_bf16x4(codes[e], w[2 * e], w[2 * e + 1]);
        uint16_t* const tile = st + kv * C::TILE;
        *reinterpret_cast<u32x4*>(tile + C::at(r, 2 * cc)) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(tile + C::at(r, 2 * cc + 1)) = u32x4{w[4], w[5], w[6], w[7]};
      }
    };

    // Q rows first: their loads are older than the staging copies, so the
    // copy waits below also cover them
    const int wrow = wave * kWaveRows + lr;
    const bool row_ok = wrow < item.nrows;
    bf16x8 qf[KSTEPS];
    int token, qh;
    B::load_q(p, sq, it.kvh, item.row0 + wrow, row_ok, lg, qf, token, qh);
    // rotary embedding: the angles are loaded now, beside Q and before the
    // first staging copies, and applied after the prologue's wait for them
    typename B::QAngles qa;
    if constexpr (ROPE) {
      if (row_ok) B::rope_load(p.rope, sq.kv_len - sq.q_len + token, lg, qa);
    }

    // per-row and per-wave key bounds
    const int shift = sq.kv_len - sq.q_len;
    {
      // the row's last visible key, kept in LDS: only blocks that cross a
      // row bound read it, and a register held across the loop for it
      // would be spilled
      int lim = it.kend - 1;
      if (p.causal) lim = min(lim, token + shift);
      lims[t] = lim - lg * 4;   // the softmax adds the lane half's offset back
    }
    const int wr0 = wave * kWaveRows;
    const int wr1 = min(item.nrows, wr0 + kWaveRows) - 1;          // last valid row of the wave
    int wlo = it.kend - 1, whi = it.kend - 1;
    if (p.causal) {
      wlo = min(wlo, (item.row0 + wr0) / p.g + shift);
      whi = min(whi, (item.row0 + wr1) / p.g + shift);
    }
    // this wave computes blocks [0, nb_w); blocks below n_full need no mask
    const int nb_w = (wr1 < wr0 || whi < kbeg) ? 0 : min(nblk, (whi - kbeg) / kBlockN + 1);
    const int n_full = min(nb_w, max(0, (wlo - kbeg + 1) / kBlockN));

    f32x16 o[DBLK];
    float m_run, l_run;
    auto init_state = [&] {
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
      m_run = -INFINITY;
      // opaque start value: otherwise the compiler folds the first block's
      // threshold m c + 8 into a constant that it keeps live (and spills)
      // across the whole loop
      asm volatile("" : "+v"(m_run));
      l_run = 0.f;
    };
    // (with rotary embedding the running state is set after the prologue,
    // where the angles are no longer live)
    if constexpr (!ROPE) init_state();
    f32x16 acc[2];
    bf16x8 pf[2][2];

    // ---- prologue: blocks 0..2 staged, 0 and 1 complete before the first
    //      barrier (fp8: all three stored)
    if constexpr (RAW8) {
      // blocks 0 and 1 copied and widened; block 2 copied into the raw area
      // block 0 has left
      if (nblk > 0) raw_dma(0);
      if (nblk > 1) raw_dma(1);
      wait_vmem();
      // Q is complete too: said here, before block 2's copy is issued, so
      // that the compiler's own wait for Q does not cover that copy
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) asm volatile("" : : "v"(qf[s]));
      if (nblk > 0) raw_convert(0);
      if (nblk > 1) raw_convert(1);
      if (nblk > 2) raw_dma(2);
    } else if constexpr (FMT == kKvFp8) {
      for (int j = 0; j < 3 && j < nblk; ++j) {
        f8_load(j);
        f8_store(j);
      }
    } else {
      for (int j = 0; j < 3 && j < nblk; ++j) stage_dma(j);
      wait_vmem_upto(nblk > 2 ? 2 * DMA_PER_TILE : 0);
    }
    if constexpr (ROPE) {
      if (row_ok) B::rope_apply(p.rope, lg, qa, qf);
      init_state();
    }
    // Q is complete here (its loads are older than the copies just waited
    // for); an empty use tells the compiler so, which keeps it from placing a
    // wait for all vector memory, in-flight copies included, inside the loop
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" : : "v"(qf[s]));
    if (nblk > 0) __syncthreads();

    // Two wave groups share each SIMD: group A (waves 0-3) and group B (waves
    // 4-7).  Both pass one barrier per block, at skewed points: after barrier
    // n, A computes block n (scores, softmax, P V); B finishes block n (P V)
    // and computes scores and softmax of block n + 1.  One wave of a SIMD
    // thus runs its softmax while the other issues MFMAs; MFMA phases run at
    // raised wave priority, so the pipe is fed first whenever the MFMA wave
    // is ready and the softmax takes the remaining issue slots.  Between barriers n
    // and n + 1 the stages of blocks n and n + 1 are read, and block n + 3 is
    // staged into the stage block n - 1 left (four stages); it must be
    // complete at barrier n + 2.
    const bool group_b = wave >= NW / 2;
    auto sm = [&](int n, auto mask_tag) {
      B::template softmax<2, decltype(mask_tag)::value>(acc, pf, o, m_run, l_run, kbeg + n * kBlockN,
                                                         decltype(mask_tag)::value ? lims[t] + lg * 4 : 0, c,
                                                         lg);
    };
    // interval after barrier n: the caller's first part (nothing for group
    // A, the MFMA phase for group B), then start staging block n + 3 (the
    // copies of all eight waves are then not issued at the same moment), the
    // rest of the work, then wait for block n + 2 (bf16) or store block n + 3
    // (fp8)
    auto interval = [&](int n, auto&& first, auto&& rest) {
      if constexpr (RAW8) {
        // copy block n + 3 (into the raw area block n + 1 has left), then
        // widen block n + 2 into the stage block n - 1 has left
        first();
        int issued = 0;
        if (n + 3 < nblk) {
          raw_dma(n + 3);
          issued = 2;
        }
        rest();
        if (n + 2 < nblk) {
          wait_vmem_upto(issued);
          raw_convert(n + 2);
        }
        return;
      }
      first();
      int issued = 0;
      if constexpr (FMT == kKvFp8) {
        if (n + 3 < nblk) f8_load(n + 3);
      } else {
        if (n + 3 < nblk) {
          stage_dma(n + 3);
          issued = 2 * DMA_PER_TILE;
        }
      }
      rest();
      if constexpr (FMT == kKvFp8) {
        if (n + 3 < nblk) f8_store(n + 3);
      } else {
        wait_vmem_upto(issued);
      }
    };

    // (an item without keys skips both: its rows get out = 0, lse = -inf)
    if (nblk > 0 && !group_b) {
      // Group A runs the softmax of block n first and then one MFMA phase
      // (P V of block n, scores of block n + 1), group B the reverse: each
      // SIMD then always pairs one wave in its MFMA phase with one in its
      // softmax, and no part of the interval has both waves issuing MFMAs
      // while the vector ALU idles.  A's copies are issued at the start of
      // the interval, B's after its MFMA phase (not between its P V and its
      // scores, which split that phase and stretched A's).
      if (nb_w > 0) B::template qk0<2>(stage_of(0), qf, acc, lr, lg);   // scores of block 0
      auto body = [&](int n, auto mode_tag) {
        constexpr int MODE = decltype(mode_tag)::value;   // of block n: 0 unmasked, 1 masked, 2 none
        __syncthreads();                                    // barrier n
        interval(
            n, [] {},
            [&] {
              if constexpr (MODE != 2) {
                __builtin_amdgcn_s_setprio(0);
                sm(n, std::bool_constant<MODE == 1>{});
                __builtin_amdgcn_s_setprio(1);
                B::template pv0<2>(stage_of(n) + C::TILE, pf, o, lr, lg);
                if (n + 1 < nb_w) B::template qk0<2>(stage_of(n + 1), qf, acc, lr, lg);
              }
            });
      };
      int n = 0;
      for (; n < n_full; ++n) body(n, std::integral_constant<int, 0>{});
      for (; n < nb_w; ++n) body(n, std::integral_constant<int, 1>{});
      for (; n < nblk; ++n) body(n, std::integral_constant<int, 2>{});
    } else if (nblk > 0) {
      // scores and softmax of block 0 before barrier 0
      if (nb_w > 0) {
        B::template qk0<2>(stage_of(0), qf, acc, lr, lg);
        if (n_full > 0) sm(0, std::false_type{});
        else sm(0, std::true_type{});
      }
      auto body = [&](int n, auto mode_tag) {
        constexpr int MODE = decltype(mode_tag)::value;   // of block n + 1: 0 unmasked, 1 masked, 2 none
        __syncthreads();                                    // barrier n
        interval(
            n,
            [&] {
              // one MFMA phase, then the copies, then the softmax
              __builtin_amdgcn_s_setprio(1);
              if (n < nb_w) B::template pv0<2>(stage_of(n) + C::TILE, pf, o, lr, lg);
              if constexpr (MODE != 2) B::template qk0<2>(stage_of(n + 1), qf, acc, lr, lg);
            },
            [&] {
              if constexpr (MODE != 2) {
                __builtin_amdgcn_s_setprio(0);
                sm(n + 1, std::bool_constant<MODE == 1>{});
              }
            });
      };
      int n = 0;
      for (; n + 1 < n_full; ++n) body(n, std::integral_constant<int, 0>{});
      for (; n + 1 < nb_w; ++n) body(n, std::integral_constant<int, 1>{});
      for (; n < nblk; ++n) body(n, std::integral_constant<int, 2>{});
    }

    if (wr1 >= wr0) {
      const float l_tot = wave_pair_sum(l_run);
      const bool live = l_tot > 0.f;
      const float inv = live ? v_scale / l_tot : 0.f;
      const float lse_v = live ? m_run * c * kLn2 + __logf(l_tot) : -INFINITY;
      if (part < 0) {
        // the two lanes of a row exchange values, so every lane of the wave
        // runs the swaps; rows past the item's end store nothing
#pragma unroll
        for (int d = 0; d < DBLK; ++d) B::store_out_block(p, q_start, token, qh, d, o[d], inv, lg, row_ok);
        if (row_ok && lg == 0 && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + q_start + token] = lse_v;
      } else if (row_ok) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            B::store4(p, part, q_start, wrow, token, qh, d * 32 + i4 * 8 + lg * 4, o[d][i4 * 4 + 0] * inv,
                      o[d][i4 * 4 + 1] * inv, o[d][i4 * 4 + 2] * inv, o[d][i4 * 4 + 3] * inv, lse_v,
                      lg == 0 && d == 0 && i4 == 0);
      }
    }
  }

  __device__ static __forceinline__ void run(const AttnParams& p) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * C::STAGE];
    __shared__ int32_t pids[PAGED ? kMaxItemPages : 1];
    __shared__ int lims[NT];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;
    const int lg = lane >> 5;
    // workgroups past the attention part of the grid store new tokens
    if (static_cast<int>(blockIdx.x) >= p.attn_blocks) {
      append_tokens(p.app, blockIdx.x - p.attn_blocks, t, NT, reinterpret_cast<int64_t*>(smem));
      return;
    }
    float qk, vs;
    scales(p, qk, vs);
    __shared__ typename B::QEntry qbuf[B::kQueueChunk];
    B::for_each_item(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      item(p, e.item, e.item.s, it, smem, lims, qk, vs, wave, lr, lg, t);
    });
  }
};

// ---------------------------------------------------------------- mixed grid
// One launch for a batch that mixes prefill-mode tiles and decode-mode
// splits: 512-thread workgroups (one per CU) whose items are either kind.  A
// prefill-mode item runs as in the prefill-mode grid; a decode-mode item runs
// on all eight waves, which split its keys.  The items are listed prefill-mode
// first (the longest work starts first), then decode-mode, so the decode
// splits fill the compute units the prefill tiles leave idle.  (The FlashInfer
// PoD-Attention page, "[Refactor] Uniform PoDAttention API with Horizontal
// Fusion SMs Schedule", Key Changes: prefill and decode requests share one
// persistent launch.)
template <int D, int FMT, bool PAGED, bool ROPE>
struct Mixed {
  using Pf = Prefill<D, FMT, PAGED, ROPE>;
  using Dc = Decode<D, FMT, PAGED, ROPE, kPrefillWaves>;
  using B = Src<D, FMT, PAGED>;
  using C = Cfg<D>;
  using Item = typename B::Item;
  static constexpr int NT = kPrefillWaves * 64;
  static constexpr int SMEM = Pf::NS * C::STAGE > Dc::kStages * C::STAGE + Dc::kCombineExtra
                                  ? Pf::NS * C::STAGE
                                  : Dc::kStages * C::STAGE + Dc::kCombineExtra;

  __device__ static __forceinline__ void run(const AttnParams& p) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];
    __shared__ int32_t pids[PAGED ? kMaxItemPages : 1];
    __shared__ int lims[NT];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;
    const int lg = lane >> 5;
    if (static_cast<int>(blockIdx.x) >= p.attn_blocks) {
      append_tokens(p.app, blockIdx.x - p.attn_blocks, t, NT, reinterpret_cast<int64_t*>(smem));
      return;
    }
    float qk, vs;
    scales(p, qk, vs);
    __shared__ typename B::QEntry qbuf[B::kQueueChunk];
    // two passes over the workgroup's entries, prefill-mode items first (each
    // queue lists them first anyway): with both item bodies inside one loop
    // the register allocator spilled 54-127 VGPRs; each pass alone spills none
    B::template for_each_item<0>(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      Pf::item(p, e.item, e.item.s, it, smem, lims, qk, vs, wave, lr, lg, t);
    });
    B::template for_each_item<1>(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      Dc::item(p, e.item, e.item.s, it, smem, qk, vs, wave, lr, lg, t);
    });
  }
};

// ---------------------------------------------------------------- fp8 QKV-Prob
// Attention with the query, key and value rows and the softmax output P all in
// fp8: the "QKV-Prob" models of the vLLM Triton FAv2 PR page ("[Kernel][Triton]
// [FP8] Adding fp8 and variable length sequence support to Triton FAv2
// kernel", feature list item 7, and the paragraph before its LM EVAL tables:
// softmax(QK^T) is quantised to fp8 before the second product).  Both
// products run on gfx950's v_mfma_f32_32x32x64_f8f6f4 with e4m3 operands:
// K and V stay raw cache codes in LDS (nothing is widened), and the query rows
// are quantised as they are loaded, by the cache's rule with q_scale.  P is
// the row's exact softmax: a first pass over the item's keys computes only
// the scores and each row's maximum m and sum l; a second pass recomputes the
// scores, rounds P / p_scale = 2^(s c - m c - log2 l - log2 p_scale) to e4m3
// with the hardware conversion (nearest, ties to even) and adds P V.  The
// output is O * p_scale * v_scale, not renormalised after the quantisation.
//
// MFMA operands (32 rows x 64 k values, 32 bytes per lane): both operands of
// the instruction map (lane half, byte) to k the same way, so any assignment
// of the 64 k values that both share gives the same sums.  Scores: lane half
// lg holds head-dim values 64 s + 32 lg + (0..31) at step s.  P V: byte
// 16 h + i of the P operand is element i of score accumulator h (key
// 32 h + 8 (i / 4) + 4 lg + i % 4), and four transposed LDS reads gather the
// V^T operand for the same keys.  Items are never split: the host plans this
// grid without key-range parts.  Prefill-mode items (more than 32 rows) run
// eight waves of 32 rows over shared 64-key tiles; decode-mode items (at most
// 32 rows) split their keys over the eight waves.
template <int D>
struct Prob8 : Src<D, kKvFp8, true> {
  using B = Src<D, kKvFp8, true>;
  using C = Cfg<D>;
  using Item = typename B::Item;
  static constexpr int NW = kPrefillWaves;
  static constexpr int NT = NW * 64;
  static constexpr int ROW = D;                   // bytes of a code row
  static constexpr int CPR = ROW / 16;            // 16-byte chunks of a row
  static constexpr int TILE = kBlockN * ROW;      // bytes of a 64-key tile
  static constexpr int STAGE = 2 * TILE;          // K tile, then V tile
  static constexpr int NS = 3;                    // ring stages
  static constexpr int KS = D / 64;               // MFMA steps over the head dim
  static constexpr int DBLK = D / 32;             // 32-wide output blocks
  static constexpr int RPW = 1024 / ROW;          // rows one wave copies with one instruction
  static constexpr int WPT = kBlockN / RPW;       // waves that copy one tile

  // Chunk c of code row r sits at c ^ sw(r).  Score reads (16 consecutive
  // rows, one chunk each) and the transposed V reads (rows {0..3, 8..11} +
  // 4 lg + 16 j, chunks c and c ^ 1 in the two lane groups of a half wave)
  // then touch distinct banks.
  __device__ static __forceinline__ int sw(int r) {
    if constexpr (D == 128) return (((r >> 1) & 1) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 2);
    else return (r >> 2) & 3;
  }

  // query row codes: head-dim values 64 s + 32 lg + (0..31) of this lane's row
  __device__ static __forceinline__ void load_q8(const AttnParams& p, const SeqInfo& sq, int kvh, int prow,
                                                 bool row_ok, int lg, i32x8 (&qf)[KS], int& token, int& qh) {
    using append_detail::enc2;
    token = prow / p.g;
    qh = kvh * p.g + (prow - token * p.g);
    const uint16_t* qrow = p.q + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D;
    u32x4 x[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * lg + 8 * t4);
        x[s][t4] = v;
      }
    const float inv = p.q_inv_scale;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        qf[s][2 * t4] = static_cast<int>(enc2(x[s][t4][0], inv) | (enc2(x[s][t4][1], inv) << 16));
        qf[s][2 * t4 + 1] = static_cast<int>(enc2(x[s][t4][2], inv) | (enc2(x[s][t4][3], inv) << 16));
      }
  }

  // copies of the tile rows of keys [kbase, kbase + 64) into stage `st`: K
  // (and V when WITH_V); rows past the item's end or on an unusable page
  // read zeros.  Returns the copies this wave issued.
  template <bool WITH_V>
  __device__ static __forceinline__ int stage(const AttnParams& p, const Item& it, uint8_t* st, int kbase,
                                              int wave, int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
    const int part = wave % WPT;
    const int r = part * RPW + lane / CPR;
    const int c = (lane % CPR) ^ sw(r);
    const char *kp, *vp;
    const bool ok = B::template row_src<true>(p, it, kbase + r, kp, vp);
    uint8_t* const dst = st + part * RPW * ROW;
    if constexpr (WPT == NW) {
      dma16<true>(ok ? kp + c * 16 : zeros, reinterpret_cast<uint16_t*>(dst));
      if constexpr (WITH_V) dma16<true>(ok ? vp + c * 16 : zeros, reinterpret_cast<uint16_t*>(dst + TILE));
      return WITH_V ? 2 : 1;
    } else {
      // half of the waves copy K, the other half V
      const bool is_v = wave >= WPT;
      if (is_v && !WITH_V) return 0;
      dma16<true>(ok ? (is_v ? vp : kp) + c * 16 : zeros, reinterpret_cast<uint16_t*>(dst + (is_v ? TILE : 0)));
      return 1;
    }
  }

  // S^T of this wave's 32 query rows against the tile's first 32 NH keys
  template <int NH>
  __device__ static __forceinline__ void qk(const uint8_t* kt, const i32x8 (&qf)[KS], f32x16 (&acc)[NH], int lr,
                                            int lg) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
    i32x8 kf[KS][NH];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int r = 32 * h + lr;
        const int c0 = 4 * s + 2 * lg;
        const u32x4 x0 = B::template lds_read<u32x4>(
            B::lds_addr(reinterpret_cast<const uint16_t*>(kt + r * ROW + ((c0 ^ sw(r)) << 4))));
        const u32x4 x1 = B::template lds_read<u32x4>(
            B::lds_addr(reinterpret_cast<const uint16_t*>(kt + r * ROW + (((c0 + 1) ^ sw(r)) << 4))));
        kf[s][h] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        acc[h] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[s][h], qf[s], acc[h], 0, 0, 0, 0, 0, 0);
  }

  // first pass: running row maximum and sum; `rel` is the last visible key
  // relative to this lane's first key of the block (MASK)
  template <int NH, bool MASK>
  __device__ static __forceinline__ void stats(f32x16 (&acc)[NH], float& m_run, float& l_run, int rel, float c) {
    if constexpr (MASK) {
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
    const float m_new = fmaxf(m_run, mx);
    const float neg = m_new == -INFINITY ? 0.f : -m_new * c;
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[h][i], c, neg));
    // (m_run = -inf: the old sum is 0 and exp2(-inf) = 0)
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
    l_run = l_run * alpha + s;
    m_run = m_new;
  }

  // second pass: the P operand, e4m3 codes of 2^(s c + neg2) = P / p_scale
  // (bytes of keys past the block's 32 NH are zero)
  template <int NH, bool MASK>
  __device__ static __forceinline__ i32x8 probs(const f32x16 (&acc)[NH], int rel, float c, float neg2) {
    i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          y[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[h][i], c, neg2));
          if (MASK && h * 32 + q4 * 8 + e > rel) y[e] = 0.f;
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
        pb[4 * h + q4] = w;
      }
    return pb;
  }

  // V^T operand of output block d: bytes 8 j + (0..7) hold keys 16 j + 4 lg +
  // (0..3) and 16 j + 8 + 4 lg + (0..3) of head-dim value 32 d + lr, the key
  // order of the P operand.  A 16-lane group addresses 8 code rows (lanes 2q
  // and 2q + 1 the two halves of row q's chunk); ds_read_b64_tr_b8 gives lane
  // i byte i of each of the 8 rows, in row order.  Keys past the tile's
  // 32 NH rows read as zero.
  template <int NH>
  __device__ static __forceinline__ i32x8 vread(const uint8_t* vt, int d, int lr, int lg) {
    const int i = lr & 15;
    const int q = i >> 1;
    const int chunk = 2 * d + (lr >> 4);
    i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 2 * NH; ++j) {
      const int row = 16 * j + 4 * lg + (q & 3) + 8 * (q >> 2);
      const uint8_t* a = vt + row * ROW + ((chunk ^ sw(row)) << 4) + 8 * (i & 1);
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2*>(
          static_cast<uintptr_t>(B::lds_addr(reinterpret_cast<const uint16_t*>(a)))));
      v[2 * j] = x[0];
      v[2 * j + 1] = x[1];
    }
    return v;
  }

  __device__ static __forceinline__ void item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq,
                                              const Item& it, uint8_t* ring, int* lims, float c, float out_scale,
                                              int wave, int lr, int lg, int t) {
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int nblk = it.kend > kbeg ? (it.kend - kbeg + kBlockN - 1) / kBlockN : 0;
    const int q_start = __builtin_amdgcn_readfirstlane(sq.q_start);
    const int wrow = wave * kWaveRows + lr;
    const bool row_ok = wrow < item.nrows;
    i32x8 qf[KS];
    int token, qh;
    load_q8(p, sq, it.kvh, item.row0 + wrow, row_ok, lg, qf, token, qh);

    // per-row and per-wave key bounds (as in the prefill-mode kernel)
    const int shift = sq.kv_len - sq.q_len;
    {
      int lim = it.kend - 1;
      if (p.causal) lim = min(lim, token + shift);
      lims[t] = lim - lg * 4;
    }
    const int wr0 = wave * kWaveRows;
    const int wr1 = min(item.nrows, wr0 + kWaveRows) - 1;
    int wlo = it.kend - 1, whi = it.kend - 1;
    if (p.causal) {
      wlo = min(wlo, (item.row0 + wr0) / p.g + shift);
      whi = min(whi, (item.row0 + wr1) / p.g + shift);
    }
    const int nb_w = (wr1 < wr0 || whi < kbeg) ? 0 : min(nblk, (whi - kbeg) / kBlockN + 1);
    const int n_full = min(nb_w, max(0, (wlo - kbeg + 1) / kBlockN));

    // one pass over the item's blocks: block n + 2 is copied while block n
    // is computed (three stages; barrier n frees the stage of block n - 1)
    auto stage_of = [&](int j) {
      return ring + (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(j)) % 3u) * STAGE;
    };
    auto pass = [&](auto v_tag, auto&& body) {
      constexpr bool WITH_V = decltype(v_tag)::value;
      int cpb = 0;
      if (nblk > 0) cpb = stage<WITH_V>(p, it, stage_of(0), kbeg, wave, lane);
      if (nblk > 1) stage<WITH_V>(p, it, stage_of(1), kbeg + kBlockN, wave, lane);
      for (int n = 0; n < nblk; ++n) {
        wait_vmem_upto(n + 1 < nblk ? cpb : 0);
        __syncthreads();
        if (n + 2 < nblk) stage<WITH_V>(p, it, stage_of(n + 2), kbeg + (n + 2) * kBlockN, wave, lane);
        if (n < nb_w) body(n, stage_of(n));
      }
      __syncthreads();   // every wave is done with the ring
    };

    // First pass: K tiles of BK1 = 128 keys (half as many barriers as 64-key
    // blocks; the pass computes little per key and no output is live yet),
    // three stages, each wave copying 16 rows of every tile.
    constexpr int BK1 = 2 * kBlockN;
    constexpr int TILE1 = BK1 * ROW;
    constexpr int CP1 = (BK1 / NW) / RPW;                 // copies per wave and tile
    static_assert(3 * TILE1 <= kRingBytes, "first-pass ring fits");
    const int nblk1 = it.kend > kbeg ? (it.kend - kbeg + BK1 - 1) / BK1 : 0;
    const int nb_w1 = (wr1 < wr0 || whi < kbeg) ? 0 : min(nblk1, (whi - kbeg) / BK1 + 1);
    const int n_full1 = min(nb_w1, max(0, (wlo - kbeg + 1) / BK1));
    auto st1_of = [&](int j) {
      return ring + (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(j)) % 3u) * TILE1;
    };
    auto stage1 = [&](int j) {
      const char* zeros = static_cast<const char*>(p.zeros);
      const int kbase = kbeg + j * BK1;
      uint8_t* const st = st1_of(j);
#pragma unroll
      for (int i = 0; i < CP1; ++i) {
        const int r0 = (wave * CP1 + i) * RPW;             // first row of this copy
        const int r = r0 + lane / CPR;
        const int cc = (lane % CPR) ^ sw(r);
        const char *kp, *vp;
        const bool ok = B::template row_src<true>(p, it, kbase + r, kp, vp);
        dma16<true>(ok ? kp + cc * 16 : zeros, reinterpret_cast<uint16_t*>(st + r0 * ROW));
      }
    };
    float m_run = -INFINITY, l_run = 0.f;
    if (nblk1 > 0) stage1(0);
    if (nblk1 > 1) stage1(1);
    for (int n = 0; n < nblk1; ++n) {
      wait_vmem_upto(n + 1 < nblk1 ? CP1 : 0);
      __syncthreads();
      if (n + 2 < nblk1) stage1(n + 2);
      if (n < nb_w1) {
        f32x16 acc[4];
        qk<4>(st1_of(n), qf, acc, lr, lg);
        if (n < n_full1) stats<4, false>(acc, m_run, l_run, 0, c);
        else stats<4, true>(acc, m_run, l_run, lims[t] - (kbeg + n * BK1), c);
      }
    }
    __syncthreads();   // every wave is done with the ring
    const float l_tot = wave_pair_sum(l_run);
    const bool live = l_tot > 0.f;
    const float neg2 = live ? -(m_run * c + __log2f(l_tot) + p.p_log2) : 0.f;

    f32x16 o[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    pass(std::true_type{}, [&](int n, const uint8_t* st) {
      f32x16 acc[2];
      qk<2>(st, qf, acc, lr, lg);
      const i32x8 pb = n < n_full ? probs<2, false>(acc, 0, c, neg2)
                                  : probs<2, true>(acc, lims[t] - (kbeg + n * kBlockN), c, neg2);
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
        o[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vread<2>(st + TILE, d, lr, lg), pb, o[d], 0, 0, 0,
                                                               0, 0, 0);
    });

    if (wr1 >= wr0) {
      const float inv = live ? out_scale : 0.f;
      const float lse_v = live ? m_run * c * kLn2 + __logf(l_tot) : -INFINITY;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) B::store_out_block(p, q_start, token, qh, d, o[d], inv, lg, row_ok);
      if (row_ok && lg == 0 && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + q_start + token] = lse_v;
    }
  }

  // ---- decode-mode items (at most 32 packed rows): the eight waves split the
  //      item's 32-key blocks (wave w takes blocks w, w + 8, ...), each with
  //      its own two-stage ring of K and V tiles, and no barrier inside the
  //      loops.  The waves' row maxima and sums (first pass) and their
  //      partial outputs (second pass) are combined through LDS in a fixed
  //      order, so the result does not depend on timing.
  static constexpr int DK = 32;                          // keys per decode-mode block
  static constexpr int DTILE = DK * ROW;                 // bytes of a K (or V) tile
  static constexpr int DSTAGE = 2 * DTILE;
  static constexpr int DCOPIES = DTILE / 1024;           // copies per tile and wave
  static constexpr int kDecBytes = NW * 2 * DSTAGE;      // the eight waves' rings
  static constexpr int kCombStride = D + 4;              // fp32 row stride of the output combine
  static constexpr int kCombBytes = (NW / 2) * kWaveRows * kCombStride * 4;
  static constexpr int kRingBytes = NS * STAGE > kDecBytes ? (NS * STAGE > kCombBytes ? NS * STAGE : kCombBytes)
                                                           : (kDecBytes > kCombBytes ? kDecBytes : kCombBytes);

  // copies of the K (and V) rows of keys [kbase, kbase + 32) into a wave's stage
  template <bool WITH_V>
  __device__ static __forceinline__ int dstage(const AttnParams& p, const Item& it, uint8_t* st, int kbase,
                                               int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
#pragma unroll
    for (int i = 0; i < DCOPIES; ++i) {
      const int r = i * RPW + lane / CPR;
      const int c = (lane % CPR) ^ sw(r);
      const char *kp, *vp;
      const bool ok = B::template row_src<true>(p, it, kbase + r, kp, vp);
      dma16<true>(ok ? kp + c * 16 : zeros, reinterpret_cast<uint16_t*>(st + i * RPW * ROW));
      if constexpr (WITH_V)
        dma16<true>(ok ? vp + c * 16 : zeros, reinterpret_cast<uint16_t*>(st + DTILE + i * RPW * ROW));
    }
    return WITH_V ? 2 * DCOPIES : DCOPIES;
  }

  // Decode-mode items of few rows keep their first-pass scores (fp32, in the
  // device work memory) instead of reading K again in the second pass.  The
  // item's block j (32 keys) holds nrows * 32 floats from float j * nrows * 32
  // on; a lane (lr, lg) of a valid row stores its 16 accumulator values there
  // as four 16-byte pieces, piece i4 at float 4 * (2 nrows i4 + nrows lg + lr),
  // so each store instruction writes one contiguous run.  The two passes then
  // move 8 * nrows bytes per key instead of the 128 bytes of a K code row.
  static constexpr int kScoreCopies = 4;                 // 16-byte pieces per lane and block
  __device__ static __forceinline__ float* score_at(float* sbase, int j, int nrows, int i4, int lr, int lg) {
    return sbase + static_cast<int64_t>(j) * nrows * 32 + (i4 * 2 * nrows + lg * nrows + lr) * 4;
  }
  // second pass with kept scores: this wave's scores of block j into the K
  // half of the stage (lane l's piece i4 at 1024 i4 + 16 l: only the lane
  // that stored it reads it back), the V rows into the V half
  __device__ static __forceinline__ int sstage(const AttnParams& p, const Item& it, uint8_t* st, float* sbase,
                                               int j, int nrows, bool row_ok, int kbase, int lane) {
    const char* zeros = static_cast<const char*>(p.zeros);
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int i4 = 0; i4 < kScoreCopies; ++i4)
      dma16<true>(row_ok ? static_cast<const void*>(score_at(sbase, j, nrows, i4, lr, lg)) : zeros,
                  reinterpret_cast<uint16_t*>(st + i4 * 1024));
#pragma unroll
    for (int i = 0; i < DCOPIES; ++i) {
      const int r = i * RPW + lane / CPR;
      const int c = (lane % CPR) ^ sw(r);
      const char *kp, *vp;
      const bool ok = B::template row_src<true>(p, it, kbase + r, kp, vp);
      dma16<true>(ok ? vp + c * 16 : zeros, reinterpret_cast<uint16_t*>(st + DTILE + i * RPW * ROW));
    }
    return kScoreCopies + DCOPIES;
  }

  __device__ static __forceinline__ void dec_item(const AttnParams& p, const WorkItem& item, const SeqInfo& sq,
                                                  const Item& it, uint8_t* ring, float* ml, int* lims, float c,
                                                  float out_scale, int wave, int lr, int lg, int t) {
    const int lane = t & 63;
    const int kbeg = item.key_begin;
    const int q_start = __builtin_amdgcn_readfirstlane(sq.q_start);
    const bool row_ok = lr < item.nrows;
    i32x8 qf[KS];
    int token, qh;
    load_q8(p, sq, it.kvh, item.row0 + lr, row_ok, lg, qf, token, qh);
    const int shift = sq.kv_len - sq.q_len;
    {
      int lim = it.kend - 1;
      if (p.causal) lim = min(lim, token + shift);
      lims[t] = lim - lg * 4;
    }
    // keys some row sees: [kbeg, whi]; keys every row sees: [kbeg, wlo]
    int wlo = it.kend - 1, whi = it.kend - 1;
    if (p.causal) {
      wlo = min(wlo, item.row0 / p.g + shift);
      whi = min(whi, (item.row0 + item.nrows - 1) / p.g + shift);
    }
    const int nb = whi < kbeg ? 0 : (whi - kbeg) / DK + 1;
    const int n_full = max(0, (wlo - kbeg + 1) / DK);
    uint8_t* const mine = ring + wave * 2 * DSTAGE;
    // scores kept between the passes (the host gives such items a place)
    const int nrows = __builtin_amdgcn_readfirstlane(item.nrows);
    const int spart = __builtin_amdgcn_readfirstlane(item.part);
    const bool keep = D == 128 && spart >= 0;
    float* const sbase = p.scores + static_cast<int64_t>(spart < 0 ? 0 : spart) * 32;
    // this wave's blocks: the next one is copied while the current one is
    // computed (its stage was read by the block before, already consumed).
    // `stage_fn` issues a block's copies and returns their count; `extra` is
    // the number of stores each body issues (in flight behind the next
    // block's copies, which complete in issue order after them)
    auto pass = [&](auto&& stage_fn, int extra, auto&& body) {
      int j = wave;
      if (j >= nb) return;
      const int cpb = stage_fn(mine, j);
      for (int i = 0; j < nb; ++i, j += NW) {
        const bool more = j + NW < nb;
        if (more) stage_fn(mine + ((i + 1) & 1) * DSTAGE, j + NW);
        wait_vmem_upto((more ? cpb : 0) + (i > 0 ? extra : 0));
        body(j, mine + (i & 1) * DSTAGE);
      }
    };
    auto stage_k = [&](uint8_t* st, int j) { return dstage<false>(p, it, st, kbeg + j * DK, lane); };
    auto stage_kv = [&](uint8_t* st, int j) { return dstage<true>(p, it, st, kbeg + j * DK, lane); };

    float m_run = -INFINITY, l_run = 0.f;
    pass(stage_k, keep ? kScoreCopies : 0, [&](int j, const uint8_t* st) {
      f32x16 acc[1];
      qk<1>(st, qf, acc, lr, lg);
      if constexpr (D == 128) {
        if (keep && row_ok) {
#pragma unroll
          for (int i4 = 0; i4 < kScoreCopies; ++i4)
            *reinterpret_cast<float4*>(score_at(sbase, j, nrows, i4, lr, lg)) =
                make_float4(acc[0][4 * i4], acc[0][4 * i4 + 1], acc[0][4 * i4 + 2], acc[0][4 * i4 + 3]);
        }
      }
      if (j < n_full) stats<1, false>(acc, m_run, l_run, 0, c);
      else stats<1, true>(acc, m_run, l_run, lims[t] - (kbeg + j * DK), c);
    });
    // the row's maximum and sum over the eight waves (in wave order)
    const float l_w = wave_pair_sum(l_run);
    if (lg == 0) {
      ml[wave * kWaveRows + lr] = m_run;
      ml[(NW + wave) * kWaveRows + lr] = l_w;
    }
    __syncthreads();
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, ml[w * kWaveRows + lr]);
    float l = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = ml[w * kWaveRows + lr];
        if (mw != -INFINITY) l += ml[(NW + w) * kWaveRows + lr] * __builtin_amdgcn_exp2f((mw - m) * c);
      }
    }
    const bool live = l > 0.f;
    const float neg2 = live ? -(m * c + __log2f(l) + p.p_log2) : 0.f;

    f32x16 o[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    auto pv = [&](int j, const uint8_t* st, const f32x16 (&acc)[1]) {
      const i32x8 pb = j < n_full ? probs<1, false>(acc, 0, c, neg2)
                                  : probs<1, true>(acc, lims[t] - (kbeg + j * DK), c, neg2);
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
        o[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vread<1>(st + DTILE, d, lr, lg), pb, o[d], 0, 0, 0,
                                                               0, 0, 0);
    };
    bool kept = false;
    if constexpr (D == 128) {
      if (keep) {
        kept = true;
        wait_vmem();   // this lane's score stores are complete before it copies them back
        auto stage_sv = [&](uint8_t* st, int j) {
          return sstage(p, it, st, sbase, j, nrows, row_ok, kbeg + j * DK, lane);
        };
        pass(stage_sv, 0, [&](int j, const uint8_t* st) {
          f32x16 acc[1];
#pragma unroll
          for (int i4 = 0; i4 < kScoreCopies; ++i4) {
            const u32x4 x = B::template lds_read<u32x4>(
                B::lds_addr(reinterpret_cast<const uint16_t*>(st + i4 * 1024 + lane * 16)));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[0][4 * i4 + e] = __uint_as_float(x[e]);
          }
          pv(j, st, acc);
        });
      }
    }
    if (!kept) {
      pass(stage_kv, 0, [&](int j, const uint8_t* st) {
        f32x16 acc[1];
        qk<1>(st, qf, acc, lr, lg);
        pv(j, st, acc);
      });
    }
    // partial outputs summed over the waves in a fixed tree: wave w + half
    // hands its sums to wave w, half = 4, 2, 1
    float* const so = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
      __syncthreads();   // rings, or the previous round's slots, are free
      if (wave >= half && wave < 2 * half) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<float4*>(so + ((wave - half) * kWaveRows + lr) * kCombStride + d * 32 + i4 * 8 +
                                       lg * 4) =
                make_float4(o[d][i4 * 4], o[d][i4 * 4 + 1], o[d][i4 * 4 + 2], o[d][i4 * 4 + 3]);
      }
      __syncthreads();
      if (wave < half) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const float4 f = *reinterpret_cast<const float4*>(so + (wave * kWaveRows + lr) * kCombStride +
                                                              d * 32 + i4 * 8 + lg * 4);
            o[d][i4 * 4] += f.x;
            o[d][i4 * 4 + 1] += f.y;
            o[d][i4 * 4 + 2] += f.z;
            o[d][i4 * 4 + 3] += f.w;
          }
      }
    }
    if (wave == 0) {
      const float inv = live ? out_scale : 0.f;
      const float lse_v = live ? m * c * kLn2 + __logf(l) : -INFINITY;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) B::store_out_block(p, q_start, token, qh, d, o[d], inv, lg, row_ok);
      if (row_ok && lg == 0 && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + q_start + token] = lse_v;
    }
  }

  __device__ static __forceinline__ void run(const AttnParams& p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];
    __shared__ int32_t pids[kMaxItemPages];
    __shared__ int lims[NT];
    __shared__ float ml[2 * NW * kWaveRows];
    __shared__ typename B::QEntry qbuf[B::kQueueChunk];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;
    const int lg = lane >> 5;
    const float c = p.qk_scale_log2;
    const float out_scale = p.v_scale;
    // prefill-mode items first, then decode-mode ones (each body in a pass of
    // its own keeps the register allocation of the other out of it)
    B::template for_each_item<0>(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      item(p, e.item, e.item.s, it, ring, lims, c, out_scale, wave, lr, lg, t);
    });
    B::template for_each_item<1>(p, qbuf, pids, t, NT, [&](const typename B::QEntry& e, const Item& it) {
      dec_item(p, e.item, e.item.s, it, ring, ml, lims, c, out_scale, wave, lr, lg, t);
    });
  }
};

template <int D>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void attn_prob8_kernel(const AttnParams p) {
  Prob8<D>::run(p);
}

// ROPE: the query rows are turned by rotary embedding as they are loaded
// (separate instantiations, so that the other kernels' register allocation
// does not carry the rotation code)
template <int D, int FMT, bool PAGED, bool ROPE, bool DECAPP = false>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(const AttnParams p) {
  Decode<D, FMT, PAGED, ROPE, kWaves, DECAPP>::run(p);
}

template <int D, int FMT, bool PAGED, bool ROPE>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void attn_prefill_kernel(const AttnParams p) {
  Prefill<D, FMT, PAGED, ROPE>::run(p);
}

template <int D, int FMT, bool PAGED, bool ROPE>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void attn_mixed_kernel(const AttnParams p) {
  Mixed<D, FMT, PAGED, ROPE>::run(p);
}

template <int D, int FMT, bool PAGED, bool ROPE>
int launch_t(const AttnParams& p, int grid, int mode, hipStream_t s) {
  if (mode == kGridDecode && p.dec_append) {
    // (the host sets dec_append only for fp8 caches with head_dim 128 and unturned keys)
    if constexpr (FMT == kKvFp8 && PAGED && D == 128 && !ROPE)
      hipLaunchKernelGGL((attn_decode_kernel<D, FMT, PAGED, ROPE, true>), dim3(grid), dim3(kThreads), 0, s, p);
    else
      return static_cast<int>(hipErrorInvalidValue);
  } else if (mode == kGridDecode)
    hipLaunchKernelGGL((attn_decode_kernel<D, FMT, PAGED, ROPE>), dim3(grid), dim3(kThreads), 0, s, p);
  else if (mode == kGridMixed)
    hipLaunchKernelGGL((attn_mixed_kernel<D, FMT, PAGED, ROPE>), dim3(grid), dim3(kPrefillWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<D, FMT, PAGED, ROPE>), dim3(grid), dim3(kPrefillWaves * 64), 0, s, p);
  return static_cast<int>(hipGetLastError());
}

template <int D, bool ROPE>
int launch_d(const AttnParams& p, int grid, int kv_format, bool paged, int mode, hipStream_t s) {
  if (!paged) return launch_t<D, kKvBf16, false, ROPE>(p, grid, mode, s);
  if (kv_format == kKvFp8) return launch_t<D, kKvFp8, true, ROPE>(p, grid, mode, s);
  return launch_t<D, kKvBf16, true, ROPE>(p, grid, mode, s);
}

}  // namespace

int launch_attention_prob8(const AttnParams& p, int grid, int head_dim, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_prob8_kernel<128>, dim3(grid), dim3(kPrefillWaves * 64), 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_prob8_kernel<64>, dim3(grid), dim3(kPrefillWaves * 64), 0, s, p);
  else
    return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

int launch_attention(const AttnParams& p, int grid, int head_dim, int kv_format, bool paged,
                     int mode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool rope = p.rope.dim > 0;
  if (head_dim == 128)
    return rope ? launch_d<128, true>(p, grid, kv_format, paged, mode, s)
                : launch_d<128, false>(p, grid, kv_format, paged, mode, s);
  if (head_dim == 64)
    return rope ? launch_d<64, true>(p, grid, kv_format, paged, mode, s)
                : launch_d<64, false>(p, grid, kv_format, paged, mode, s);
  return static_cast<int>(hipErrorInvalidValue);
}

}  // namespace vpk
