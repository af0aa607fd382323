// Attention over a paged KV cache for packed variable-length queries, gfx950.
//
// One workgroup (4 wavefronts, 256 threads) processes one work item at a time:
// up to 128 packed query rows of one sequence under one kv head, against the
// keys [key_begin, key_end) of that sequence.  Rows are (token, query head)
// pairs packed token-major, so the g query heads that share a kv head
// (grouped-query attention, vLLM Triton FAv2 PR page, feature list) all use
// each K/V tile staged in LDS.
//
// Per 64-key block:
//   a2  the block's K rows and V rows are gathered through the sequence's page
//       list (one page table for K and V: TransformerEngine KV-cache PR page,
//       Description) with 16-byte loads; fp8 e4m3fn codes are widened to bf16
//       exactly; K is stored row-major, V transposed (keys contiguous per
//       head-dim row), both in LDS;  keys past the item's end read as zero.
//   a3  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//       column and 32 of the block's 64 keys, the other 32 sit in lane ^ 32.
//   a4  keys beyond the item's end, or (causal) beyond token + Lk - Lq, are
//       set to -inf; only blocks that cross that bound are masked.
//   a5  online softmax in base 2 (scale * log2 e folded into one multiply):
//       row max over registers plus one permlane32 swap, running max and sum,
//       rescale of the output accumulator only when some row's max moved.
//   a6  O^T += V^T P^T on the same MFMA, P rounded to bf16 in registers.
//   a7  out = O / l (bf16) and lse = m ln 2 + ln l, or for a split part the
//       fp32 normalised partial and its lse for the merge pass.
//
// The online-softmax formulation and the split of the key range into parts
// that are merged afterwards follow the FlashAttention-2 design the pages
// build on ("Add flash_attn_varlen_func_with_kvcache", Limitation and the
// discussion of split-KV for decoding); the tiling, the transposed S layout
// and the LDS layouts here are this library's own for CDNA4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"

namespace vpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Cfg {
  static constexpr int KP = D + 8;              // K tile row pitch (bf16 elements)
  static constexpr int VP = kBlockN + 8;        // V^T tile row pitch (bf16 elements)
  static constexpr int K_ELEMS = kBlockN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dim
  static constexpr int DBLK = D / 32;           // 32-wide output blocks over the head dim
};

// e4m3fn code -> bf16 bits (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 8;
  const uint32_t em = c & 0x7Fu;
  // exponent field >= 1: rebias 7 -> 127 and move the 3 mantissa bits up by 4
  const uint32_t normal = (em << 4) + (120u << 7);
  // exponent field 0: m * 2^-9, normalised through an exact float product
  const uint32_t sub = __float_as_uint(static_cast<float>(em) * 0.001953125f) >> 16;
  uint32_t r = em >= 8u ? normal : sub;
  r = em == 0x7Fu ? 0x7FC0u : r;   // NaN
  return sign | r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Position of key k (0..63) inside a V^T row.  Within each group of 16 keys the
// quads are stored in the order 0, 2, 1, 3, so that the 8 keys one lane feeds
// to a PV k-step (keys 4l..4l+3 and 8+4l..8+4l+3 for lane half l) are adjacent.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

__device__ __forceinline__ float wave_pair_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float wave_pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int D, int FMT, bool PAGED>
struct Kernel {
  using C = Cfg<D>;
  static constexpr int ESIZE = FMT == kKvFp8 ? 1 : 2;       // bytes per stored element
  static constexpr int EPC = 16 / ESIZE;                    // elements per 16-byte chunk
  static constexpr int CPK = D / EPC;                       // chunks per key row
  static constexpr int KPASS = kBlockN * CPK / kThreads;    // K chunks per thread per block
  static constexpr int KSTRIDE = kThreads / CPK;            // keys between a thread's K chunks
  static constexpr int VTHREADS = 16 * CPK;                 // threads that load V (4 keys each)
  static_assert(KPASS >= 1 && KPASS * kThreads == kBlockN * CPK, "K load split");
  static_assert(VTHREADS <= kThreads, "V load split");

  struct Regs {
    u32x4 k[KPASS];
    u32x4 v[4];
  };

  // Global address (in elements) of key `key` of the item for kv head `kvh`.
  // Returns -1 when the page id is unusable.
  __device__ static __forceinline__ int64_t row_elem(const AttnParams& p, const int32_t* pids,
                                                     int first_page, int kn_start, int key,
                                                     int kvh) {
    if constexpr (PAGED) {
      int pi, slot;
      if (p.page_shift >= 0) {
        pi = key >> p.page_shift;
        slot = key & (p.page_size - 1);
      } else {
        pi = key / p.page_size;
        slot = key - pi * p.page_size;
      }
      const int page = pids[pi - first_page];
      if (page < 0) return -1;
      return ((static_cast<int64_t>(page) * p.page_size + slot) * p.hkv + kvh) * D;
    } else {
      return (static_cast<int64_t>(kn_start + key) * p.hkv + kvh) * D;
    }
  }

  __device__ static __forceinline__ void load_block(const AttnParams& p, Regs& r,
                                                    const int32_t* pids, int first_page,
                                                    int kn_start, int kvh, int kbase,
                                                    int kend) {
    const int t = threadIdx.x;
    const char* kb = static_cast<const char*>(p.k);
    const char* vb = static_cast<const char*>(p.v);
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int kl = t / CPK + i * KSTRIDE;
      const int key = kbase + kl;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key < kend) {
        const int64_t e = row_elem(p, pids, first_page, kn_start, key, kvh);
        if (e >= 0)
          val = *reinterpret_cast<const u32x4*>(kb + (e + (t % CPK) * EPC) * ESIZE);
      }
      r.k[i] = val;
    }
    if (t < VTHREADS) {
      const int quad = t & 15;
      const int chunk = t >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kbase + quad * 4 + i;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (key < kend) {
          const int64_t e = row_elem(p, pids, first_page, kn_start, key, kvh);
          if (e >= 0) val = *reinterpret_cast<const u32x4*>(vb + (e + chunk * EPC) * ESIZE);
        }
        r.v[i] = val;
      }
    }
  }

  __device__ static __forceinline__ void store_block(const Regs& r, uint16_t* klds,
                                                     uint16_t* vlds) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int kl = t / CPK + i * KSTRIDE;
      const int c = t % CPK;
      if constexpr (FMT == kKvFp8) {
        u32x4 lo, hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = r.k[i][w];
          const uint32_t b0 = e4m3_to_bf16(x & 0xFF), b1 = e4m3_to_bf16((x >> 8) & 0xFF);
          const uint32_t b2 = e4m3_to_bf16((x >> 16) & 0xFF), b3 = e4m3_to_bf16(x >> 24);
          if (w < 2) {
            lo[2 * w] = b0 | (b1 << 16);
            lo[2 * w + 1] = b2 | (b3 << 16);
          } else {
            hi[2 * (w - 2)] = b0 | (b1 << 16);
            hi[2 * (w - 2) + 1] = b2 | (b3 << 16);
          }
        }
        *reinterpret_cast<u32x4*>(klds + kl * C::KP + c * 16) = lo;
        *reinterpret_cast<u32x4*>(klds + kl * C::KP + c * 16 + 8) = hi;
      } else {
        *reinterpret_cast<u32x4*>(klds + kl * C::KP + c * 8) = r.k[i];
      }
    }
    if (t < VTHREADS) {
      const int quad = t & 15;
      const int chunk = t >> 4;
      const int pos = vt_pos(quad * 4);
      if constexpr (FMT == kKvFp8) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int sh = 8 * (j & 3);
          const uint32_t e0 = e4m3_to_bf16((r.v[0][j >> 2] >> sh) & 0xFF);
          const uint32_t e1 = e4m3_to_bf16((r.v[1][j >> 2] >> sh) & 0xFF);
          const uint32_t e2 = e4m3_to_bf16((r.v[2][j >> 2] >> sh) & 0xFF);
          const uint32_t e3 = e4m3_to_bf16((r.v[3][j >> 2] >> sh) & 0xFF);
          u32x2 w2 = {e0 | (e1 << 16), e2 | (e3 << 16)};
          *reinterpret_cast<u32x2*>(vlds + (chunk * 16 + j) * C::VP + pos) = w2;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sh = 16 * (j & 1);
          const uint32_t e0 = (r.v[0][j >> 1] >> sh) & 0xFFFF;
          const uint32_t e1 = (r.v[1][j >> 1] >> sh) & 0xFFFF;
          const uint32_t e2 = (r.v[2][j >> 1] >> sh) & 0xFFFF;
          const uint32_t e3 = (r.v[3][j >> 1] >> sh) & 0xFFFF;
          u32x2 w2 = {e0 | (e1 << 16), e2 | (e3 << 16)};
          *reinterpret_cast<u32x2*>(vlds + (chunk * 8 + j) * C::VP + pos) = w2;
        }
      }
    }
  }

  __device__ static void run(const AttnParams& p) {
    __shared__ __attribute__((aligned(16))) uint16_t klds[C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vlds[C::V_ELEMS];
    __shared__ int32_t pids[PAGED ? kMaxItemPages : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lr = lane & 31;   // query column of this lane
    const int lg = lane >> 5;   // lane half

    int it = blockIdx.x, it_end = blockIdx.x + 1;
    if (p.persistent) {
      it = p.queue_start[blockIdx.x];
      it_end = p.queue_start[blockIdx.x + 1];
    }

    for (; it < it_end; ++it) {
      const WorkItem item = p.items[it];
      const SeqInfo sq = p.seqs[item.seq];
      const int kvh = item.kv_head;
      const int kbeg = item.key_begin;
      const int kend = item.key_end;

      // ---- page ids of the item's key range -> LDS
      int first_page = 0;
      if constexpr (PAGED) {
        if (kend > kbeg) {
          first_page = kbeg / p.page_size;
          const int last_page = (kend - 1) / p.page_size;
          const int32_t* bt = p.block_table + static_cast<int64_t>(item.seq) * p.max_pages;
          __syncthreads();   // previous item may still read pids
          for (int i = t; i <= last_page - first_page; i += kThreads) {
            int pg = bt[first_page + i];
            if (pg < 0 || pg >= p.num_pages) {
              atomicOr(p.err_flag, 1);
              pg = -1;
            }
            pids[i] = pg;
          }
          __syncthreads();
        }
      }

      // ---- this wave's query rows -> registers (B operand of S^T = K Q^T)
      const int wrow = wave * kWaveRows + lr;             // row within the tile
      const bool row_ok = wrow < item.nrows;
      const bool wave_active = wave * kWaveRows < item.nrows;
      const int prow = item.row0 + wrow;                  // packed row within the sequence
      const int token = prow / p.g;
      const int qh = kvh * p.g + (prow - token * p.g);
      bf16x8 qf[C::KSTEPS];
      {
        const uint16_t* qrow = p.q + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row_ok) v = *reinterpret_cast<const u32x4*>(qrow + s * 16 + lg * 8);
          qf[s] = __builtin_bit_cast(bf16x8, v);
        }
      }

      // last visible key of this lane's row, and of the tile's first row
      const int shift = sq.kv_len - sq.q_len;
      int lim = kend - 1;
      if (p.causal) lim = min(lim, token + shift);
      int tile_lim = kend - 1;
      if (p.causal) tile_lim = min(tile_lim, item.row0 / p.g + shift);

      f32x16 o[C::DBLK];
#pragma unroll
      for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
      float m_run = -INFINITY;
      float l_run = 0.f;

      Regs regs;
      if (kend > kbeg) load_block(p, regs, pids, first_page, sq.kn_start, kvh, kbeg, kend);

      for (int kbase = kbeg; kbase < kend; kbase += kBlockN) {
        __syncthreads();                 // everyone is done reading the previous block
        store_block(regs, klds, vlds);
        __syncthreads();                 // block visible to all waves
        if (kbase + kBlockN < kend)
          load_block(p, regs, pids, first_page, sq.kn_start, kvh, kbase + kBlockN, kend);
        if (!wave_active) continue;

        // ---- a3: S^T = K Q^T, two 32-key halves
        f32x16 acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
#pragma unroll
          for (int s = 0; s < C::KSTEPS; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                klds + (h * 32 + lr) * C::KP + s * 16 + lg * 8);
            acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc[h], 0, 0, 0);
          }
        }

        // ---- a4 + a5: scale, mask, running max
        const bool need_mask = kbase + kBlockN - 1 > tile_lim;
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float sv = acc[h][i] * p.qk_scale_log2;
            if (need_mask) {
              const int key = kbase + h * 32 + (i >> 2) * 8 + lg * 4 + (i & 3);
              sv = key <= lim ? sv : -INFINITY;
            }
            acc[h][i] = sv;
            mx = fmaxf(mx, sv);
          }
        mx = wave_pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        float psum = 0.f;
        bf16x8 pf[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = __builtin_amdgcn_exp2f(acc[h][i] - m_use);
            psum += pv;
            pf[h][i >> 3][i & 7] = static_cast<__bf16>(pv);
          }
        l_run = l_run * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
        }

        // ---- a6: O^T += V^T P^T
#pragma unroll
        for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                  vlds + (d * 32 + lr) * C::VP + h * 32 + hh * 16 + lg * 8);
              o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[h][hh], o[d], 0, 0, 0);
            }
      }

      // ---- a7: epilogue
      if (wave_active) {
        const float l_tot = wave_pair_sum(l_run);
        const bool live = l_tot > 0.f;
        const float inv = live ? p.v_scale / l_tot : 0.f;
        const float lse_v = live ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
        if (row_ok) {
          if (item.part < 0) {
            uint16_t* orow = p.out + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D;
#pragma unroll
            for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = d * 32 + i4 * 8 + lg * 4;
                u32x2 w2;
                w2[0] = f32_to_bf16_rne(o[d][i4 * 4 + 0] * inv) |
                        (static_cast<uint32_t>(f32_to_bf16_rne(o[d][i4 * 4 + 1] * inv)) << 16);
                w2[1] = f32_to_bf16_rne(o[d][i4 * 4 + 2] * inv) |
                        (static_cast<uint32_t>(f32_to_bf16_rne(o[d][i4 * 4 + 3] * inv)) << 16);
                *reinterpret_cast<u32x2*>(orow + d0) = w2;
              }
            if (lg == 0 && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + sq.q_start + token] = lse_v;
          } else {
            float* prow_o = p.part_o + static_cast<int64_t>(item.part + wrow) * D;
#pragma unroll
            for (int d = 0; d < C::DBLK; ++d)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = d * 32 + i4 * 8 + lg * 4;
                float4 f;
                f.x = o[d][i4 * 4 + 0] * inv;
                f.y = o[d][i4 * 4 + 1] * inv;
                f.z = o[d][i4 * 4 + 2] * inv;
                f.w = o[d][i4 * 4 + 3] * inv;
                *reinterpret_cast<float4*>(prow_o + d0) = f;
              }
            if (lg == 0) p.part_lse[item.part + wrow] = lse_v;
          }
        }
      }
    }
  }
};

template <int D, int FMT, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const AttnParams p) {
  Kernel<D, FMT, PAGED>::run(p);
}

template <int D, int FMT, bool PAGED>
int launch_t(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, FMT, PAGED>), dim3(grid), dim3(kThreads), 0, s, p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_attention(const AttnParams& p, int grid, int head_dim, int kv_format, bool paged,
                     void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) {
    if (!paged) return launch_t<128, kKvBf16, false>(p, grid, s);
    if (kv_format == kKvFp8) return launch_t<128, kKvFp8, true>(p, grid, s);
    return launch_t<128, kKvBf16, true>(p, grid, s);
  }
  if (head_dim == 64) {
    if (!paged) return launch_t<64, kKvBf16, false>(p, grid, s);
    if (kv_format == kKvFp8) return launch_t<64, kKvFp8, true>(p, grid, s);
    return launch_t<64, kKvBf16, true>(p, grid, s);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

}  // namespace vpk
