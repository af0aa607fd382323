"""Seeded synthetic workloads for varlen attention over a paged KV cache.

Five named workloads mirror the batch shapes the pages discuss: a tiny
correctness case, varlen prefill without a cache, paged decode, chunked prefill
over a cached prefix, and a mixed prefill+decode batch over an fp8 cache.

Representation (numpy, host memory):
  * bf16 tensors are ``uint16`` bit patterns (RNE from float32, via torch's cast);
  * fp8 tensors are ``uint8`` OCP e4m3fn codes;
  * index arrays are ``int32``.

Layouts:
  q          [Tq, Hq, D]          packed tokens of all sequences ("THD")
  k_new/v_new[Tn, Hkv, D]         packed new tokens
  k_cache    [P, S, Hkv, D]       page pool; page p, slot s, kv head h
  block_table[B, max_pages]       page ids, padded with -1
  lse        [Hq, Tq]             (produced by the method, not here)

The pre-existing cache prefix of the fp8 workload is produced with torch's
float8_e4m3fn cast of ``fp32(x) * fp32(1/scale)``; that is input preparation,
and the method's own append quantises the new tokens independently.

Random draw order for seed ``s`` (``numpy.random.default_rng(s)``):
  1. lengths (q/new lengths, then cache lengths, per workload rule);
  2. Q values, float32 N(0,1), shape [Tq, Hq, D];
  3. K values for every sequence's full key range, [sum Lk, Hkv, D], then V;
  4. page permutation of the pool;
  5. filler values for pool slots that hold no key (N(0,1), or NaN when
     ``poison`` is set).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0

# name -> static description; lengths are drawn by ``_draw_lengths``.
WORKLOADS = {
    "tiny": dict(B=2, Hq=2, Hkv=2, D=64, page_size=4, causal=True, cache_dtype="bf16"),
    "varlen_prefill": dict(B=16, Hq=32, Hkv=8, D=128, page_size=0, causal=True, cache_dtype=None),
    "paged_decode": dict(B=64, Hq=32, Hkv=8, D=128, page_size=16, causal=True, cache_dtype="bf16"),
    "chunked_prefill": dict(B=8, Hq=32, Hkv=8, D=128, page_size=64, causal=True, cache_dtype="bf16"),
    "mixed_fp8": dict(B=64, Hq=32, Hkv=8, D=128, page_size=16, causal=True, cache_dtype="fp8"),
}

# Per-workload seed base: workload N of the list above uses seed N + 1000 * rep.
SEED_BASE = {"tiny": 1, "varlen_prefill": 2, "paged_decode": 3, "chunked_prefill": 4, "mixed_fp8": 5}


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    causal: bool
    scale: float
    q: np.ndarray                       # uint16 [Tq, Hq, D]
    cu_seqlens_q: np.ndarray            # int32 [B+1]
    k_new: Optional[np.ndarray]         # uint16 [Tn, Hkv, D]
    v_new: Optional[np.ndarray]
    cu_seqlens_knew: Optional[np.ndarray]
    k_cache: Optional[np.ndarray]       # uint16 | uint8 [P, S, Hkv, D]
    v_cache: Optional[np.ndarray]
    cache_dtype: Optional[str]          # "bf16" | "fp8" | None
    block_table: Optional[np.ndarray]   # int32 [B, max_pages]
    cache_seqlens: Optional[np.ndarray] # int32 [B]
    kv_scale: Optional[tuple]           # (k_scale, v_scale) float32, fp8 only
    # float32 values before the bf16 rounding (tiny workload only)
    f32: Optional[dict] = None

    @property
    def Tq(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def Tn(self) -> int:
        return 0 if self.cu_seqlens_knew is None else int(self.cu_seqlens_knew[-1])

    @property
    def num_pages(self) -> int:
        return 0 if self.k_cache is None else int(self.k_cache.shape[0])

    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    def new_lens(self) -> np.ndarray:
        if self.cu_seqlens_knew is None:
            return np.zeros(self.B, np.int64)
        return np.diff(self.cu_seqlens_knew)

    def cache_lens(self) -> np.ndarray:
        if self.cache_seqlens is None:
            return np.zeros(self.B, np.int64)
        return self.cache_seqlens.astype(np.int64)

    def kv_lens(self) -> np.ndarray:
        return self.cache_lens() + self.new_lens()


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn codes with torch's cast (used only to prepare a cache prefix)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact); used for input preparation only."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rope_tables(max_positions: int, rotary_dim: int, base: float = 10000.0):
    """Angle tables for rotary embedding: (cos, sin), float32 [max_positions, rotary_dim / 2].

    Entry [m, i] is cos / sin of m * base ** (-2 i / rotary_dim), computed in
    float64 and rounded once to float32.  This is a caller-side input (like a
    weight): neither the oracle nor the kernels compute the angles.
    """
    half = rotary_dim // 2
    theta = np.float64(base) ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _draw_lengths(name: str, rng: np.random.Generator):
    """Return (q_lens, new_lens, cache_lens) as int64 arrays."""
    if name == "tiny":
        ql = np.array([3, 5]); cl = np.array([7, 0])
        return ql, ql.copy(), cl
    if name == "varlen_prefill":
        ql = rng.integers(256, 2048, size=16, endpoint=True)
        return ql, ql.copy(), np.zeros(16, np.int64)
    if name == "paged_decode":
        ql = np.ones(64, np.int64)
        cl = rng.integers(1024, 4096, size=64, endpoint=True)
        return ql, ql.copy(), cl
    if name == "chunked_prefill":
        ql = rng.integers(128, 512, size=8, endpoint=True)
        cl = rng.integers(2048, 8192, size=8, endpoint=True)
        return ql, ql.copy(), cl
    if name == "mixed_fp8":
        pq = rng.integers(1024, 2048, size=4, endpoint=True)
        pc = rng.integers(0, 1024, size=4, endpoint=True)
        dc = rng.integers(512, 8192, size=60, endpoint=True)
        ql = np.concatenate([pq, np.ones(60, np.int64)])
        cl = np.concatenate([pc, dc])
        return ql, ql.copy(), cl
    raise KeyError(name)


def make_custom(*, q_lens, new_lens, cache_lens, Hq, Hkv, D, page_size, causal=True,
                cache_dtype="bf16", seed=0, scale=None, pool_factor=1.25,
                poison=False, extra_pages=0, name="custom", tiny_table=False,
                value_std=1.0, lengths_only=False) -> Workload:
    """Draw a workload with explicit per-sequence lengths.

    ``cache_dtype=None`` means there is no cache: attention runs over the new
    tokens only and ``cache_lens`` must be all zero.
    ``new_lens`` entries may be 0; pass ``new_lens=None`` for a call without new
    K/V (attention over the cache only).
    ``lengths_only`` skips every value draw (q/k/v/caches are empty arrays);
    lengths and the page-table rule are kept, the permutation itself differs.
    """
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, np.int64)
    B = len(q_lens)
    has_new = new_lens is not None
    new_lens = np.zeros(B, np.int64) if new_lens is None else np.asarray(new_lens, np.int64)
    cache_lens = np.asarray(cache_lens, np.int64)
    if cache_dtype is None:
        assert not cache_lens.any(), "a call without a cache has no cached prefix"
        assert has_new, "a call without a cache needs new K/V"
    kv_lens = cache_lens + new_lens
    scale = (1.0 / math.sqrt(D)) if scale is None else scale

    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_kn = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(kv_lens.sum())

    if lengths_only:
        Tq_, Tk_ = 0, 0
    else:
        Tq_, Tk_ = Tq, Tk
    q32 = rng.standard_normal((Tq_, Hq, D), dtype=np.float32) * np.float32(value_std)
    k32 = rng.standard_normal((Tk_, Hkv, D), dtype=np.float32) * np.float32(value_std)
    v32 = rng.standard_normal((Tk_, Hkv, D), dtype=np.float32) * np.float32(value_std)
    q = to_bf16_bits(q32)
    kb = to_bf16_bits(k32)
    vb = to_bf16_bits(v32)
    cu_k = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int64)

    # split every sequence's keys into its cached prefix and its new tokens
    new_idx = np.concatenate([np.arange(cu_k[b] + cache_lens[b], cu_k[b + 1]) for b in range(B)]
                             ).astype(np.int64) if Tk_ else np.zeros(0, np.int64)
    k_new = kb[new_idx] if has_new else None
    v_new = vb[new_idx] if has_new else None

    wl = dict(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size,
              causal=bool(causal), scale=float(scale), q=q, cu_seqlens_q=cu_q,
              k_new=k_new, v_new=v_new, cu_seqlens_knew=cu_kn if has_new else None,
              cache_dtype=cache_dtype, k_cache=None, v_cache=None, block_table=None,
              cache_seqlens=None, kv_scale=None)

    if cache_dtype is not None:
        S = page_size
        need = -(-kv_lens // S)
        if tiny_table:
            pool = 6
            perm = rng.permutation(pool)
            bt = perm.reshape(B, -1).astype(np.int32)
            max_pages = bt.shape[1]
        else:
            pool = int(math.ceil(pool_factor * need.sum())) + extra_pages
            pool = max(pool, int(need.sum()), 1)
            perm = rng.permutation(pool)
            max_pages = max(int(need.max()) if B else 0, 1)
            bt = np.full((B, max_pages), -1, np.int32)
            off = 0
            for b in range(B):
                bt[b, :need[b]] = perm[off:off + need[b]]
                off += need[b]
        shape = (pool, S, Hkv, D)
        if lengths_only:
            empty = np.zeros((0, S, Hkv, D), np.uint8 if cache_dtype == "fp8" else np.uint16)
            wl.update(k_cache=empty, v_cache=empty.copy(), block_table=bt,
                      cache_seqlens=cache_lens.astype(np.int32),
                      kv_scale=(np.float32(1), np.float32(1)) if cache_dtype == "fp8" else None)
            return Workload(**wl)
        if poison:
            fill_k = np.full(shape, np.nan, np.float32)
            fill_v = np.full(shape, np.nan, np.float32)
        else:
            fill_k = rng.standard_normal(shape, dtype=np.float32)
            fill_v = rng.standard_normal(shape, dtype=np.float32)
        # slot coordinates of every cached (prefix) token
        pre_src, pre_page, pre_slot = [], [], []
        for b in range(B):
            t = np.arange(cache_lens[b])
            pre_src.append(cu_k[b] + t)
            pre_page.append(bt[b, t // S] if len(t) else np.zeros(0, np.int64))
            pre_slot.append(t % S)
        pre_src = np.concatenate(pre_src).astype(np.int64)
        pre_page = np.concatenate(pre_page).astype(np.int64)
        pre_slot = np.concatenate(pre_slot).astype(np.int64)
        if cache_dtype == "bf16":
            kc = to_bf16_bits(fill_k)
            vc = to_bf16_bits(fill_v)
            kc[pre_page, pre_slot] = kb[pre_src]
            vc[pre_page, pre_slot] = vb[pre_src]
            kv_scale = None
        elif cache_dtype == "fp8":
            kf = bf16_bits_to_f32(kb)
            vf = bf16_bits_to_f32(vb)
            k_scale = np.float32(np.abs(kf).max() if kf.size else 1.0) / np.float32(E4M3_MAX)
            v_scale = np.float32(np.abs(vf).max() if vf.size else 1.0) / np.float32(E4M3_MAX)
            k_scale = np.float32(k_scale if k_scale > 0 else 1.0)
            v_scale = np.float32(v_scale if v_scale > 0 else 1.0)
            if poison:
                kc = np.full(shape, 0x7F, np.uint8)
                vc = np.full(shape, 0x7F, np.uint8)
            else:
                spread = np.float32(E4M3_MAX / 8.0)
                kc = to_e4m3_codes(np.clip(fill_k * spread, -E4M3_MAX, E4M3_MAX))
                vc = to_e4m3_codes(np.clip(fill_v * spread, -E4M3_MAX, E4M3_MAX))
            inv_k = np.float32(1.0) / k_scale
            inv_v = np.float32(1.0) / v_scale
            kc[pre_page, pre_slot] = to_e4m3_codes(kf[pre_src] * inv_k)
            vc[pre_page, pre_slot] = to_e4m3_codes(vf[pre_src] * inv_v)
            kv_scale = (np.float32(k_scale), np.float32(v_scale))
        else:
            raise ValueError(cache_dtype)
        wl.update(k_cache=kc, v_cache=vc, block_table=bt,
                  cache_seqlens=cache_lens.astype(np.int32), kv_scale=kv_scale)
        if tiny_table or name == "tiny":
            wl["f32"] = dict(q=q32, k=k32, v=v32, cu_k=cu_k)
    return Workload(**wl)


def make_workload(name: str, rep: int = 0, *, poison: bool = False,
                  lengths_only: bool = False) -> Workload:
    """The named workload with seed ``SEED_BASE[name] + 1000 * rep``."""
    spec = WORKLOADS[name]
    seed = SEED_BASE[name] + 1000 * rep
    rng = np.random.default_rng(seed)
    ql, nl, cl = _draw_lengths(name, rng)
    # the lengths consumed the first draws of this stream; the tensor draws
    # come from a stream seeded one step later so that they do not depend on
    # how many numbers the length rule drew
    return make_custom(q_lens=ql, new_lens=nl, cache_lens=cl, Hq=spec["Hq"], Hkv=spec["Hkv"],
                       D=spec["D"], page_size=spec["page_size"], causal=spec["causal"],
                       cache_dtype=spec["cache_dtype"], seed=seed + 500, poison=poison,
                       name=name, tiny_table=(name == "tiny"), lengths_only=lengths_only)


def subset(wl: Workload, seqs) -> Workload:
    """The sub-batch of sequences ``seqs`` (in that order) of a workload, over the same page pools:
    its query rows, new tokens, length arrays and block-table rows.  Input preparation only (used to
    time the parts of a mixed batch alone)."""
    seqs = [int(b) for b in seqs]
    ql = wl.q_lens()[seqs]
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = (np.concatenate([wl.q[wl.cu_seqlens_q[b]:wl.cu_seqlens_q[b + 1]] for b in seqs])
         if seqs else wl.q[:0])
    k_new = v_new = cu_kn = None
    if wl.cu_seqlens_knew is not None:
        nl = wl.new_lens()[seqs]
        cu_kn = np.concatenate([[0], np.cumsum(nl)]).astype(np.int32)
        sl = [slice(int(wl.cu_seqlens_knew[b]), int(wl.cu_seqlens_knew[b + 1])) for b in seqs]
        k_new = np.concatenate([wl.k_new[s] for s in sl]) if seqs else wl.k_new[:0]
        v_new = np.concatenate([wl.v_new[s] for s in sl]) if seqs else wl.v_new[:0]
    bt = wl.block_table[seqs] if wl.block_table is not None else None
    cl = wl.cache_seqlens[seqs] if wl.cache_seqlens is not None else None
    return dataclasses.replace(wl, name=f"{wl.name}[{len(seqs)} seqs]", B=len(seqs), q=q, cu_seqlens_q=cu_q,
                               k_new=k_new, v_new=v_new, cu_seqlens_knew=cu_kn, block_table=bt,
                               cache_seqlens=cl, f32=None)
