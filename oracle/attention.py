"""Plain float64 attention over a paged KV cache (oracle; test infrastructure only).

The computation (no tiling, no splitting, no fusion):

  1. append   -- every new token j of sequence b lands at logical position
                 Lc_b + j of that sequence: page block_table[b, pos // S],
                 slot pos % S, all kv heads; stored as bf16 bits, or as e4m3fn
                 codes of fp32(x) * fp32(1/scale).  ("Add
                 flash_attn_varlen_func_with_kvcache", Usage: the cache is
                 updated in place; Minor Changes: the cache length is a
                 per-sequence attribute, new tokens have their own cumulative
                 offsets.)
  2. de-page  -- the keys/values of sequence b are the first Lk_b = Lc_b + Ln_b
                 logical positions read back through its block-table row,
                 dequantised.  ("Add KV cache for paged/non-paged attention",
                 Description: the unfused path turns the paged cache into a
                 contiguous one via the page table; K and V share the table.)
                 Attention therefore sees the new tokens as stored, i.e. after
                 the append (for fp8 they pass through the quantiser).
  3. scores   -- S = scale * Q_b[:, h] K_b[:, h // g]^T with g = Hq / Hkv
                 (grouped-query heads, consecutive groups; vLLM Triton FAv2 PR
                 page, feature list).
  4. mask     -- key j is visible to query i iff j < Lk and, when causal,
                 j <= i + Lk - Lq: the causal diagonal is aligned to the end of
                 the key range, so the last query sees every key (cutlass-sycl
                 "Extend FlashAttention Prefill with KV cache", description:
                 cached plus current KV, causal or not).
  5. softmax  -- m = row max; out = sum_j exp(S_ij - m) V_j / sum_j exp(S_ij - m);
                 lse = m + ln(sum_j exp(S_ij - m)); a row with no visible key
                 gives out = 0 and lse = -inf.

Inputs are raw representations: bf16 as uint16 bits ("bf16"), fp8 as uint8
e4m3fn codes with a float32 scale ("fp8"), or plain float32 ("f32", used by the
oracle's self-checks on the fp32 tiny workload).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import prob8 as _prob8
from . import rope as _rope
from .formats import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode


def _decode(arr: np.ndarray, dtype: str, scale: Optional[float] = None) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        return e4m3fn_decode(arr) * np.float64(np.float32(scale))
    if dtype == "f32":
        return np.asarray(arr, np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def _encode(rows: np.ndarray, src_dtype: str, cache_dtype: str, scale: Optional[float]) -> np.ndarray:
    """Stored representation of new K/V rows in a cache of ``cache_dtype``."""
    if cache_dtype == src_dtype:
        return np.array(rows, copy=True)          # bf16 -> bf16 (and f32 -> f32): byte copy
    if cache_dtype == "fp8":
        if src_dtype == "bf16":
            x32 = (np.asarray(rows, np.uint16).astype(np.uint32) << 16).view(np.float32)
        elif src_dtype == "f32":
            x32 = np.asarray(rows, np.float32)
        else:
            raise ValueError(src_dtype)
        inv = np.float32(1.0) / np.float32(scale)      # fp32 reciprocal of the scale
        with np.errstate(over="ignore", invalid="ignore"):
            prod = (x32 * inv).astype(np.float32)
        # 1/scale > 0, so the product has the input's sign; for a NaN input the
        # input's sign is the one stored (a NaN product's sign is not defined)
        prod = np.where(np.signbit(x32), -np.abs(prod), np.abs(prod)).astype(np.float32)
        return e4m3fn_encode(prod)
    raise ValueError(f"cannot store {src_dtype} in a {cache_dtype} cache")


def append(k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table, cache_seqlens,
           page_size: int, cache_dtype: str, kv_scale=None, new_dtype: str = "bf16"):
    """Return copies of (k_cache, v_cache) after writing every new token in place.

    Only slots [Lc_b, Lc_b + Ln_b) of each sequence change; every other byte of
    the pool is left as it was.  ``cache_seqlens`` is the length before the
    append and is not changed.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    if k_new is None:
        return kc, vc
    ks = vs = None
    if cache_dtype == "fp8":
        ks, vs = kv_scale
    B = len(cu_seqlens_knew) - 1
    for b in range(B):
        lc = int(cache_seqlens[b])
        for j in range(int(cu_seqlens_knew[b]), int(cu_seqlens_knew[b + 1])):
            pos = lc + (j - int(cu_seqlens_knew[b]))
            page = int(block_table[b, pos // page_size])
            slot = pos % page_size
            kc[page, slot] = _encode(k_new[j], new_dtype, cache_dtype, ks)
            vc[page, slot] = _encode(v_new[j], new_dtype, cache_dtype, vs)
    return kc, vc


def depage(pool: np.ndarray, table_row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Logical positions [0, length) of one sequence, gathered through its table row."""
    t = np.arange(length)
    return pool[np.asarray(table_row)[t // page_size], t % page_size]


def sequence_kv(b: int, *, k_new=None, v_new=None, cu_seqlens_knew=None, k_cache=None,
                v_cache=None, block_table=None, cache_seqlens=None, page_size=0,
                cache_dtype=None, kv_scale=None, new_dtype="bf16"):
    """Dequantised (K_b, V_b), float64 [Lk, Hkv, D], as attention sees them.

    With a cache, ``k_cache``/``v_cache`` must already hold the appended tokens.
    Without a cache the keys are the sequence's new tokens.
    """
    ln = 0 if cu_seqlens_knew is None else int(cu_seqlens_knew[b + 1] - cu_seqlens_knew[b])
    if k_cache is not None:
        lk = int(cache_seqlens[b]) + ln
        ks = vs = None
        if cache_dtype == "fp8":
            ks, vs = kv_scale
        K = _decode(depage(k_cache, block_table[b], lk, page_size), cache_dtype, ks)
        V = _decode(depage(v_cache, block_table[b], lk, page_size), cache_dtype, vs)
        return K, V
    s, e = int(cu_seqlens_knew[b]), int(cu_seqlens_knew[b + 1])
    return _decode(k_new[s:e], new_dtype), _decode(v_new[s:e], new_dtype)


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool, scale: float,
           rows: Optional[Sequence[int]] = None, return_probs: bool = False,
           key_range: Optional[tuple] = None):
    """Attention of one sequence.

    Q [Lq, Hq, D], K/V [Lk, Hkv, D] float64.  ``rows`` selects query indices
    (default: all), which lets a caller check single rows of a large batch.
    ``key_range=(k0, k1)`` restricts the visible keys to k0 <= j < k1 on top of
    the mask (one part of a split of the key range).
    Returns out [len(rows), Hq, D] and lse [Hq, len(rows)] (float64), plus the
    probability matrices [Hq, len(rows), Lk] when ``return_probs``.
    """
    Lq, Hq, D = Q.shape
    Lk, Hkv = K.shape[0], K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    rows = np.arange(Lq) if rows is None else np.asarray(rows, np.int64)
    R = len(rows)
    out = np.zeros((R, Hq, D), np.float64)
    lse = np.full((Hq, R), -np.inf, np.float64)
    probs = np.zeros((Hq, R, Lk), np.float64) if return_probs else None
    j = np.arange(Lk)
    visible = np.ones((R, Lk), bool)
    if causal:
        visible = j[None, :] <= (rows[:, None] + (Lk - Lq))
    if key_range is not None:
        visible = visible & (j[None, :] >= key_range[0]) & (j[None, :] < key_range[1])
    for h in range(Hq):
        kvh = h // g
        S = scale * (Q[rows, h, :] @ K[:, kvh, :].T)          # [R, Lk]
        S = np.where(visible, S, -np.inf)
        m = S.max(axis=1) if Lk else np.full(R, -np.inf)
        live = np.isfinite(m)
        if not live.any():
            continue
        P = np.exp(S[live] - m[live, None])
        l = P.sum(axis=1)
        out[live, h, :] = (P @ V[:, kvh, :]) / l[:, None]
        lse[h, live] = m[live] + np.log(l)
        if return_probs:
            probs[h, live] = P / l[:, None]
    if return_probs:
        return out, lse, probs
    return out, lse


def attend_rows(*args, **kwargs):
    """Alias of ``attend`` with an explicit ``rows`` selection (kept for readability at call sites)."""
    return attend(*args, **kwargs)


def merge_partials(parts):
    """Combine partial results over disjoint key ranges into the full result.

    ``parts`` is a list of (out_s [R, D], lse_s [R]) where out_s is already
    normalised over its own range.  lse = ln sum_s exp(lse_s);
    out = sum_s exp(lse_s - lse) * out_s.  Ranges where a row sees nothing carry
    lse_s = -inf and contribute nothing; a row that sees nothing anywhere gets
    out = 0, lse = -inf.
    """
    lses = np.stack([np.asarray(p[1], np.float64) for p in parts])       # [n, R]
    outs = np.stack([np.asarray(p[0], np.float64) for p in parts])       # [n, R, D]
    mx = lses.max(axis=0)
    live = np.isfinite(mx)
    safe_mx = np.where(live, mx, 0.0)
    w = np.exp(lses - safe_mx[None, :])                                  # exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = np.where(live, safe_mx + np.log(np.where(live, tot, 1.0)), -np.inf)
    out = np.where(live[:, None], (w[:, :, None] * outs).sum(axis=0) / np.where(live, tot, 1.0)[:, None], 0.0)
    return out, lse


def run_call(*, q, cu_seqlens_q, k_new=None, v_new=None, cu_seqlens_knew=None, k_cache=None,
             v_cache=None, block_table=None, cache_seqlens=None, page_size=0, causal=True,
             scale=None, kv_scale=None, cache_dtype=None, Hkv=None, q_dtype="bf16",
             new_dtype="bf16", seqs: Optional[Sequence[int]] = None, rope=None, prob8=None):
    """One whole call: append, then attention for every sequence.

    Returns dict(out [Tq, Hq, D], lse [Hq, Tq], k_cache, v_cache) with float64
    outputs and the caches as stored after the append.  ``seqs`` restricts the
    attention to some sequences (rows of the others stay 0 / -inf).  ``rope``
    (dict with cos, sin, rotary_dim, interleaved) first turns the query rows
    and the new key rows by their positions (``oracle.rope``); values and the
    cached rows are not turned.  ``prob8`` (dict with q_scale, p_scale and
    optionally band and score_err; fp8 cache only) runs the attention as fp8
    "QKV-Prob" (``oracle.prob8``): the query codes are taken after the
    rotation, and the result also holds q_codes [Tq, Hq, D] and, with a band,
    bound and absum [Tq, Hq, D] and tmax [Hq, Tq].
    """
    if rope is not None:
        if q_dtype != "bf16" or new_dtype != "bf16":
            raise ValueError("rotary embedding is defined here for bf16 rows")
        qpos, kpos = _rope.positions(cu_seqlens_q, cu_seqlens_knew, cache_seqlens)
        args = (rope["cos"], rope["sin"], int(rope["rotary_dim"]), bool(rope["interleaved"]))
        q = _rope.rotate_bf16(q, qpos, *args)
        if k_new is not None:
            k_new = _rope.rotate_bf16(k_new, kpos, *args)
    Q = _decode(q, q_dtype)
    Tq, Hq, D = Q.shape
    band = None
    if prob8 is not None:
        if q_dtype != "bf16" or cache_dtype != "fp8" or k_cache is None:
            raise ValueError("QKV-Prob attention is defined here for bf16 queries over an fp8 cache")
        q_codes = _encode(q, "bf16", "fp8", prob8["q_scale"])
        band = prob8.get("band")
        bound = np.zeros((Tq, Hq, D), np.float64)
        absum = np.zeros((Tq, Hq, D), np.float64)
        tmax = np.zeros((Hq, Tq), np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if k_cache is not None and k_new is not None:
        kc, vc = append(k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                        cache_seqlens, page_size, cache_dtype, kv_scale, new_dtype)
    else:
        kc, vc = k_cache, v_cache
    out = np.zeros((Tq, Hq, D), np.float64)
    lse = np.full((Hq, Tq), -np.inf, np.float64)
    B = len(cu_seqlens_q) - 1
    for b in (range(B) if seqs is None else seqs):
        s, e = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        K, V = sequence_kv(b, k_new=k_new, v_new=v_new, cu_seqlens_knew=cu_seqlens_knew,
                           k_cache=kc, v_cache=vc, block_table=block_table,
                           cache_seqlens=cache_seqlens, page_size=page_size,
                           cache_dtype=cache_dtype, kv_scale=kv_scale, new_dtype=new_dtype)
        if e > s and prob8 is not None:
            r = _prob8.attend(q_codes[s:e], prob8["q_scale"], K, V, causal, scale, prob8["p_scale"],
                              band=band, score_err=prob8.get("score_err", 0.0))
            out[s:e] = r[0]
            lse[:, s:e] = r[1]
            if band is not None:
                bound[s:e] = r[2]
                absum[s:e] = r[3]["absum"]
                tmax[:, s:e] = r[3]["tmax"]
        elif e > s:
            o, l = attend(Q[s:e], K, V, causal, scale)
            out[s:e] = o
            lse[:, s:e] = l
    res = dict(out=out, lse=lse, k_cache=kc, v_cache=vc)
    if prob8 is not None:
        res["q_codes"] = q_codes
        if band is not None:
            res.update(bound=bound, absum=absum, tmax=tmax)
    return res


def run_workload(wl, seqs=None):
    """``run_call`` on a synthetic workload object (attributes as produced by the generator)."""
    return run_call(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q, k_new=wl.k_new, v_new=wl.v_new,
                    cu_seqlens_knew=wl.cu_seqlens_knew, k_cache=wl.k_cache, v_cache=wl.v_cache,
                    block_table=wl.block_table, cache_seqlens=wl.cache_seqlens,
                    page_size=wl.page_size, causal=wl.causal, scale=wl.scale,
                    kv_scale=wl.kv_scale, cache_dtype=wl.cache_dtype, seqs=seqs)
