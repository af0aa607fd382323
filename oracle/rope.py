"""Rotary position embedding of the query rows and new key rows (oracle side).

Test infrastructure, like the rest of ``oracle/``.

The pages name rotary embedding for inference as the step that comes with the
KV-cache path ("Add KV cache for paged/non-paged attention", TransformerEngine
PR, Description: RoPE to be fixed for inference) but do not define it.  This
follows the published method (Su et al., "RoFormer: Enhanced Transformer with
Rotary Position Embedding", 2021, section 3.4): a vector's coordinates are
taken in pairs, and pair i at position m is turned by the angle m * theta_i.
The caller supplies the angles as tables cos[m, i], sin[m, i] (float32,
[max_positions, rotary_dim / 2]); the first ``rotary_dim`` coordinates are
turned, the others are left as they are.  Two pairings are common: the
half-split one (coordinate i with i + rotary_dim / 2) and the interleaved one
(coordinate 2i with 2i + 1).

Readings taken where the pages are silent:
  * positions: new token j of sequence b sits at Lc_b + j, the slot the append
    writes; query row i sits at Lk_b - Lq_b + i, the key position its
    end-aligned causal bound stops at;
  * the rotated rows replace the bf16 inputs, so they are bf16 values; the
    rounding to bf16 decides a stored code, so it is taken in the kernel's
    precision: each product rounded to float32, their difference (or sum)
    rounded to float32, then round-to-nearest-even to bf16.
"""
from __future__ import annotations

import numpy as np


def bf16_round_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN stays NaN (quiet)."""
    x32 = np.ascontiguousarray(x32, np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    r[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return r


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def positions(cu_seqlens_q, cu_seqlens_knew, cache_seqlens, q_start=None, q_len=None, total_q=None):
    """(query-row positions [Tq], new-token positions [Tn]) as int64; -1 for rows no sequence names.

    ``q_start`` / ``q_len`` give the query rows of each sequence when they are
    not the packed ``cu_seqlens_q`` ranges (then ``total_q`` is the row count).
    """
    if q_start is None:
        cu = np.asarray(cu_seqlens_q, np.int64)
        q_start, q_len, total_q = cu[:-1], np.diff(cu), int(cu[-1])
    q_start = np.asarray(q_start, np.int64)
    q_len = np.asarray(q_len, np.int64)
    B = q_start.size
    ln = np.zeros(B, np.int64) if cu_seqlens_knew is None else np.diff(np.asarray(cu_seqlens_knew, np.int64))
    lc = np.zeros(B, np.int64) if cache_seqlens is None else np.asarray(cache_seqlens, np.int64)
    lk = lc + ln
    qpos = np.full(int(total_q), -1, np.int64)
    kpos = np.full(int(ln.sum()), -1, np.int64)
    for b in range(B):
        qpos[q_start[b]:q_start[b] + q_len[b]] = lk[b] - q_len[b] + np.arange(q_len[b])
        if cu_seqlens_knew is not None:
            s = int(cu_seqlens_knew[b])
            kpos[s:s + ln[b]] = lc[b] + np.arange(ln[b])
    return qpos, kpos


def rotate_bf16(x_bits: np.ndarray, pos: np.ndarray, cos32: np.ndarray, sin32: np.ndarray,
                rotary_dim: int, interleaved: bool) -> np.ndarray:
    """Rotated copy of bf16 rows x [T, H, D] (uint16 bits), row t at position pos[t].

    Rows with pos < 0 are returned unchanged.  Coordinates >= rotary_dim are
    copied.  For a pair (a, b) with angle (c, s):
        a' = bf16(f32(f32(a c) - f32(b s))),  b' = bf16(f32(f32(a s) + f32(b c))).
    """
    x_bits = np.asarray(x_bits, np.uint16)
    out = np.array(x_bits, copy=True)
    R = int(rotary_dim)
    half = R // 2
    if half == 0:
        return out
    live = np.nonzero(np.asarray(pos) >= 0)[0]
    if live.size == 0:
        return out
    x = _bf16_to_f32(x_bits[live])                       # [n, H, D] float32
    c = np.asarray(cos32, np.float32)[np.asarray(pos)[live]][:, None, :]   # [n, 1, half]
    s = np.asarray(sin32, np.float32)[np.asarray(pos)[live]][:, None, :]
    if interleaved:
        a, b = x[..., 0:R:2], x[..., 1:R:2]
    else:
        a, b = x[..., :half], x[..., half:R]
    with np.errstate(over="ignore", invalid="ignore"):
        a2 = (a * c).astype(np.float32) - (b * s).astype(np.float32)
        b2 = (a * s).astype(np.float32) + (b * c).astype(np.float32)
    ra, rb = bf16_round_bits(a2.astype(np.float32)), bf16_round_bits(b2.astype(np.float32))
    rows = out[live]
    if interleaved:
        rows[..., 0:R:2], rows[..., 1:R:2] = ra, rb
    else:
        rows[..., :half], rows[..., half:R] = ra, rb
    out[live] = rows
    return out
