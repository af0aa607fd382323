"""fp8 "QKV-Prob" attention, plain float64 (oracle; test infrastructure only).

The vLLM Triton FAv2 PR page ("[Kernel][Triton][FP8] Adding fp8 and variable
length sequence support to Triton FAv2 kernel", feature list item 7 and the
paragraph before the LM EVAL tables) names models whose attention runs with
Q, K and V in fp8 and whose softmax output is quantised to fp8 before the
second product, at some cost in accuracy.  The page fixes neither the fp8
variant, nor the scales, nor where a tiled kernel quantises.  Readings used
here (the plainest the page supports):

  1. query codes -- each query element (after rotary embedding, when a call
     asks for it) is stored as e4m3fn by the cache's rule with a per-tensor
     q_scale: code = E(fp32(q) * fp32(1 / q_scale)), E = nearest e4m3fn value,
     ties to the even code, saturating at +-448 (``formats``).
  2. keys and values -- the e4m3fn cache codes with k_scale and v_scale, as in
     the 8-bit cache path (``attention``).
  3. scores -- S_ij = scale * (q_scale qcode_i) . (k_scale kcode_j), with the
     usual mask (end of the keys; causal diagonal aligned to the end).
  4. softmax -- P_ij = exp(S_ij - LSE_i), LSE_i = ln sum_j exp(S_ij) over the
     visible keys: the row's exact softmax, not one relative to a partial
     maximum of some block of keys, so the result does not depend on how a
     kernel tiles the keys.
  5. P quantisation -- pcode_ij = E(P_ij / p_scale) with a per-tensor p_scale
     (the natural choice 1 / 448 maps P = 1 to the largest finite code); the
     decision is taken on the float64 value.
  6. second product -- out_i = p_scale * sum_j pcode_ij * (v_scale vcode_j);
     no renormalisation after the quantisation.
  7. lse_i = LSE_i; a row with no visible key gives out = 0, lse = -inf.

Where a kernel computes P in float32, the value P / p_scale can land on the
other side of a rounding boundary than the float64 value does.  ``attend``
therefore also reports, for a relative band around every boundary, the
largest change of out that such flips can cause (``bound``): an element
whose value lies within the band may take either neighbouring code.  The
band of element (i, j) is ``band + score_err * (T_ij + max_j' T_ij')`` with
T_ij = scale * sum_d |q_id k_jd|: a product unit whose sums carry an error
of up to score_err * sum |terms| moves S_ij by at most score_err * T_ij and
the LSE by at most score_err * max_j T_ij, and P by the exponential of
their difference.  For the same reason ``attend`` reports T's row maximum
(``tmax``, to bound the LSE) and p_scale * sum_j |pcode_ij| |v_jd|
(``absum``, to bound the error of the second product's sums).

Pinned by tests/test_oracle_prob8.py: the float64 encoder against brute force
over the code table; rows whose probabilities are exact e4m3 values (one
visible key, equal scores over a power-of-two count of keys) against closed
forms; LSE and the quantised probabilities against the plain attention of
``attention.attend`` and a brute-force encoder; the query codes against
torch's float8_e4m3fn cast.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .formats import _POS, e4m3fn_decode, e4m3fn_encode_f64

# default relative band around rounding boundaries (see ``attend``)
DEFAULT_BAND = 2.0 ** -12


def flip_bound(y: np.ndarray, band):
    """For values y >= 0 (P / p_scale): which lie within a relative ``band``
    (a number, or an array shaped like y) of a rounding boundary between two
    neighbouring e4m3fn values, and the gap between those two values (0 where
    no flip is possible)."""
    y = np.asarray(y, np.float64)
    hi = np.searchsorted(_POS, y, side="left")
    hi_c = np.clip(hi, 1, 0x7E)
    lo_c = hi_c - 1
    lo_v, hi_v = _POS[lo_c], _POS[hi_c]
    mid = 0.5 * (lo_v + hi_v)
    near = (np.abs(y - mid) <= band * y) & (y <= _POS[0x7E])
    return near, np.where(near, hi_v - lo_v, 0.0)


def attend(Qc: np.ndarray, q_scale: float, K: np.ndarray, V: np.ndarray, causal: bool, scale: float,
           p_scale: float, rows: Optional[Sequence[int]] = None, band: Optional[float] = None,
           return_codes: bool = False, score_err: float = 0.0):
    """QKV-Prob attention of one sequence.

    Qc [Lq, Hq, D] uint8 query codes; K, V [Lk, Hkv, D] float64, dequantised
    (scales applied).  ``rows`` selects query indices.  Returns out
    [R, Hq, D] and lse [Hq, R]; with ``band`` also bound [R, Hq, D], the
    largest change of out that flips of codes within the band (widened by
    ``score_err`` as the module text says) can cause, and a dict with tmax
    [Hq, R] and absum [R, Hq, D]; with ``return_codes`` also pcodes
    [Hq, R, Lk] (uint8; 0 for masked keys).
    """
    Q = e4m3fn_decode(Qc) * np.float64(np.float32(q_scale))
    Lq, Hq, D = Q.shape
    Lk, Hkv = K.shape[0], K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    ps = np.float64(np.float32(p_scale))
    rows = np.arange(Lq) if rows is None else np.asarray(rows, np.int64)
    R = len(rows)
    out = np.zeros((R, Hq, D), np.float64)
    lse = np.full((Hq, R), -np.inf, np.float64)
    bound = np.zeros((R, Hq, D), np.float64) if band is not None else None
    tmax = np.zeros((Hq, R), np.float64) if band is not None else None
    absum = np.zeros((R, Hq, D), np.float64) if band is not None else None
    codes_all = np.zeros((Hq, R, Lk), np.uint8) if return_codes else None
    j = np.arange(Lk)
    visible = np.ones((R, Lk), bool)
    if causal:
        visible = j[None, :] <= (rows[:, None] + (Lk - Lq))
    for h in range(Hq):
        kvh = h // g
        S = scale * (Q[rows, h, :] @ K[:, kvh, :].T)                 # step 3
        S = np.where(visible, S, -np.inf)
        m = S.max(axis=1) if Lk else np.full(R, -np.inf)
        live = np.isfinite(m)
        if not live.any():
            continue
        L = m[live] + np.log(np.exp(S[live] - m[live, None]).sum(axis=1))   # step 4
        P = np.exp(S[live] - L[:, None])
        y = P / ps                                                      # step 5
        pc = e4m3fn_encode_f64(y)
        w = e4m3fn_decode(pc) * ps
        out[live, h, :] = w @ V[:, kvh, :]                              # step 6
        lse[h, live] = L
        if band is not None:
            T = scale * (np.abs(Q[rows[live], h, :]) @ np.abs(K[:, kvh, :]).T)
            T = np.where(visible[live], T, 0.0)
            tm = T.max(axis=1)
            _, gap = flip_bound(y, band + score_err * (T + tm[:, None]))
            bound[live, h, :] = (gap * ps) @ np.abs(V[:, kvh, :])
            tmax[h, live] = tm
            absum[live, h, :] = np.abs(w) @ np.abs(V[:, kvh, :])
        if return_codes:
            codes_all[h, live] = pc
    res = [out, lse]
    if band is not None:
        res.append(bound)
        res.append(dict(tmax=tmax, absum=absum))
    if return_codes:
        res.append(codes_all)
    return tuple(res)
