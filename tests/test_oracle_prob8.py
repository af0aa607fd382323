"""Pins for the oracle's fp8 "QKV-Prob" attention (CPU only).

Facts used, none taken from the function under test:
  * the float64 encoder against brute force over the 127 finite magnitudes;
  * rows whose probabilities are exact e4m3 values: one visible key (P = 1)
    gives that key's value row; 2^k keys with equal scores (P = 2^-k) give
    the mean of their value rows (numpy's mean);
  * the row LSE equals the plain attention's (``oracle.attend``, pinned in
    test_oracle_attention.py) on the dequantised query codes, and every
    probability code equals the brute-force encoding of that attention's
    probability over p_scale, except within the stated band of a rounding
    boundary, where either neighbour is accepted;
  * the output differs from the plain attention by at most the quantisation
    error of e4m3 (half a step: 2^-4 of a normal value, 2^-10 below 2^-6);
  * the query codes of ``run_call(prob8=...)`` equal torch's float8_e4m3fn
    cast of fp32(q) * fp32(1 / q_scale) wherever that cast is finite.
Planted mistakes (a dropped p_scale, no normalisation, an unquantised P, the
query scale left out) each fail one of these; the last test plants them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3fn_decode, e4m3fn_encode_f64
from oracle import prob8 as P8

_VALS = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))   # finite magnitudes, codes 0..0x7E


def _brute_encode(y):
    """Nearest finite e4m3fn magnitude by exhaustive search, ties to the even code."""
    out = np.empty(len(y), np.uint8)
    for i, v in enumerate(y):
        if v >= 448.0:
            out[i] = 0x7E
            continue
        d = np.abs(_VALS - v)
        best = np.flatnonzero(d == d.min())
        out[i] = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
    return out


def test_encode_f64_against_brute_force():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        rng.uniform(0, 1, 2000) * 2.0 ** rng.integers(-12, 9, 2000),
        0.5 * (_VALS[:-1] + _VALS[1:]),                      # exact midpoints
        np.nextafter(0.5 * (_VALS[:-1] + _VALS[1:]), 0),     # just below
        np.nextafter(0.5 * (_VALS[:-1] + _VALS[1:]), 1e9),   # just above
        _VALS, [0.0, 447.9, 448.0, 460.0, 1e6],
    ])
    assert np.array_equal(e4m3fn_encode_f64(y), _brute_encode(y))


def _codes(rng, shape, lo=-1.0, hi=1.0, scale=1.0):
    x = rng.uniform(lo, hi, shape).astype(np.float32) / np.float32(scale)
    return oracle.e4m3fn_encode(x)


def test_single_visible_key_gives_its_value_row():
    rng = np.random.default_rng(1)
    L, H, D = 5, 2, 16
    Qc = _codes(rng, (L, H, D), scale=1 / 64)
    K = e4m3fn_decode(_codes(rng, (L, H, D), scale=1 / 64)) / 64
    V = e4m3fn_decode(_codes(rng, (L, H, D), scale=1 / 64)) / 64
    for p_scale in (1 / 448, 1 / 256, 1 / 64):
        out, lse = P8.attend(Qc, 1 / 64, K, V, causal=True, scale=0.3, p_scale=p_scale)
        # row 0 sees key 0 alone: P = 1, code of 1 / p_scale, value row 0
        w = e4m3fn_decode(e4m3fn_encode_f64(np.array([1 / np.float64(np.float32(p_scale))])))[0]
        w *= np.float64(np.float32(p_scale))
        np.testing.assert_allclose(out[0], w * V[0], rtol=1e-15, atol=0)
        assert abs(w - 1) < 2.0 ** -4
    # 1 / 256 maps P = 1 exactly onto code 256
    out, _ = P8.attend(Qc, 1 / 64, K, V, causal=True, scale=0.3, p_scale=1 / 256)
    assert np.array_equal(out[0], V[0])


@pytest.mark.parametrize("k", [0, 1, 3, 6])
def test_equal_scores_give_the_mean(k):
    rng = np.random.default_rng(k)
    n, H, D = 2 ** k, 1, 32
    Qc = _codes(rng, (3, H, D), scale=1 / 16)
    K = np.repeat(e4m3fn_decode(_codes(rng, (1, H, D))), n, axis=0)   # every key the same
    V = e4m3fn_decode(_codes(rng, (n, H, D))) * 0.5
    out, lse = P8.attend(Qc, 1 / 16, K, V, causal=False, scale=0.125, p_scale=2.0 ** -8)
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=0), out.shape), rtol=1e-14, atol=1e-15)
    s = 0.125 * (e4m3fn_decode(Qc[:, 0]) * np.float64(np.float32(1 / 16))) @ K[0, 0]
    np.testing.assert_allclose(lse[0], s + math.log(n), rtol=1e-13, atol=1e-13)


def _case(seed, Lq, Lk, Hq, Hkv, D, q_scale, causal):
    rng = np.random.default_rng(seed)
    Qc = _codes(rng, (Lq, Hq, D), -2, 2, q_scale)
    K = e4m3fn_decode(_codes(rng, (Lk, Hkv, D), -2, 2, 0.02)) * np.float64(np.float32(0.02))
    V = e4m3fn_decode(_codes(rng, (Lk, Hkv, D), -1, 1, 0.01)) * np.float64(np.float32(0.01))
    return Qc, K, V


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("p_scale", [1 / 448, 2.0 ** -7])
def test_against_plain_attention(causal, p_scale):
    Lq, Lk, Hq, Hkv, D, q_scale, scale = 24, 40, 4, 2, 32, 0.015, 0.4
    Qc, K, V = _case(3, Lq, Lk, Hq, Hkv, D, q_scale, causal)
    band = 2.0 ** -12
    out, lse, bound, aux, pc = P8.attend(Qc, q_scale, K, V, causal, scale, p_scale, band=band,
                                         return_codes=True)
    Qd = e4m3fn_decode(Qc) * np.float64(np.float32(q_scale))
    ref_out, ref_lse, probs = oracle.attend(Qd, K, V, causal, scale, return_probs=True)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)
    ps = np.float64(np.float32(p_scale))
    y = probs / ps                                                   # [Hq, Lq, Lk]
    want = _brute_encode(y.reshape(-1)).reshape(y.shape)
    near, _ = P8.flip_bound(y, band)
    diff = pc != want
    assert not (diff & ~near).any()
    assert np.abs(pc.astype(int) - want.astype(int))[diff].max(initial=0) <= 1
    # quantisation error of each weight: half a step of e4m3 at that value
    half = np.maximum(2.0 ** -4 * probs, 2.0 ** -10 * ps)             # [Hq, Lq, Lk]
    g = Hq // Hkv
    for h in range(Hq):
        lim = half[h] @ np.abs(V[:, h // g, :])                      # [Lq, D]
        assert (np.abs(out[:, h, :] - ref_out[:, h, :]) <= lim + 1e-15).all()
    # P was quantised: the output is not the plain attention
    assert np.abs(out - ref_out).max() > 1e-6
    # the bound covers flips of the codes inside the band: each flip moves one
    # weight by one step of e4m3 at that value
    assert (bound >= 0).all()
    # the two neighbours of a value near a midpoint: c (below it) and c + 1
    c = np.where(e4m3fn_decode(want) <= y, want.astype(int), want.astype(int) - 1).clip(0, 0x7D)
    step = (e4m3fn_decode((c + 1).astype(np.uint8)) - e4m3fn_decode(c.astype(np.uint8))) * ps
    for h in range(Hq):
        fl = np.where(near[h], step[h], 0.0) @ np.abs(V[:, h // g, :])
        np.testing.assert_allclose(bound[:, h, :], fl, rtol=1e-12, atol=1e-300)
    # absum is sum_j |w_j| |v_j|, with w the dequantised weights
    for h in range(Hq):
        wv = (e4m3fn_decode(pc[h]) * ps) @ np.abs(V[:, h // g, :])
        np.testing.assert_allclose(aux["absum"][:, h, :], wv, rtol=1e-12)


def test_score_error_widens_the_band():
    Lq, Lk, Hq, Hkv, D, q_scale, scale = 16, 32, 2, 1, 32, 0.015, 0.4
    Qc, K, V = _case(4, Lq, Lk, Hq, Hkv, D, q_scale, False)
    b0 = P8.attend(Qc, q_scale, K, V, False, scale, 1 / 448, band=2.0 ** -12)[2]
    b1, aux = P8.attend(Qc, q_scale, K, V, False, scale, 1 / 448, band=2.0 ** -12, score_err=2.0 ** -10)[2:4]
    assert (b1 >= b0).all() and b1.sum() > b0.sum()
    Qd = e4m3fn_decode(Qc) * np.float64(np.float32(q_scale))
    T = scale * np.einsum("qd,kd->qk", np.abs(Qd[:, 0]), np.abs(K[:, 0]))
    np.testing.assert_allclose(aux["tmax"][0], T.max(axis=1), rtol=1e-12)


def test_bound_counts_only_codes_near_a_boundary():
    y = np.array([1.0, 1.0625, 1.0625 * (1 + 2.0 ** -14), 0.5 * (416 + 448), 2.0 ** -10, 500.0, 0.0])
    near, gap = P8.flip_bound(y, 2.0 ** -12)
    assert near.tolist() == [False, True, True, True, True, False, False]
    assert gap.tolist() == [0.0, 0.125, 0.125, 32.0, 2.0 ** -9, 0.0, 0.0]


def test_query_codes_match_torch_cast():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, S = 2, 4, 2, 32, 8
    q32 = rng.normal(0, 1, (10, Hq, D)).astype(np.float32)
    q = (q32.view(np.uint32) >> 16).astype(np.uint16)               # bf16 bits (truncated)
    cu = np.array([0, 4, 10], np.int32)
    kc = _codes(rng, (6, S, Hkv, D))
    vc = _codes(rng, (6, S, Hkv, D))
    bt = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    lens = np.array([20, 17], np.int32)
    q_scale = 0.0137
    r = oracle.run_call(q=q, cu_seqlens_q=cu, k_cache=kc, v_cache=vc, block_table=bt, cache_seqlens=lens,
                        page_size=S, causal=True, kv_scale=(0.02, 0.01), cache_dtype="fp8", Hkv=Hkv,
                        prob8=dict(q_scale=q_scale, p_scale=1 / 448))
    x = (q.astype(np.uint32) << 16).view(np.float32) * (np.float32(1) / np.float32(q_scale))
    t = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    fin = np.abs(x) < 448
    assert fin.mean() > 0.99
    assert np.array_equal(r["q_codes"][fin], t[fin])
    # the rows of each sequence are the single-sequence function's
    for b in range(B):
        K = e4m3fn_decode(oracle.depage(kc, bt[b], lens[b], S)) * np.float64(np.float32(0.02))
        V = e4m3fn_decode(oracle.depage(vc, bt[b], lens[b], S)) * np.float64(np.float32(0.01))
        o, l = P8.attend(r["q_codes"][cu[b]:cu[b + 1]], q_scale, K, V, True, 1 / math.sqrt(D), 1 / 448)
        assert np.array_equal(r["out"][cu[b]:cu[b + 1]], o)


def test_planted_mistakes_fail(monkeypatch):
    """Each plausible slip in the oracle breaks one of the pins above."""
    Lq, Lk, Hq, Hkv, D, q_scale, scale = 8, 16, 2, 1, 16, 0.015, 0.4
    Qc, K, V = _case(9, Lq, Lk, Hq, Hkv, D, q_scale, True)
    good = P8.attend(Qc, q_scale, K, V, True, scale, 1 / 448)[0]
    Qd = e4m3fn_decode(Qc) * np.float64(np.float32(q_scale))
    ref_out, _, probs = oracle.attend(Qd, K, V, True, scale, return_probs=True)

    def within_quant_error(out):
        half = np.maximum(2.0 ** -4 * probs, 2.0 ** -10 / 448)
        return all((np.abs(out[:, h] - ref_out[:, h]) <= half[h] @ np.abs(V[:, 0]) + 1e-15).all()
                   for h in range(Hq))

    assert within_quant_error(good)
    real_encode = P8.e4m3fn_encode_f64
    # p_scale dropped from the dequantisation: weights 448 times too large
    monkeypatch.setattr(P8, "e4m3fn_decode", lambda c: e4m3fn_decode(c) * 448)
    assert not within_quant_error(P8.attend(Qc, q_scale, K, V, True, scale, 1 / 448)[0])
    monkeypatch.undo()
    # P not quantised (codes replaced by the exact values)
    monkeypatch.setattr(P8, "e4m3fn_encode_f64", lambda y: y)
    monkeypatch.setattr(P8, "e4m3fn_decode", lambda c: np.asarray(c, np.float64) if c.dtype != np.uint8
                        else e4m3fn_decode(c))
    exact = P8.attend(Qc, q_scale, K, V, True, scale, 1 / 448)[0]
    assert np.abs(exact - ref_out).max() < 1e-12            # the "QKV-Prob" effect is gone
    monkeypatch.undo()
    assert P8.e4m3fn_encode_f64 is real_encode
    # query scale left out: the LSE no longer matches the plain attention
    _, lse_bad = P8.attend(Qc, 1.0, K, V, True, scale, 1 / 448)
    _, lse_ref = oracle.attend(Qd, K, V, True, scale)
    assert np.abs(lse_bad - lse_ref).max() > 1e-3
