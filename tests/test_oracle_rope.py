"""Pins of the oracle's rotary embedding (oracle/rope.py) against facts that do
not come from the oracle itself: torch's float32 -> bfloat16 cast, rotation
as multiplication by a unit complex number (RoFormer, section 3.4), the
identity at position 0, hand-stated positions, and attention scores that
depend on positions only through their differences."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from synth import rope_tables


def _bf16_f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 130, 200000))).astype(np.float32)
    # exact ties (low half 0x8000) with odd and even kept halves, and carries into the exponent
    ties = (rng.integers(0, 1 << 16, 4000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)
    ties = ties[np.isfinite(ties.view(np.float32))]
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-45, -1e-45,
                        1.1754942e-38], np.float64).astype(np.float32)
    special = np.concatenate([special, np.array([0x7F7FFFFF, 0x3F80FFFF, 0x3F818000, 0x3F808000],
                                                np.uint32).view(np.float32)])
    for arr in (x, ties.view(np.float32), special):
        assert np.array_equal(rope.bf16_round_bits(arr), _torch_bf16_bits(arr))
    nan = np.array([np.nan, -np.nan], np.float32)
    assert np.all(np.isnan(_bf16_f64(rope.bf16_round_bits(nan))))


def _complex_route(x_bits, pos, R, interleaved, base):
    """Exact rotation (float64) of bf16 rows as a complex product; coordinates >= R unchanged."""
    x = _bf16_f64(x_bits)
    half = R // 2
    theta = base ** (-2.0 * np.arange(half) / R)
    w = np.exp(1j * np.asarray(pos, np.float64)[:, None, None] * theta[None, None, :])
    if interleaved:
        z = x[..., 0:R:2] + 1j * x[..., 1:R:2]
    else:
        z = x[..., :half] + 1j * x[..., half:R]
    z = z * w
    y = x.copy()
    if interleaved:
        y[..., 0:R:2], y[..., 1:R:2] = z.real, z.imag
    else:
        y[..., :half], y[..., half:R] = z.real, z.imag
    return x, y


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("R,D", [(128, 128), (64, 128), (32, 64)])
def test_rotation_is_a_complex_product(interleaved, R, D):
    rng = np.random.default_rng(2 + R + D + interleaved)
    T, H, base = 300, 3, 10000.0
    cos, sin = rope_tables(5000, R, base)
    x_bits = _torch_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    pos = rng.integers(0, 5000, T)
    got = _bf16_f64(rope.rotate_bf16(x_bits, pos, cos, sin, R, interleaved))
    x, exact = _complex_route(x_bits, pos, R, interleaved, base)
    # bf16 keeps 8 significant bits: half an ulp is at most 2^-8 of the value;
    # the float32 products and the fp32 angle tables add far less
    if interleaved:
        a, b = x[..., 0:R:2], x[..., 1:R:2]
    else:
        a, b = x[..., :R // 2], x[..., R // 2:R]
    ab = np.abs(a) + np.abs(b)
    mag = np.repeat(ab, 2, axis=-1) if interleaved else np.concatenate([ab, ab], axis=-1)
    err = np.abs(got[..., :R] - exact[..., :R])
    assert np.all(err <= 2.0 ** -8 * np.abs(exact[..., :R]) + 2.0 ** -20 * mag)
    assert np.array_equal(rope.rotate_bf16(x_bits, pos, cos, sin, R, interleaved)[..., R:], x_bits[..., R:])
    # each pair keeps its length (up to the same rounding)
    g = got[..., :R]
    ga, gb = (g[..., 0::2], g[..., 1::2]) if interleaved else (g[..., :R // 2], g[..., R // 2:])
    assert np.allclose(np.hypot(ga, gb), np.hypot(a, b), rtol=2.0 ** -7, atol=1e-6)


def test_position_zero_and_unnamed_rows_are_unchanged():
    rng = np.random.default_rng(3)
    cos, sin = rope_tables(10, 64)
    x_bits = _torch_bf16_bits(rng.standard_normal((5, 2, 64)).astype(np.float32))
    for inter in (False, True):
        assert np.array_equal(rope.rotate_bf16(x_bits, np.zeros(5, np.int64), cos, sin, 64, inter), x_bits)
        out = rope.rotate_bf16(x_bits, np.array([-1, 3, -1, 2, -1]), cos, sin, 64, inter)
        assert np.array_equal(out[[0, 2, 4]], x_bits[[0, 2, 4]])
        assert not np.array_equal(out[1], x_bits[1])


def test_positions_by_hand():
    # sequence 0: 1 new token over a cache of 7 -> both at 7; sequence 1: 3 new over 2 -> 2, 3, 4
    qpos, kpos = rope.positions([0, 1, 4], [0, 1, 4], [7, 2])
    assert qpos.tolist() == [7, 2, 3, 4] and kpos.tolist() == [7, 2, 3, 4]
    # cache-only decode: the query is the last cached key, position Lc - 1
    qpos, kpos = rope.positions([0, 1], None, [9])
    assert qpos.tolist() == [8] and kpos.size == 0
    # no cache: positions count from 0; more keys than queries: queries at the end
    qpos, kpos = rope.positions([0, 2], [0, 5], None)
    assert qpos.tolist() == [3, 4] and kpos.tolist() == [0, 1, 2, 3, 4]
    # query rows given by start and length, with unnamed rows
    qpos, _ = rope.positions(None, [0, 2, 3], [4, 0], q_start=[5, 0], q_len=[2, 1], total_q=8)
    assert qpos.tolist() == [0, -1, -1, -1, -1, 4, 5, -1]   # sequence 0: Lk = 4 + 2, two queries


@pytest.mark.parametrize("interleaved", [False, True])
def test_run_call_scores_depend_on_position_differences(interleaved):
    """Attention with rotated q / k equals attention whose score of query i and
    key j is Re(sum over pairs of zq_i conj(zk_j) exp(1j (m_i - n_j) theta))
    on the unrotated vectors, plus the unrotated coordinates' dot product."""
    rng = np.random.default_rng(4 + interleaved)
    Hq, Hkv, D, R, S, base = 4, 2, 64, 32, 4, 10000.0
    lc, ln = 11, 6                      # 11 cached keys, 6 new tokens, 6 queries
    lk = lc + ln
    cos, sin = rope_tables(64, R, base)
    raw_k = rng.standard_normal((lk, Hkv, D)).astype(np.float32)
    raw_q = rng.standard_normal((ln, Hq, D)).astype(np.float32)
    v = _torch_bf16_bits(rng.standard_normal((lk, Hkv, D)).astype(np.float32))
    k_bits = _torch_bf16_bits(raw_k)
    q_bits = _torch_bf16_bits(raw_q)
    # the cached keys were turned when they were appended: their positions 0 .. lc-1
    _, k_rot_exact = _complex_route(k_bits[:lc], np.arange(lc), R, interleaved, base)
    cached = _torch_bf16_bits(k_rot_exact.astype(np.float32))
    pages = lk // S + 2
    perm = rng.permutation(pages)
    kc = np.zeros((pages, S, Hkv, D), np.uint16)
    vc = np.zeros((pages, S, Hkv, D), np.uint16)
    bt = perm[None, :].astype(np.int32)
    for t in range(lc):
        kc[bt[0, t // S], t % S] = cached[t]
        vc[bt[0, t // S], t % S] = v[t]
    res = oracle.run_call(q=q_bits, cu_seqlens_q=np.array([0, ln], np.int32), k_new=k_bits[lc:],
                          v_new=v[lc:], cu_seqlens_knew=np.array([0, ln], np.int32), k_cache=kc,
                          v_cache=vc, block_table=bt, cache_seqlens=np.array([lc], np.int32), page_size=S,
                          causal=True, cache_dtype="bf16",
                          rope=dict(cos=cos, sin=sin, rotary_dim=R, interleaved=interleaved))
    # relative form, float64, from the unrotated bf16 vectors
    theta = base ** (-2.0 * np.arange(R // 2) / R)
    xq, xk, xv = _bf16_f64(q_bits), _bf16_f64(k_bits), _bf16_f64(v)
    m = lc + np.arange(ln)              # query positions
    n = np.arange(lk)                   # key positions
    pair = (lambda x: x[..., 0:R:2] + 1j * x[..., 1:R:2]) if interleaved else \
        (lambda x: x[..., :R // 2] + 1j * x[..., R // 2:R])
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    ref = np.zeros((ln, Hq, D))
    for h in range(Hq):
        zq, zk = pair(xq[:, h]), pair(xk[:, h // g])
        phase = np.exp(1j * (m[:, None, None] - n[None, :, None]) * theta[None, None, :])
        s = np.real((zq[:, None, :] * np.conj(zk[None, :, :]) * phase).sum(-1))
        s += xq[:, h, R:] @ xk[:, h // g, R:].T
        s = s * scale
        s[n[None, :] > m[:, None]] = -np.inf
        p = np.exp(s - s.max(1, keepdims=True))
        ref[:, h] = (p / p.sum(1, keepdims=True)) @ xv[:, h // g]
    # the oracle rounds the turned q / k to bf16 (about 2^-9 of each value)
    assert np.abs(res["out"] - ref).max() < 1e-2
    # the appended rows are the turned new keys
    for j in range(ln):
        t = lc + j
        _, ex = _complex_route(k_bits[t:t + 1], np.array([t]), R, interleaved, base)
        got = _bf16_f64(res["k_cache"][bt[0, t // S], t % S])
        assert np.all(np.abs(got - ex[0]) <= 2.0 ** -8 * np.abs(ex[0]) + 1e-6)
