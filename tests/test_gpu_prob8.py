"""GPU parity of the fp8 "QKV-Prob" attention against the oracle (``oracle.prob8``).

The oracle decides every probability code in float64.  The kernel decides it
in float32 from scores summed by gfx950's fp8 matrix cores, which do not sum
exactly: each product of a 64-term group is cut to a grid about 13 bits below
the group's largest product (448 + 0.1406 gives 448.125; 448 + 0.0176 gives
448).  On codes of amax-scaled normal data the sums deviate from exact ones
by at most 2^-14.8 of the sum of their terms' magnitudes (262,144 sums), on
random full-range codes by 2^-12.8.  Two kinds of tests follow from that:

* exact scores: query and key codes from two binades ([1/8, 1/2)), so every
  product is a multiple of 2^-12 while the grid is at most 2^-16 -- the score
  sums are exact and only float32 rounding of exp2, log2 and the fma moves
  P / p_scale, far inside the band (relative 2^-12) around each rounding
  boundary in which the test accepts either neighbouring code;
* the pages' distributions (normal data, amax-scaled codes): the band is
  widened by SCORE_ERR = 2^-12 times the score magnitudes (7x the largest
  deviation measured on such codes).

The output bound per element is

    |out - ref| <= bound + SCORE_ERR * absum + 2^-8 |ref| + 1e-6

``bound`` is the largest change flips inside the band can make, SCORE_ERR *
absum covers the error of the second product's sums, 2^-8 |ref| the bf16
rounding of the output.  LSE: |lse - ref| <= score_err * tmax + 1e-4 (tmax =
the row's largest scale * sum_d |q k|).  Rows that see no key must be 0 with
lse -inf, exactly.
"""
import dataclasses
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import varlen_paged_kv_amd as vpk
from gpu_util import DeviceCall, say, to_np_out
from synth import make_custom, make_workload, rope_tables

pytestmark = pytest.mark.gpu

SCORE_ERR = 2.0 ** -12
BAND = 2.0 ** -12


def _q_scale(wl, shrink=1.0):
    q = (wl.q.astype(np.uint32) << 16).view(np.float32)
    return float(np.float32(np.abs(q).max() / 448.0 * shrink))


def _run(dc, q_scale, p_scale, rope=None):
    wl = dc.wl
    kw = {}
    if rope is not None:
        kw = dict(rope_cos=rope["cos_dev"], rope_sin=rope["sin_dev"], rotary_dim=rope["rotary_dim"],
                  interleaved=rope["interleaved"])
    return vpk.attn_varlen_paged_qkv_prob_fwd(
        dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl, wl.page_size,
        wl.causal, wl.scale, wl.kv_scale, q_scale=q_scale, p_scale=p_scale, host_index=dc.host, **kw)


def _oracle(wl, q_scale, p_scale, with_new=True, rope=None, seqs=None, score_err=SCORE_ERR):
    rp = None if rope is None else {k: rope[k] for k in ("cos", "sin", "rotary_dim", "interleaved")}
    return oracle.run_call(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q,
                           k_new=wl.k_new if with_new else None, v_new=wl.v_new if with_new else None,
                           cu_seqlens_knew=wl.cu_seqlens_knew if with_new else None,
                           k_cache=wl.k_cache, v_cache=wl.v_cache, block_table=wl.block_table,
                           cache_seqlens=wl.cache_seqlens, page_size=wl.page_size, causal=wl.causal,
                           scale=wl.scale, kv_scale=wl.kv_scale, cache_dtype="fp8", rope=rp, seqs=seqs,
                           prob8=dict(q_scale=q_scale, p_scale=p_scale, band=BAND, score_err=score_err))


def check_prob8(out_np, lse_np, ref, label, rows=None, score_err=SCORE_ERR):
    """out [R, Hq, D], lse [Hq, R] against the oracle's result (restricted to ``rows``)."""
    r_out, r_lse, bound, absum, tmax = (ref["out"], ref["lse"], ref["bound"], ref["absum"], ref["tmax"])
    if rows is not None:
        r_out, bound, absum = r_out[rows], bound[rows], absum[rows]
        r_lse, tmax = r_lse[:, rows], tmax[:, rows]
    dead = np.isneginf(r_lse)
    assert np.array_equal(np.isneginf(lse_np), dead), f"{label}: -inf rows differ"
    assert np.all(out_np[dead.T] == 0), f"{label}: rows with no key must be 0"
    assert np.all(np.isfinite(out_np)), f"{label}: non-finite output"
    live = ~dead.T
    err = np.abs(out_np - r_out)
    lim = bound + SCORE_ERR * absum + 2.0 ** -8 * np.abs(r_out) + 1e-6
    bad = (err > lim) & live[:, :, None]
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} elements beyond the bound; first {tuple(i)}: "
                             f"got {out_np[tuple(i)]:.6g} want {r_out[tuple(i)]:.6g} bound {lim[tuple(i)]:.3g}")
    lerr = np.abs(lse_np[~dead] - r_lse[~dead])
    llim = (score_err * tmax + 1e-4)[~dead]
    assert np.all(lerr <= llim), f"{label}: lse beyond the bound (max err {lerr.max():.3e})"
    flips = float((bound > 0).mean())
    return float(err[live].max(initial=0.0)), float(lerr.max(initial=0.0)), flips


def _case(wl, label, q_scale, p_scale, with_new=True, rope=None, score_err=SCORE_ERR):
    say(f"[case] {label}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} S={wl.page_size} causal={wl.causal} "
        f"seed={wl.seed} q_scale={q_scale:.4g} p_scale={p_scale:.4g}")
    dc = DeviceCall(wl, with_new=with_new)
    if rope is not None:
        rope = dict(rope, cos_dev=torch.from_numpy(rope["cos"]).cuda(), sin_dev=torch.from_numpy(rope["sin"]).cuda())
    out, lse = _run(dc, q_scale, p_scale, rope)
    torch.cuda.synchronize()
    ref = _oracle(wl, q_scale, p_scale, with_new, rope, score_err=score_err)
    kc, vc = dc.cache_host()
    assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), f"{label}: cache bytes"
    mx, le, fl = check_prob8(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref, label,
                             score_err=score_err)
    say(f"[ok] {label}: max err {mx:.2e} lse {le:.2e} elements with a possible flip {fl:.2%}")
    return out, lse


SMALL = [
    # label, q_lens, new_lens, cache_lens, Hq, Hkv, D, S, causal
    ("prefill_D128", [200, 77], [200, 77], [0, 100], 8, 2, 128, 16, True),
    ("decode_D128", [1, 1, 1, 1], [1, 1, 1, 1], [300, 1, 64, 1000], 8, 2, 128, 16, True),
    ("mixed_D128_S5", [3, 130, 1, 40], [3, 130, 1, 40], [77, 10, 900, 0], 8, 2, 128, 5, True),
    ("noncausal_D128", [65, 1, 33], [65, 1, 33], [64, 7, 0], 4, 4, 128, 32, False),
    ("D64_g8", [1, 90, 3], [1, 90, 3], [500, 40, 12], 16, 2, 64, 16, True),
    ("D64_noncausal_S3", [20, 1], [20, 1], [5, 64], 4, 2, 64, 3, False),
    ("rows_without_keys", [9, 4], [2, 4], [0, 0], 4, 2, 128, 8, True),
    ("empty_sequences", [0, 70, 0, 1], [0, 70, 0, 1], [10, 0, 0, 5], 8, 1, 128, 16, True),
    ("many_tiles_g1", [600], [600], [100], 2, 2, 128, 64, True),
    ("decode_long_32_rows", [4, 1, 2], [4, 1, 2], [8000, 3000, 33], 16, 2, 128, 16, True),
    ("decode_D64_S7", [1, 2, 1], [1, 2, 1], [2000, 77, 5], 8, 4, 64, 7, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("p_scale", [1.0 / 448.0, 2.0 ** -7])
def test_small_cases(case, p_scale):
    label, ql, nl, cl, hq, hkv, d, s, causal = case
    wl = make_custom(q_lens=ql, new_lens=nl, cache_lens=cl, Hq=hq, Hkv=hkv, D=d, page_size=s, causal=causal,
                     cache_dtype="fp8", seed=zlib.crc32(label.encode()) % 1000)
    _case(wl, f"{label} p_scale={p_scale:.4g}", _q_scale(wl), p_scale)


def _exact_scores(wl, seed):
    """The workload with query, key and new-key values drawn from the e4m3 values of [1/8, 1/2)
    (random signs), q_scale = k_scale = v_scale = 1 and scale 1: every score sum is exact."""
    rng = np.random.default_rng(seed)
    window = np.array([c for c in range(0x7F) if 0.125 <= oracle.e4m3fn_decode(np.uint8(c)) < 0.5], np.uint8)

    def codes(shape):
        c = window[rng.integers(0, len(window), size=shape)]
        return (c | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)).astype(np.uint8)

    def bf16_of(c):
        return (oracle.e4m3fn_decode(c).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)

    kc = codes(wl.k_cache.shape)
    vc = oracle.e4m3fn_encode(rng.standard_normal(wl.v_cache.shape).astype(np.float32))
    kn = bf16_of(codes(wl.k_new.shape)) if wl.k_new is not None else None
    vn = bf16_of(oracle.e4m3fn_encode(rng.standard_normal(wl.v_new.shape).astype(np.float32))) \
        if wl.v_new is not None else None
    return dataclasses.replace(wl, q=bf16_of(codes(wl.q.shape)), k_cache=kc, v_cache=vc, k_new=kn, v_new=vn,
                               kv_scale=(np.float32(1), np.float32(1)), scale=1.0)


EXACT = [
    ("prefill_D128", [200, 77], [0, 100], 8, 2, 128, 16, True),
    ("mixed_D128_S5", [3, 130, 1, 40, 1], [77, 10, 900, 0, 1], 8, 2, 128, 5, True),
    ("noncausal_D128_g1", [65, 1], [64, 300], 4, 4, 128, 32, False),
    ("D64_g8", [1, 90, 3], [500, 40, 12], 16, 2, 64, 16, True),
]


@pytest.mark.parametrize("case", EXACT, ids=[c[0] for c in EXACT])
def test_exact_scores(case):
    """Score sums exact on both sides: the probability codes may differ only within the float32
    rounding band, which the oracle's band (no widening) covers."""
    label, ql, cl, hq, hkv, d, s, causal = case
    seed = zlib.crc32(label.encode()) % 1000
    wl = make_custom(q_lens=ql, new_lens=ql, cache_lens=cl, Hq=hq, Hkv=hkv, D=d, page_size=s, causal=causal,
                     cache_dtype="fp8", seed=seed)
    wl = _exact_scores(wl, seed + 1)
    _case(wl, f"exact scores {label}", 1.0, 1.0 / 448.0, score_err=0.0)


@pytest.mark.parametrize("persistent", [0, 1])
def test_persistent_and_one_workgroup_per_item(persistent):
    """The same batch with and without the persistent queues: identical bits (the item's work does
    not depend on which workgroup runs it)."""
    wl = make_custom(q_lens=[1, 300, 1, 40, 2], new_lens=[1, 300, 1, 40, 2], cache_lens=[3000, 100, 700, 50, 9],
                     Hq=8, Hkv=2, D=128, page_size=16, causal=True, cache_dtype="fp8", seed=77)
    vpk.set_option("persistent", persistent)
    try:
        out, lse = _case(wl, f"persistent={persistent}", _q_scale(wl), 1.0 / 448.0, with_new=False)
        vpk.set_option("persistent", 1 - persistent)
        dc = DeviceCall(wl, with_new=False)
        out2, lse2 = _run(dc, _q_scale(wl), 1.0 / 448.0)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        assert torch.equal(lse, lse2)
    finally:
        vpk.set_option("persistent", -1)


def test_kept_scores_equal_a_second_read_of_k():
    """Decode-mode rows of at most 8 packed rows keep their first-pass scores in the workspace, where the
    second pass reads them back instead of the K codes; without room (or with option keep_scores 0) the
    second pass reads K again.  Both recompute nothing differently: the bits must be equal."""
    wl = make_custom(q_lens=[1, 2, 1, 8, 1, 0], new_lens=[1, 2, 1, 8, 1, 0], cache_lens=[3000, 700, 0, 64, 5000, 9],
                     Hq=8, Hkv=2, D=128, page_size=16, causal=True, cache_dtype="fp8", seed=4242)
    q_scale, p_scale = _q_scale(wl), 1.0 / 448.0
    say(f"[case] kept scores vs K read again: rows 4, 8, 4, 32, 4 per kv head, seed {wl.seed}")
    runs = {}
    try:
        dc = DeviceCall(wl)
        out, lse = _run(dc, q_scale, p_scale)                 # the binding's workspace holds the scores
        torch.cuda.synchronize()
        runs["kept"] = (out.clone(), lse.clone(), dc.cache_host())
        vpk.set_option("keep_scores", 0)
        dc = DeviceCall(wl)
        out, lse = _run(dc, q_scale, p_scale)
        torch.cuda.synchronize()
        runs["option off"] = (out.clone(), lse.clone(), dc.cache_host())
        vpk.set_option("keep_scores", 1)
        vpk.AUTO_WORKSPACE = False
        s = torch.cuda.Stream()
        buf = torch.empty(64 * 1024, dtype=torch.uint8, device="cuda")   # no room for the 300 KB of scores
        vpk.set_workspace(buf, stream=s)
        dc = DeviceCall(wl)
        with torch.cuda.stream(s):
            out, lse = vpk.attn_varlen_paged_qkv_prob_fwd(
                dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl, wl.page_size,
                wl.causal, wl.scale, wl.kv_scale, q_scale=q_scale, p_scale=p_scale, host_index=dc.host, stream=s)
        s.synchronize()
        runs["small workspace"] = (out.clone(), lse.clone(), dc.cache_host())
        vpk.set_workspace(None, stream=s)
        s.synchronize()
    finally:
        vpk.set_option("keep_scores", 1)
        vpk.AUTO_WORKSPACE = True
    o0, l0, (k0, v0) = runs["kept"]
    for name in ("option off", "small workspace"):
        o, l, (k, v) = runs[name]
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), f"{name}: out differs from kept scores"
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32)), f"{name}: lse differs from kept scores"
        assert np.array_equal(k, k0) and np.array_equal(v, v0), f"{name}: cache bytes differ"
    ref = _oracle(wl, q_scale, p_scale)
    assert np.array_equal(k0, ref["k_cache"]) and np.array_equal(v0, ref["v_cache"]), "cache bytes"
    mx, le, fl = check_prob8(to_np_out(o0), l0.cpu().numpy().astype(np.float64), ref, "kept scores")
    say(f"[ok] kept scores: bitwise equal to K read again (option and small workspace); max err {mx:.2e}")


def test_saturating_query_codes():
    """A q_scale below amax / 448: the largest query values saturate at +-448 on both sides."""
    wl = make_custom(q_lens=[50, 1], new_lens=[50, 1], cache_lens=[20, 300], Hq=4, Hkv=2, D=128, page_size=16,
                     causal=True, cache_dtype="fp8", seed=8)
    qs = _q_scale(wl, shrink=0.25)
    ref = _oracle(wl, qs, 1 / 448.0)
    assert (ref["q_codes"] & 0x7F == 0x7E).mean() > 0.001
    _case(wl, "saturating q", qs, 1 / 448.0)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotary_embedding(interleaved):
    wl = make_custom(q_lens=[70, 1, 5], new_lens=[70, 1, 5], cache_lens=[30, 200, 0], Hq=8, Hkv=2, D=128,
                     page_size=16, causal=True, cache_dtype="fp8", seed=31)
    cos, sin = rope_tables(512, 64)
    rope = dict(cos=cos, sin=sin, rotary_dim=64, interleaved=interleaved)
    _case(wl, f"rope interleaved={interleaved}", _q_scale(wl), 1 / 448.0, rope=rope)


def test_full_size_mixed_fp8():
    """The mixed prefill + decode workload over its fp8 cache at full size, in the launch
    configuration the bench times: every sequence against the oracle."""
    wl = make_workload("mixed_fp8")
    qs = _q_scale(wl)
    say(f"[case] full size mixed_fp8 QKV-Prob: Tq={wl.Tq} Tn={wl.Tn} pages={wl.num_pages}")
    dc = DeviceCall(wl)
    out, lse = _run(dc, qs, 1 / 448.0)
    torch.cuda.synchronize()
    o_all = to_np_out(out)
    l_all = lse.cpu().numpy().astype(np.float64)
    kc, vc = dc.cache_host()
    say(f"[step] GPU call done, running the oracle on all {wl.B} sequences")
    ref = _oracle(wl, qs, 1 / 448.0)
    assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"])
    mx, le, fl = check_prob8(o_all, l_all, ref, "mixed_fp8 (all sequences)")
    say(f"[ok] mixed_fp8 QKV-Prob: max err {mx:.2e} lse {le:.2e} possible flips {fl:.2%}")


def test_close_to_plain_fp8_attention():
    """The quantisation of Q and P moves the result only by a few e4m3 steps: against the plain
    attention of the same fp8 cache, the error stays within the pages' fp8 tolerance."""
    wl = make_custom(q_lens=[120, 1, 1], new_lens=[120, 1, 1], cache_lens=[200, 900, 40], Hq=8, Hkv=2, D=128,
                     page_size=16, causal=True, cache_dtype="fp8", seed=12)
    dc = DeviceCall(wl)
    out, lse = _run(dc, _q_scale(wl), 1 / 448.0)
    torch.cuda.synchronize()
    plain = oracle.run_call(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q, k_new=wl.k_new, v_new=wl.v_new,
                            cu_seqlens_knew=wl.cu_seqlens_knew, k_cache=wl.k_cache, v_cache=wl.v_cache,
                            block_table=wl.block_table, cache_seqlens=wl.cache_seqlens, page_size=wl.page_size,
                            causal=True, scale=wl.scale, kv_scale=wl.kv_scale, cache_dtype="fp8")
    err = np.abs(to_np_out(out) - plain["out"])
    say(f"[ok] QKV-Prob against plain fp8-KV attention: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() < 0.1 and err.mean() < 1e-2


N_FUZZ = 100


def _fuzz_spec(i):
    """Fuzz case i of the dense tier, over an fp8 cache (the QKV-Prob call needs one)."""
    from test_gpu_fuzz import fuzz_case
    spec = dict(fuzz_case(i), cache_dtype="fp8", seed=9500 + i)
    if spec["page_size"] == 0:
        spec["page_size"] = 16
    return spec


def test_fuzz_specs_reach_the_boundaries():
    specs = [_fuzz_spec(i) for i in range(N_FUZZ)]
    assert {s["D"] for s in specs} == {64, 128}
    assert {s["Hq"] // s["Hkv"] for s in specs} == {1, 4, 8}
    assert {s["causal"] for s in specs} == {True, False}
    rows = [q * (s["Hq"] // s["Hkv"]) for s in specs for q in s["q_lens"]]
    assert 32 in rows and 0 in rows and any(r > 256 for r in rows)


@pytest.mark.parametrize("i", range(N_FUZZ))
def test_fuzz(i):
    spec = _fuzz_spec(i)
    wl = make_custom(**spec)
    p_scale = 1.0 / 448.0 if i % 2 == 0 else 2.0 ** -6
    _case(wl, f"QKV-Prob fuzz {i} q={spec['q_lens']} new={spec['new_lens']} cache={spec['cache_lens']}",
          _q_scale(wl), p_scale, with_new=spec["new_lens"] is not None)
