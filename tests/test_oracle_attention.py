"""Pins for the oracle's attention, append and merge (CPU only).

Each check is independent of the oracle's own code path:
  * facts fixed by the mathematics: probability rows sum to 1; a single visible
    key returns its V row; equal scores return the mean of V; a split of the
    key range merged by LSE equals the one-shot result;
  * structural facts: results do not depend on where pages sit in the pool;
    a dense cache through an identity table equals attention without a cache;
    cache-plus-new attention equals one-shot causal attention over the
    concatenated sequence (this fixes the end-aligned causal diagonal);
  * library special cases: torch's scaled_dot_product_attention in float64
    (grouped-query heads via enable_gqa, causal via is_causal on square
    blocks), torch.logsumexp;
  * brute force: scalar pure-Python loops on the fp32 tiny workload.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attend, merge_partials, run_call, run_workload
from oracle.formats import bf16_bits_to_f64
from synth import make_custom, make_workload


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- math facts

def test_probability_rows_sum_to_one():
    Q, K, V = _rand((7, 4, 16), 1), _rand((11, 2, 16), 2), _rand((11, 2, 16), 3)
    for causal in (False, True):
        _, _, P = attend(Q, K, V, causal, 0.25, return_probs=True)
        s = P.sum(axis=-1)
        assert np.allclose(s, 1.0, atol=1e-12, rtol=0)
        if causal:   # masked entries are exactly zero: row i sees i + Lk - Lq + 1 keys
            for i in range(7):
                assert np.all(P[:, i, i + 11 - 7 + 1:] == 0)
                assert np.all(P[:, i, :i + 11 - 7 + 1] > 0)


def test_single_visible_key_returns_its_value_row():
    # causal, no cached prefix, Lq = Lk: query 0 sees only key 0
    Q, K, V = _rand((5, 4, 8), 4), _rand((5, 2, 8), 5), _rand((5, 2, 8), 6)
    out, lse = attend(Q, K, V, True, 0.3)
    for h in range(4):
        kvh = h // 2
        assert np.array_equal(out[0, h], V[0, kvh])
        assert lse[h, 0] == pytest.approx(0.3 * float(Q[0, h] @ K[0, kvh]), abs=1e-14)


def test_equal_scores_return_mean_of_visible_values():
    Lq, Lk = 4, 9
    Q = np.zeros((Lq, 2, 8))
    K, V = _rand((Lk, 1, 8), 7), _rand((Lk, 1, 8), 8)
    out, lse = attend(Q, K, V, True, 0.5)
    for i in range(Lq):
        n = i + Lk - Lq + 1
        for h in range(2):
            assert np.allclose(out[i, h], V[:n, 0].mean(axis=0), atol=1e-14, rtol=0)
            assert lse[h, i] == pytest.approx(math.log(n), abs=1e-14)


def test_closed_form_two_keys():
    # scores [1, 0] -> p = [e, 1] / (e + 1)
    Q = np.array([[[1.0, 0.0]]])
    K = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    V = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])
    out, lse = attend(Q, K, V, False, 1.0)
    e = math.e
    assert np.allclose(out[0, 0], [(e * 1 + 3) / (e + 1), (e * 2 + 4) / (e + 1)], atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(e + 1), abs=1e-15)


def test_no_visible_key_gives_zero_and_minus_inf():
    # causal with Lq > Lk: the first Lq - Lk queries see nothing
    Q, K, V = _rand((6, 2, 8), 9), _rand((2, 2, 8), 10), _rand((2, 2, 8), 11)
    out, lse = attend(Q, K, V, True, 0.5)
    assert np.all(out[:4] == 0) and np.all(np.isneginf(lse[:, :4]))
    assert np.all(np.isfinite(lse[:, 4:]))
    out0, lse0 = attend(Q, K[:0], V[:0], False, 0.5)
    assert np.all(out0 == 0) and np.all(np.isneginf(lse0))


@pytest.mark.parametrize("causal", [False, True])
def test_split_merge_equals_one_shot(causal):
    Lq, Lk = 6, 23
    Q, K, V = _rand((Lq, 4, 16), 12), _rand((Lk, 2, 16), 13), _rand((Lk, 2, 16), 14)
    out, lse = attend(Q, K, V, causal, 0.2)
    for cuts in ([0, 23], [0, 8, 23], [0, 3, 4, 17, 20, 23], [0, 0, 23]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, l = attend(Q, K, V, causal, 0.2, key_range=(a, b))
            parts.append((o, l))
        for h in range(4):
            mo, ml = merge_partials([(o[:, h], l[h]) for o, l in parts])
            assert np.allclose(mo, out[:, h], atol=1e-12, rtol=0)
            assert np.allclose(ml, lse[h], atol=1e-12, rtol=0)


# ---------------------------------------------------------- library special cases

@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_matches_torch_sdpa_fp64(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    for Lq, Lk, causal in ((9, 9, True), (5, 13, False), (13, 13, False)):
        Q = rng.standard_normal((Lq, Hq, 32))
        K = rng.standard_normal((Lk, Hkv, 32))
        V = rng.standard_normal((Lk, Hkv, 32))
        out, lse = attend(Q, K, V, causal, 0.17)
        tq = torch.from_numpy(Q).permute(1, 0, 2)[None]
        tk = torch.from_numpy(K).permute(1, 0, 2)[None]
        tv = torch.from_numpy(V).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.17,
                                             enable_gqa=(Hq != Hkv))
        assert np.allclose(out, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
        # lse against torch.logsumexp of the scores (kv head via repeat_interleave)
        kk = torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=1)
        s = 0.17 * torch.einsum("ihd,jhd->hij", torch.from_numpy(Q), kk)
        if causal:
            s = s.masked_fill(~torch.ones(Lq, Lk, dtype=torch.bool).tril(), -math.inf)
        assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


def test_end_aligned_causal_mask_matches_tril_offset():
    # torch.tril with diagonal Lk - Lq keeps exactly the keys j <= i + Lk - Lq
    Lq, Lk = 5, 12
    Q, K, V = _rand((Lq, 2, 16), 15), _rand((Lk, 2, 16), 16), _rand((Lk, 2, 16), 17)
    out, _ = attend(Q, K, V, True, 0.25)
    mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)
    ref = F.scaled_dot_product_attention(torch.from_numpy(Q).permute(1, 0, 2),
                                         torch.from_numpy(K).permute(1, 0, 2),
                                         torch.from_numpy(V).permute(1, 0, 2),
                                         attn_mask=mask, scale=0.25)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


# ------------------------------------------------------------- paging / cache facts

def _call(wl, **over):
    kw = dict(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q, k_new=wl.k_new, v_new=wl.v_new,
              cu_seqlens_knew=wl.cu_seqlens_knew, k_cache=wl.k_cache, v_cache=wl.v_cache,
              block_table=wl.block_table, cache_seqlens=wl.cache_seqlens,
              page_size=wl.page_size, causal=wl.causal, scale=wl.scale,
              kv_scale=wl.kv_scale, cache_dtype=wl.cache_dtype)
    kw.update(over)
    return run_call(**kw)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_page_permutation_invariance(cache_dtype):
    wl = make_custom(q_lens=[3, 1, 6], new_lens=[3, 1, 6], cache_lens=[9, 0, 14], Hq=4, Hkv=2,
                     D=16, page_size=4, cache_dtype=cache_dtype, seed=21)
    base = _call(wl)
    rng = np.random.default_rng(5)
    P = wl.k_cache.shape[0]
    perm = rng.permutation(P)              # new position of old page p is perm[p]
    kc = np.empty_like(wl.k_cache); vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache; vc[perm] = wl.v_cache
    bt = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    moved = _call(wl, k_cache=kc, v_cache=vc, block_table=bt)
    assert np.array_equal(base["out"], moved["out"])
    assert np.array_equal(base["lse"], moved["lse"])
    assert np.array_equal(base["k_cache"][wl.block_table[0, 0]], moved["k_cache"][bt[0, 0]])


def test_dense_identity_table_equals_no_cache():
    # each sequence owns one page holding all its keys: the paged call must equal
    # attention over the same keys passed as new tokens without any cache
    lens = [5, 8, 3]
    S = 8
    wl = make_custom(q_lens=lens, new_lens=lens, cache_lens=[0, 0, 0], Hq=4, Hkv=2, D=16,
                     page_size=S, cache_dtype="bf16", seed=22, pool_factor=1.0)
    assert wl.k_cache.shape[0] == 3
    ident = np.arange(3, dtype=np.int32)[:, None]
    kc = np.zeros_like(wl.k_cache); vc = np.zeros_like(wl.v_cache)
    paged = _call(wl, k_cache=kc, v_cache=vc, block_table=ident)
    plain = _call(wl, k_cache=None, v_cache=None, block_table=None, cache_seqlens=None,
                  cache_dtype=None)
    assert np.array_equal(paged["out"], plain["out"])
    assert np.array_equal(paged["lse"], plain["lse"])


@pytest.mark.parametrize("lc,ln", [(7, 3), (0, 5), (12, 1), (4, 0)])
def test_cache_plus_new_equals_one_shot(lc, ln):
    # one sequence: cached prefix of lc tokens plus ln new tokens (q_len = ln)
    # must equal causal attention over all lc + ln tokens with every token as a
    # query, restricted to the last ln query rows
    Hq, Hkv, D, S = 4, 2, 16, 4
    full = make_custom(q_lens=[lc + ln], new_lens=[lc + ln], cache_lens=[0], Hq=Hq, Hkv=Hkv,
                       D=D, page_size=S, cache_dtype=None, seed=23)
    one = _call(full)
    # build the chunked call from the same tokens
    need = -(-(lc + ln) // S)
    pool = need + 2
    kc = np.zeros((pool, S, Hkv, D), np.uint16); vc = np.zeros_like(kc)
    bt = np.array([np.random.default_rng(1).permutation(pool)[:need]], np.int32)
    for t in range(lc):
        kc[bt[0, t // S], t % S] = full.k_new[t]
        vc[bt[0, t // S], t % S] = full.v_new[t]
    q = full.q[lc:]
    chunk = run_call(q=q, cu_seqlens_q=np.array([0, ln], np.int32),
                     k_new=full.k_new[lc:] if ln else None, v_new=full.v_new[lc:] if ln else None,
                     cu_seqlens_knew=np.array([0, ln], np.int32) if ln else None,
                     k_cache=kc, v_cache=vc, block_table=bt,
                     cache_seqlens=np.array([lc], np.int32), page_size=S, causal=True,
                     scale=full.scale, cache_dtype="bf16")
    assert np.allclose(chunk["out"], one["out"][lc:], atol=1e-12, rtol=0)
    assert np.allclose(chunk["lse"], one["lse"][:, lc:], atol=1e-12, rtol=0)


def test_append_touches_exactly_the_new_slots_bf16():
    wl = make_custom(q_lens=[2, 3], new_lens=[2, 3], cache_lens=[5, 4], Hq=4, Hkv=2, D=8,
                     page_size=4, seed=24)
    kc, vc = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, wl.k_cache, wl.v_cache,
                           wl.block_table, wl.cache_seqlens, 4, "bf16")
    # flat slot index page * S + slot, computed here from the block table
    flat_k = kc.reshape(-1, 2, 8); orig = wl.k_cache.reshape(-1, 2, 8)
    touched = set()
    j = 0
    for b, (lc, ln) in enumerate([(5, 2), (4, 3)]):
        for t in range(lc, lc + ln):
            idx = int(wl.block_table[b][t // 4]) * 4 + t % 4
            touched.add(idx)
            assert np.array_equal(flat_k[idx], wl.k_new[j])
            assert np.array_equal(vc.reshape(-1, 2, 8)[idx], wl.v_new[j])
            j += 1
    for idx in range(flat_k.shape[0]):
        if idx not in touched:
            assert np.array_equal(flat_k[idx], orig[idx])


def test_append_fp8_codes_and_dequant_error():
    wl = make_custom(q_lens=[3], new_lens=[3], cache_lens=[2], Hq=2, Hkv=1, D=32,
                     page_size=2, cache_dtype="fp8", seed=25)
    kc, _ = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, wl.k_cache, wl.v_cache,
                          wl.block_table, wl.cache_seqlens, 2, "fp8", wl.kv_scale)
    ks = np.float32(wl.kv_scale[0])
    for j in range(3):
        t = 2 + j
        codes = kc[wl.block_table[0, t // 2], t % 2]
        x = bf16_bits_to_f64(wl.k_new[j])
        # torch's narrowing cast of the fp32 product gives the same bytes (|x/s| <= 448 here)
        prod = (x.astype(np.float32) * (np.float32(1) / ks)).astype(np.float32)
        tcodes = torch.from_numpy(prod).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, tcodes)
        # the dequantised value is within half a step of x: relative 2^-4 for normals
        deq = oracle.e4m3fn_decode(codes) * np.float64(ks)
        assert np.all(np.abs(deq - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * ks) + 1e-12)


def test_append_fp8_special_values_keep_the_input_sign():
    """Specials through the fp8 append, against the e4m3fn bit definition (sign bit 7, exponent
    bits 6..3, mantissa bits 2..0; S.1111.111 is NaN; 448 = 0.1111.110 the largest finite value):
    a NaN is stored as the NaN code of its own sign, infinities and values past 448 saturate to
    +-448 with their sign, and -0 keeps its sign.  The pages leave NaN handling open; the reading
    taken is that the stored code carries the input's sign bit (1/scale > 0 cannot change it)."""
    specials = {0x7FC0: 0x7F, 0xFFC0: 0xFF, 0x7F81: 0x7F, 0xFF81: 0xFF, 0x7FFF: 0x7F, 0xFFFF: 0xFF,
                0x7F80: 0x7E, 0xFF80: 0xFE, 0x0000: 0x00, 0x8000: 0x80, 0x4580: 0x7E, 0xC580: 0xFE}
    bits = np.array(list(specials), np.uint16)            # 12 values: one row of one token
    expect = np.array(list(specials.values()), np.uint8)
    for scale in (np.float32(1.0), np.float32(0.25)):
        k_new = np.zeros((1, 1, 16), np.uint16)
        k_new[0, 0, :12] = bits
        cache = np.full((1, 4, 1, 16), 0x11, np.uint8)
        kc, vc = oracle.append(k_new, k_new.copy(), np.array([0, 1], np.int32), cache, cache.copy(),
                               np.array([[0]], np.int32), np.array([2], np.int32), 4, "fp8", (scale, scale))
        got = kc[0, 2, 0, :12]
        # with scale 1/4 every finite non-zero value is multiplied by 4 and still saturates or stays
        # zero; NaN and the sign of zero do not depend on the scale
        assert np.array_equal(got, expect), (scale, [hex(x) for x in got])
        assert np.array_equal(kc[0, [0, 1, 3]], cache[0, [0, 1, 3]])   # other slots untouched


# ------------------------------------------------------------------- brute force

def _brute(q, k, v, lq, lk, causal, scale, g):
    """Scalar loops over python floats: one (query, head) at a time."""
    Hq, D = len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(lq)]
    lse = [[-math.inf] * lq for _ in range(Hq)]
    for i in range(lq):
        for h in range(Hq):
            kh = h // g
            scores = []
            for j in range(lk):
                if causal and j > i + lk - lq:
                    continue
                s = 0.0
                for d in range(D):
                    s += float(q[i][h][d]) * float(k[j][kh][d])
                scores.append((j, s * scale))
            if not scores:
                continue
            mx = max(s for _, s in scores)
            w = [(j, math.exp(s - mx)) for j, s in scores]
            tot = sum(x for _, x in w)
            for d in range(D):
                out[i][h][d] = sum(x * float(v[j][kh][d]) for j, x in w) / tot
            lse[h][i] = mx + math.log(tot)
    return np.array(out), np.array(lse)


def test_tiny_fp32_against_brute_force():
    wl = make_workload("tiny")
    f = wl.f32
    B = wl.B
    # the fp32 originals, laid out through the same block table as the bf16 cache
    S = wl.page_size
    kc = np.zeros(wl.k_cache.shape, np.float32); vc = np.zeros_like(kc)
    cl = wl.cache_lens()
    for b in range(B):
        for t in range(int(cl[b])):
            kc[wl.block_table[b, t // S], t % S] = f["k"][f["cu_k"][b] + t]
            vc[wl.block_table[b, t // S], t % S] = f["v"][f["cu_k"][b] + t]
    new_rows = np.concatenate([np.arange(f["cu_k"][b] + cl[b], f["cu_k"][b + 1]) for b in range(B)])
    res = run_call(q=f["q"], cu_seqlens_q=wl.cu_seqlens_q, k_new=f["k"][new_rows],
                   v_new=f["v"][new_rows], cu_seqlens_knew=wl.cu_seqlens_knew, k_cache=kc,
                   v_cache=vc, block_table=wl.block_table, cache_seqlens=wl.cache_seqlens,
                   page_size=S, causal=True, scale=wl.scale, cache_dtype="f32",
                   q_dtype="f32", new_dtype="f32")
    for b in range(B):
        s, e = wl.cu_seqlens_q[b], wl.cu_seqlens_q[b + 1]
        lk = int(f["cu_k"][b + 1] - f["cu_k"][b])
        ks = f["k"][f["cu_k"][b]:f["cu_k"][b + 1]]
        vs = f["v"][f["cu_k"][b]:f["cu_k"][b + 1]]
        bo, bl = _brute(f["q"][s:e].tolist(), ks.tolist(), vs.tolist(), e - s, lk, True,
                        wl.scale, wl.Hq // wl.Hkv)
        assert np.allclose(res["out"][s:e], bo, atol=1e-12, rtol=0)
        assert np.allclose(res["lse"][:, s:e], bl, atol=1e-12, rtol=0)


def test_tiny_workload_shape_matches_its_description():
    wl = make_workload("tiny")
    assert wl.B == 2 and wl.Hq == 2 and wl.Hkv == 2 and wl.D == 64 and wl.page_size == 4
    assert wl.q_lens().tolist() == [3, 5] and wl.new_lens().tolist() == [3, 5]
    assert wl.cache_lens().tolist() == [7, 0]
    assert sorted(wl.block_table.ravel().tolist()) == list(range(6))
    assert wl.scale == pytest.approx(1 / 8)


def test_run_workload_rows_against_attend_rows():
    wl = make_workload("tiny")
    full = run_workload(wl)
    K, V = oracle.sequence_kv(0, k_new=wl.k_new, v_new=wl.v_new, cu_seqlens_knew=wl.cu_seqlens_knew,
                              k_cache=full["k_cache"], v_cache=full["v_cache"],
                              block_table=wl.block_table, cache_seqlens=wl.cache_seqlens,
                              page_size=wl.page_size, cache_dtype="bf16")
    Q = bf16_bits_to_f64(wl.q[0:3])
    o, l = oracle.attend_rows(Q, K, V, True, wl.scale, rows=[2, 0])
    assert np.array_equal(o[0], full["out"][2]) and np.array_equal(o[1], full["out"][0])
    assert np.array_equal(l[:, 0], full["lse"][:, 2])
