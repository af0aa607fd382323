"""fp8 cache, batches of decode-mode sequences only (at most 32 packed rows each, head_dim 128).

Such a call launches no standalone append: the decode-mode item whose key
range holds a new token forms the token's codes from k_new / v_new with the
append's encoder, uses them, and stores them into the cache.  The cache bytes
must still be the oracle's append bit for bit, attention within the fp8
tolerances, and the prepared and allocation-free entry points bitwise equal
to the direct call.  A new token on a page id past num_pages is dropped and
flagged, and its slot reads as zero, as with the standalone append.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_paged_kv_amd as vpk
from gpu_util import DeviceCall, check_attention, dev_bf16, dev_i32, dev_u8, run_and_check, say, to_np_out
from synth import make_custom

pytestmark = pytest.mark.gpu

CASES = [
    # label, q_lens, cache_lens, Hq, Hkv, S
    ("q1_g4_S16", [1] * 12, [0, 15, 16, 31, 1, 2000, 700, 63, 64, 3000, 5, 128], 32, 8, 16),
    ("q1to8_g4_S5", [1, 2, 8, 3, 1], [0, 44, 100, 5, 999], 8, 2, 5),
    ("g1_q32_S16", [32, 1, 7], [64, 10, 0], 2, 2, 16),
]


def _wl(case, seed):
    label, ql, cl, hq, hkv, S = case
    return make_custom(q_lens=ql, new_lens=ql, cache_lens=cl, Hq=hq, Hkv=hkv, D=128, page_size=S,
                       causal=True, cache_dtype="fp8", seed=seed)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.fixture(autouse=True)
def _restore():
    yield
    vpk.set_option("force_splits", 0)


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_items_store_their_tokens(case, splits):
    vpk.set_option("force_splits", splits)
    wl = _wl(case, seed=300 + splits)
    dc, out, lse = run_and_check(wl, f"{case[0]} splits {splits}")
    kc, vc = dc.cache_host()
    # prepared plan and allocation-free entry: bitwise the direct call (fresh caches each)
    dp = DeviceCall(wl)
    plan = vpk.Plan(wl.cu_seqlens_q, wl.Hq, wl.Hkv, wl.D, cu_seqlens_knew=wl.cu_seqlens_knew,
                    cache_seqlens=wl.cache_seqlens, block_table=wl.block_table, page_size=wl.page_size,
                    num_pages=wl.k_cache.shape[0], max_pages_per_seq=wl.block_table.shape[1],
                    cache_dtype="fp8", causal=wl.causal)
    o2, l2 = plan.run(dp.q, dp.k_new, dp.v_new, dp.k_cache, dp.v_cache, dp.bt, scale=wl.scale,
                      kv_scale=wl.kv_scale)
    torch.cuda.synchronize()
    dn = DeviceCall(wl)
    o3 = torch.empty_like(dn.q)
    l3 = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dn.q.device)
    vpk.attn_varlen_paged_fwd_noalloc(
        dn.q, dn.cu_q, dn.k_new, dn.v_new, dn.cu_kn, dn.k_cache, dn.v_cache, dn.bt, dn.cl, wl.page_size,
        wl.causal, wl.scale, wl.kv_scale, out=o3, lse=l3, host_index=dn.host)
    torch.cuda.synchronize()
    for name, o, l, d in (("prepared", o2, l2, dp), ("allocation-free", o3, l3, dn)):
        assert np.array_equal(_bits(o), _bits(out)), f"{name}: out differs from the direct call"
        assert np.array_equal(_bits(l), _bits(lse)), f"{name}: lse differs from the direct call"
        k2, v2 = d.cache_host()
        assert np.array_equal(k2, kc) and np.array_equal(v2, vc), f"{name}: cache bytes differ"
    say(f"[ok] {case[0]} splits {splits}: prepared and allocation-free runs bitwise equal")


def test_decode_page_guard():
    """A new token whose page id is past num_pages: dropped, flagged, and its slot reads as zero."""
    wl = make_custom(q_lens=[1, 1, 2], new_lens=[1, 1, 2], cache_lens=[20, 16, 40], Hq=16, Hkv=4, D=128,
                     page_size=16, causal=True, cache_dtype="fp8", seed=77)
    S, P = wl.page_size, wl.num_pages
    spare = 4
    fill = np.random.default_rng(6)
    ext_k = np.concatenate([wl.k_cache, fill.integers(0, 120, (spare,) + wl.k_cache.shape[1:]).astype(np.uint8)])
    ext_v = np.concatenate([wl.v_cache, fill.integers(0, 120, (spare,) + wl.v_cache.shape[1:]).astype(np.uint8)])
    bt = wl.block_table.copy()
    bt[0, 1] = P + 1   # sequence 0: keys 16..19 cached, key 20 new
    bt[1, 1] = P + 2   # sequence 1: key 16 new
    kc_d, vc_d = dev_u8(ext_k), dev_u8(ext_v)
    say(f"[case] fp8 decode page guard: num_pages {P}, ids {P + 1} and {P + 2} in the spare range")
    vpk.device_error()
    out, lse = vpk.attn_varlen_paged_fwd(
        dev_bf16(wl.q), dev_i32(wl.cu_seqlens_q), dev_bf16(wl.k_new), dev_bf16(wl.v_new),
        dev_i32(wl.cu_seqlens_knew), kc_d[:P], vc_d[:P], dev_i32(bt), dev_i32(wl.cache_seqlens), S, wl.causal,
        wl.scale, wl.kv_scale,
        host_index=dict(cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_knew=wl.cu_seqlens_knew,
                        cache_seqlens=wl.cache_seqlens))
    torch.cuda.synchronize()
    assert vpk.device_error() == 1, "the device error flag was not raised"
    rk, rv = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, ext_k, ext_v, bt, wl.cache_seqlens, S, "fp8",
                           wl.kv_scale)
    rk[P:], rv[P:] = ext_k[P:], ext_v[P:]
    assert np.array_equal(kc_d.cpu().numpy(), rk) and np.array_equal(vc_d.cpu().numpy(), rv), "cache bytes differ"
    Q = oracle.bf16_bits_to_f64(wl.q)
    ref_out = np.zeros((wl.Tq, wl.Hq, wl.D))
    ref_lse = np.full((wl.Hq, wl.Tq), -np.inf)
    for b in range(wl.B):
        K, V = oracle.sequence_kv(b, k_new=wl.k_new, v_new=wl.v_new, cu_seqlens_knew=wl.cu_seqlens_knew,
                                  k_cache=rk, v_cache=rv, block_table=bt, cache_seqlens=wl.cache_seqlens,
                                  page_size=S, cache_dtype="fp8", kv_scale=wl.kv_scale)
        K, V = K.copy(), V.copy()
        if bt[b, 1] >= P:
            K[16:32], V[16:32] = 0.0, 0.0
        s0, e0 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        o, l = oracle.attend(Q[s0:e0], K, V, wl.causal, wl.scale)
        ref_out[s0:e0], ref_lse[:, s0:e0] = o, l
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, "fp8",
                    label="fp8 decode page guard")
    say("[ok] fp8 decode page guard: flagged, dropped, read as zero")


def test_device_scales():
    """A prepared run with the scales in device memory: bitwise the direct call with the same scales on
    the host (the decode-mode items form the reciprocals of the device scales as the append does)."""
    wl = _wl(CASES[1], seed=401)
    ks = (np.asarray(wl.kv_scale, np.float32) * np.float32(1.25)).astype(np.float32)
    dd = DeviceCall(wl)
    out, lse = vpk.attn_varlen_paged_fwd(dd.q, dd.cu_q, dd.k_new, dd.v_new, dd.cu_kn, dd.k_cache, dd.v_cache,
                                         dd.bt, dd.cl, wl.page_size, wl.causal, wl.scale,
                                         (float(ks[0]), float(ks[1])), host_index=dd.host)
    torch.cuda.synchronize()
    dp = DeviceCall(wl)
    plan = vpk.Plan(wl.cu_seqlens_q, wl.Hq, wl.Hkv, wl.D, cu_seqlens_knew=wl.cu_seqlens_knew,
                    cache_seqlens=wl.cache_seqlens, block_table=wl.block_table, page_size=wl.page_size,
                    num_pages=wl.k_cache.shape[0], max_pages_per_seq=wl.block_table.shape[1],
                    cache_dtype="fp8", causal=wl.causal)
    o2, l2 = plan.run(dp.q, dp.k_new, dp.v_new, dp.k_cache, dp.v_cache, dp.bt, scale=wl.scale,
                      kv_scale=torch.from_numpy(ks.copy()).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o2), _bits(out)) and np.array_equal(_bits(l2), _bits(lse)), "out / lse differ"
    k1, v1 = dd.cache_host()
    k2, v2 = dp.cache_host()
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2), "cache bytes differ"
    say("[ok] fp8 decode, device scales: bitwise the direct call")
