"""GPU parity of attn_varlen_paged_rope_fwd (rotary embedding of the query rows
and the new key rows, then append and attention) against the oracle's
``run_call(rope=...)``.

* cache bytes after the append (the turned keys, bf16 or fp8 codes): bit-exact;
* attention values: the tolerances of the other parity tests;
* q and k_new are left unchanged by the call.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_paged_kv_amd as vpk
from synth import make_custom, make_workload, rope_tables

from gpu_util import DeviceCall, check_attention, say, to_np_out

pytestmark = pytest.mark.gpu


def _oracle(wl, with_new, rope, seqs=None):
    return oracle.run_call(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q,
                           k_new=wl.k_new if with_new else None, v_new=wl.v_new if with_new else None,
                           cu_seqlens_knew=wl.cu_seqlens_knew if with_new else None,
                           k_cache=wl.k_cache, v_cache=wl.v_cache, block_table=wl.block_table,
                           cache_seqlens=wl.cache_seqlens, page_size=wl.page_size, causal=wl.causal,
                           scale=wl.scale, kv_scale=wl.kv_scale, cache_dtype=wl.cache_dtype, seqs=seqs,
                           rope=rope)


def _rope_call(dc, cos_d, sin_d, R, inter):
    wl = dc.wl
    return vpk.attn_varlen_paged_rope_fwd(
        dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl, wl.page_size,
        wl.causal, wl.scale, wl.kv_scale if dc.fp8 else None, rope_cos=cos_d, rope_sin=sin_d, rotary_dim=R,
        interleaved=inter, host_index=dc.host)


CASES = [
    # label, q_lens, new_lens, cache_lens, Hq, Hkv, D, S, causal, cache, rotary_dim, interleaved
    ("mixed_bf16_R128", [1, 37, 1, 300, 1], [1, 37, 1, 300, 1], [500, 40, 1000, 0, 77], 8, 2, 128, 16, True,
     "bf16", 128, False),
    ("mixed_fp8_R64_interleaved", [3, 1, 70, 1], [3, 1, 70, 1], [41, 300, 9, 2000], 8, 2, 128, 16, True, "fp8",
     64, True),
    ("no_cache_D64_R32", [200, 3, 90], [200, 3, 90], [0, 0, 0], 4, 4, 64, 0, True, None, 32, False),
    ("cache_only_R128_interleaved", [1, 1, 3], None, [300, 1200, 64], 8, 2, 128, 64, True, "bf16", 128, True),
    ("noncausal_S5_D64_R48", [3, 70, 1], [3, 70, 1], [10, 0, 257], 4, 1, 64, 5, False, "bf16", 48, False),
    # half-split pairs three k-steps apart (rotary_dim 96), turned in the kernels, decode rows between
    ("mixed_fp8_R96", [1, 50, 1, 1, 90], [1, 50, 1, 1, 90], [700, 20, 0, 64, 300], 8, 2, 128, 16, True, "fp8",
     96, False),
    ("prefill_bf16_R64_S64", [130, 257, 8], [130, 257, 8], [33, 0, 500], 8, 2, 128, 64, True, "bf16", 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_against_oracle(case):
    label, ql, nl, cl, Hq, Hkv, D, S, causal, cache, R, inter = case
    wl = make_custom(q_lens=ql, new_lens=nl, cache_lens=cl, Hq=Hq, Hkv=Hkv, D=D, page_size=S, causal=causal,
                     cache_dtype=cache, seed=61 + len(label))
    with_new = wl.k_new is not None
    say(f"[case] rope {label}")
    max_pos = int(wl.kv_lens().max()) + 3
    cos, sin = rope_tables(max_pos, R)
    dc = DeviceCall(wl, with_new=with_new)
    q0 = dc.q.clone()
    k0 = dc.k_new.clone() if with_new else None
    out, lse = _rope_call(dc, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), R, inter)
    torch.cuda.synchronize()
    assert torch.equal(dc.q, q0) and (k0 is None or torch.equal(dc.k_new, k0)), "inputs were modified"
    ref = _oracle(wl, with_new, dict(cos=cos, sin=sin, rotary_dim=R, interleaved=inter))
    kind = "fp8" if wl.cache_dtype == "fp8" else "bf16"
    errs = check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"], kind,
                           label=label)
    kc, vc = dc.cache_host()
    if kc is not None:
        assert np.array_equal(kc, ref["k_cache"]), f"{label}: k_cache bytes differ"
        assert np.array_equal(vc, ref["v_cache"]), f"{label}: v_cache bytes differ"
    say(f"[ok] rope {label}: max {errs[0]:.2e} mean {errs[1]:.2e} lse {errs[2]:.2e}")


def test_rope_full_size_mixed_fp8():
    """The mixed prefill + decode batch over an fp8 cache (64 sequences, 6.5k new
    tokens, up to 8k keys) with rotary embedding: every appended byte, and the
    attention of every sequence."""
    wl = make_workload("mixed_fp8")
    R = wl.D
    cos, sin = rope_tables(int(wl.kv_lens().max()) + 1, R)
    say(f"[case] rope full size mixed_fp8: Tq={wl.Tq} Tn={wl.Tn}")
    dc = DeviceCall(wl)
    out, lse = _rope_call(dc, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), R, False)
    torch.cuda.synchronize()
    ref = _oracle(wl, True, dict(cos=cos, sin=sin, rotary_dim=R, interleaved=False))
    kc, vc = dc.cache_host()
    assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), "cache bytes differ"
    o_all, l_all = to_np_out(out), lse.cpu().numpy().astype(np.float64)
    errs = check_attention(o_all, l_all, ref["out"], ref["lse"], "fp8", label="rope mixed_fp8 (all sequences)")
    for b in range(wl.B):
        s, e = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        check_attention(o_all[s:e], l_all[:, s:e], ref["out"][s:e], ref["lse"][:, s:e], "fp8",
                        label=f"rope mixed_fp8 seq {b}")
    say(f"[ok] rope full size mixed_fp8: all {wl.B} sequences; max {errs[0]:.2e} mean {errs[1]:.2e} "
        f"lse {errs[2]:.2e}")


N_FUZZ = 80


def _fuzz_rope(i):
    """Fuzz case i of the dense tier with a rotary dim (a multiple of 16 up to the head dim) and a pairing."""
    from test_gpu_fuzz import fuzz_case
    spec = fuzz_case(i)
    if i % 4:
        # three draws in four made valid: no sequence with more query rows than keys
        nl = spec["new_lens"]
        for b, q in enumerate(spec["q_lens"]):
            lk = spec["cache_lens"][b] + (nl[b] if nl else 0)
            if q > lk:
                if spec["cache_dtype"]:
                    spec["cache_lens"][b] += q - lk
                else:
                    nl[b] = q
    rng = np.random.default_rng(9700 + i)
    R = 16 * int(rng.integers(1, spec["D"] // 16 + 1))
    return spec, R, bool(rng.integers(0, 2))


def test_rope_fuzz_draws_reach_both_pairings_and_dims():
    draws = [_fuzz_rope(i) for i in range(N_FUZZ)]
    assert {inter for _, _, inter in draws} == {True, False}
    assert any(R == s["D"] for s, R, _ in draws) and any(R % 32 == 16 for _, R, _ in draws)


@pytest.mark.parametrize("i", range(N_FUZZ))
def test_rope_fuzz(i):
    """The dense tier's draws with rotary embedding: against the oracle, or, where a sequence has more query
    rows than keys (its first rows would have negative positions), refused before anything is enqueued."""
    spec, R, inter = _fuzz_rope(i)
    wl = make_custom(**spec)
    with_new = wl.k_new is not None
    cos, sin = rope_tables(int(wl.kv_lens().max()) + 3, R)
    dc = DeviceCall(wl, with_new=with_new)
    if np.any(wl.q_lens() > wl.kv_lens()):
        kc0, vc0 = dc.cache_host()
        with pytest.raises(vpk.VpkError) as ei:
            _rope_call(dc, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), R, inter)
        assert ei.value.status == 1, ei.value   # VPK_ERROR_INVALID_VALUE
        kc1, vc1 = dc.cache_host()
        if kc0 is not None:
            assert np.array_equal(kc0, kc1) and np.array_equal(vc0, vc1), "a refused call wrote the cache"
        return
    out, lse = _rope_call(dc, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), R, inter)
    torch.cuda.synchronize()
    ref = _oracle(wl, with_new, dict(cos=cos, sin=sin, rotary_dim=R, interleaved=inter))
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    "fp8" if wl.cache_dtype == "fp8" else "bf16", label=f"rope fuzz {i} R={R} inter={inter}")
    kc, vc = dc.cache_host()
    if kc is not None:
        assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), f"rope fuzz {i}: cache"
