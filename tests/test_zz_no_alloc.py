"""The allocation-free entry point (attn_varlen_paged_fwd_noalloc) against
attn_varlen_paged_fwd, through the C ABI: two calls in a row, the second with
a smaller batch, each bitwise equal to the direct call on the same inputs and
within the oracle's tolerances, with the library's own memory unchanged."""
import numpy as np
import pytest
import torch

import varlen_paged_kv_amd as vpk
from synth import make_custom
from varlen_paged_kv_amd import _lib

from gpu_util import DeviceCall, check_attention, oracle_full, say, to_np_out

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _noalloc(dc):
    wl = dc.wl
    out = torch.empty_like(dc.q)
    lse = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dc.q.device)
    return vpk.attn_varlen_paged_fwd_noalloc(
        dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl, wl.page_size,
        wl.causal, wl.scale, wl.kv_scale if dc.fp8 else None, out=out, lse=lse, host_index=dc.host)


@pytest.fixture(autouse=True)
def _one_launch():
    # the allocation-free call runs a batch with both kinds of items in one
    # launch (it has no side stream for two grids); the direct call it is
    # compared with bit for bit does the same under this option
    vpk.set_option("mixed_grid", 1)
    yield
    vpk.set_option("mixed_grid", -1)


def test_noalloc_two_calls_match_the_direct_call():
    cases = [
        # a mixed batch over an fp8 cache: both grids, split parts (merge pass) from the scratch
        ("mixed_fp8", make_custom(q_lens=[1, 37, 1, 300, 1, 1], new_lens=[1, 37, 1, 300, 1, 1],
                                  cache_lens=[3000, 40, 1000, 0, 77, 2500], Hq=8, Hkv=2, D=128, page_size=16,
                                  causal=True, cache_dtype="fp8", seed=81)),
        # then a smaller batch (bf16 cache, head_dim 64): the scratch keeps the first call's contents
        ("small_bf16", make_custom(q_lens=[3, 1], new_lens=[3, 1], cache_lens=[20, 500], Hq=4, Hkv=2, D=64,
                                   page_size=4, causal=True, cache_dtype="bf16", seed=82)),
    ]
    for label, wl in cases:
        dc = DeviceCall(wl)
        say(f"[case] noalloc {label}: B={wl.B} Tq={wl.Tq}")
        ref_out, ref_lse = dc.run()
        torch.cuda.synchronize()
        mem0 = vpk.library_memory()
        out, lse = _noalloc(dc)
        torch.cuda.synchronize()
        assert vpk.library_memory() == mem0, "the allocation-free call changed the library's own memory"
        assert np.array_equal(_bits(out), _bits(ref_out)), f"{label}: out differs from the direct call"
        assert np.array_equal(_bits(lse), _bits(ref_lse)), f"{label}: lse differs from the direct call"
        ref = oracle_full(wl)
        check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                        "fp8" if dc.fp8 else "bf16", label=f"noalloc {label}")
        kc, vc = dc.cache_host()
        assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), f"{label}: cache bytes"
        say(f"[ok] noalloc {label}: bitwise equal to the direct call, within the oracle tolerances")


def test_noalloc_needs_every_host_index_array():
    wl = make_custom(q_lens=[2], new_lens=[2], cache_lens=[5], Hq=4, Hkv=2, D=128, page_size=16,
                     causal=True, cache_dtype="bf16", seed=83)
    dc = DeviceCall(wl)
    out = torch.empty_like(dc.q)
    host = dict(dc.host)
    host["block_table"] = None
    with pytest.raises(vpk.VpkError) as ei:
        vpk.attn_varlen_paged_fwd_noalloc(dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache,
                                          dc.bt, dc.cl, wl.page_size, wl.causal, wl.scale, out=out, host_index=host)
    assert ei.value.status == _lib.VPK_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
