"""The dense fuzz tier's cases through every form of the call.

With the option mixed_grid 1 (every batch that holds both kinds of items in
one launch), the direct call is checked against the oracle (attention within
the tolerances, appended cache bytes exact); the prepared call (vpk_plan_run),
the allocation-free call and the page-list form, each on fresh copies of the
inputs, must then give the direct call's output, lse and cache bytes bit for
bit.
"""
import numpy as np
import pytest
import torch

import varlen_paged_kv_amd as vpk
from synth import make_custom

from gpu_util import DeviceCall, run_and_check, say
from test_gpu_fuzz import fuzz_case
from test_gpu_list import _list_call

pytestmark = pytest.mark.gpu

N_CASES = 200


@pytest.fixture(autouse=True)
def _one_launch():
    vpk.set_option("mixed_grid", 1)
    yield
    vpk.set_option("mixed_grid", -1)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _plan(dc):
    wl = dc.wl
    has_cache = wl.k_cache is not None
    return vpk.Plan(wl.cu_seqlens_q, wl.Hq, wl.Hkv, wl.D,
                    cu_seqlens_knew=wl.cu_seqlens_knew if dc.with_new else None,
                    cache_seqlens=wl.cache_seqlens if has_cache else None,
                    block_table=wl.block_table if has_cache else None,
                    page_size=wl.page_size if has_cache else 0,
                    num_pages=wl.k_cache.shape[0] if has_cache else 0,
                    max_pages_per_seq=wl.block_table.shape[1] if has_cache else 0,
                    cache_dtype=wl.cache_dtype if has_cache else "bf16", causal=wl.causal)


@pytest.mark.parametrize("i", range(N_CASES))
def test_forms_agree(i):
    spec = fuzz_case(i)
    wl = make_custom(**spec)
    dc, out, lse = run_and_check(wl, f"forms {i} q={spec['q_lens']} new={spec['new_lens']} "
                                     f"cache={spec['cache_lens']}", with_new=spec["new_lens"] is not None)
    caches = dc.cache_host()
    kv = wl.kv_scale if dc.fp8 else None
    dp = DeviceCall(wl, with_new=dc.with_new)
    o2, l2 = _plan(dp).run(dp.q, dp.k_new, dp.v_new, dp.k_cache, dp.v_cache, dp.bt, scale=wl.scale, kv_scale=kv)
    dn = DeviceCall(wl, with_new=dc.with_new)
    o3 = torch.empty_like(dn.q)
    l3 = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dn.q.device)
    vpk.attn_varlen_paged_fwd_noalloc(dn.q, dn.cu_q, dn.k_new, dn.v_new, dn.cu_kn, dn.k_cache, dn.v_cache, dn.bt,
                                      dn.cl, wl.page_size, wl.causal, wl.scale, kv, out=o3, lse=l3,
                                      host_index=dn.host)
    dl = DeviceCall(wl, with_new=dc.with_new)
    cu = wl.cu_seqlens_q.astype(np.int64)
    o4, l4 = _list_call(dl, dl.q, cu[:-1], np.diff(cu))
    torch.cuda.synchronize()
    for name, o, l, d in (("prepared", o2, l2, dp), ("allocation-free", o3, l3, dn), ("page-list", o4, l4, dl)):
        assert np.array_equal(_bits(o), _bits(out)), f"case {i} {name}: out differs from the direct call"
        assert np.array_equal(_bits(l), _bits(lse)), f"case {i} {name}: lse differs from the direct call"
        if caches[0] is not None:
            k2, v2 = d.cache_host()
            assert np.array_equal(k2, caches[0]) and np.array_equal(v2, caches[1]), f"case {i} {name}: cache bytes"
    say(f"[ok] forms {i}: prepared, allocation-free and page-list calls bitwise equal to the direct call")
