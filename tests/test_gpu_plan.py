"""Prepared calls (vpk_plan_create / vpk_plan_run) on the GPU.

A plan's run must match the oracle (attention within tolerance, appended
cache bytes exact) and give the direct call's bits (same kernels, same work
list); a run captured into a graph must do both on every replay, with the
program's own eager work between the replays."""
import dataclasses
import gc

import numpy as np
import pytest
import torch

import varlen_paged_kv_amd as vpk
from synth import make_custom

from gpu_util import DeviceCall, check_attention, oracle_full, say, to_np_out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_options():
    # a batch with both kinds of items runs in one launch in both the direct
    # call and the plan run, so that the two can be compared bit for bit (by
    # default a direct call runs two grids side by side and a plan run the
    # one launch; each is checked against the oracle elsewhere as well)
    vpk.set_option("mixed_grid", 1)
    yield
    vpk.set_option("force_splits", 0)
    vpk.set_option("mixed_grid", -1)


def _plan_for(dc):
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


def _run_plan(plan, dc, out=None, lse=None):
    wl = dc.wl
    return plan.run(dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, dc.bt, scale=wl.scale,
                    kv_scale=wl.kv_scale if dc.fp8 else None, out=out, lse=lse)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _check_oracle(dc, out, lse, label, q_bits=None):
    """out / lse of a run on dc's inputs (q replaced by q_bits when given) against the oracle,
    and the device caches against the oracle's append."""
    wl = dc.wl
    if q_bits is not None:
        wl = dataclasses.replace(wl, q=q_bits)
    ref = oracle_full(wl, with_new=dc.with_new)
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    "fp8" if dc.fp8 else "bf16", label=label)
    kc, vc = dc.cache_host()
    if kc is not None:
        assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), f"{label}: cache bytes"


def _mixed(cache_dtype, seed):
    # decode rows (q_len 1), a short and a long prefill, a sequence with no
    # cached prefix; page size 16
    return make_custom(q_lens=[1, 37, 1, 300, 1], new_lens=[1, 37, 1, 300, 1],
                       cache_lens=[500, 40, 1000, 0, 77], Hq=8, Hkv=2, D=128, page_size=16,
                       causal=True, cache_dtype=cache_dtype, seed=seed)


CASES = {
    "mixed_bf16": lambda: _mixed("bf16", 31),
    "mixed_fp8": lambda: _mixed("fp8", 32),
    "no_cache_D64": lambda: make_custom(q_lens=[200, 3, 90], new_lens=[200, 3, 90], cache_lens=[0, 0, 0],
                                        Hq=4, Hkv=4, D=64, page_size=0, causal=True, cache_dtype=None,
                                        seed=33),
    "cache_only": lambda: make_custom(q_lens=[1, 1, 40], new_lens=None, cache_lens=[300, 1200, 64],
                                      Hq=8, Hkv=2, D=128, page_size=64, causal=True, cache_dtype="bf16",
                                      seed=34),
}


@pytest.mark.parametrize("mixed_grid", [0, 1])
@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("case", sorted(CASES))
def test_plan_run_equals_direct_call(case, splits, mixed_grid):
    vpk.set_option("force_splits", splits)
    vpk.set_option("mixed_grid", mixed_grid)
    wl = CASES[case]()
    dc = DeviceCall(wl, with_new=wl.k_new is not None)
    say(f"[case] plan {case} splits={splits} mixed_grid={mixed_grid}")
    ref_out, ref_lse = dc.run()
    plan = _plan_for(dc)
    out, lse = _run_plan(plan, dc)
    torch.cuda.synchronize()
    _check_oracle(dc, out, lse, f"plan {case} splits={splits}")
    assert np.array_equal(_bits(out), _bits(ref_out)), f"{case}: out differs"
    assert np.array_equal(_bits(lse), _bits(ref_lse)), f"{case}: lse differs"
    assert plan.device_error() == 0
    # a second run of the same plan (partials and flag reused)
    out2, lse2 = _run_plan(plan, dc)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out2), _bits(ref_out)) and np.array_equal(_bits(lse2), _bits(ref_lse))
    plan.close()
    say(f"[ok] plan {case} splits={splits}: within the oracle tolerances, bitwise equal to the direct call")


@pytest.mark.parametrize("case", ["mixed_bf16", "mixed_fp8"])
def test_plan_run_in_graph_replays(case):
    vpk.set_option("force_splits", 2)   # the merge pass is captured too
    wl = CASES[case]()
    dc = DeviceCall(wl)
    plan = _plan_for(dc)
    out = torch.empty_like(dc.q)
    lse = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dc.q.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run_plan(plan, dc, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gc.collect()   # no earlier graph may be collected during the capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run_plan(plan, dc, out, lse)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(3):
        # eager work between replays: new query values in the captured buffer
        dc.q.copy_(torch.randn(dc.q.shape, generator=gen).to(torch.bfloat16).to(dc.q.device))
        g.replay()
        torch.cuda.synchronize()
        q_bits = dc.q.view(torch.int16).cpu().numpy().view(np.uint16)
        _check_oracle(dc, out, lse, f"{case} replay {rep}", q_bits=q_bits)
        ref_out, ref_lse = dc.run()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(ref_out)), f"{case}: replay {rep} out differs"
        assert np.array_equal(_bits(lse), _bits(ref_lse)), f"{case}: replay {rep} lse differs"
    del g
    gc.collect()
    plan.close()
    say(f"[ok] graph replays of {case}: within the oracle tolerances, bitwise equal to eager calls")


def test_device_scales_follow_changes_between_graph_replays():
    """fp8 plan run with the scales in device memory: bitwise equal to the direct
    call with the same scales on the host, also in a captured graph whose scale
    buffer the program rewrites between replays."""
    vpk.set_option("force_splits", 2)
    wl = CASES["mixed_fp8"]()
    dc = DeviceCall(wl)
    plan = _plan_for(dc)
    ks_host = np.asarray(wl.kv_scale, np.float32)
    ks_dev = torch.from_numpy(ks_host.copy()).cuda()

    def direct(ks):
        return vpk.attn_varlen_paged_fwd(dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache,
                                         dc.bt, dc.cl, wl.page_size, wl.causal, wl.scale,
                                         (float(ks[0]), float(ks[1])), host_index=dc.host)

    out = torch.empty_like(dc.q)
    lse = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dc.q.device)
    plan.run(dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, dc.bt, scale=wl.scale, kv_scale=ks_dev,
             out=out, lse=lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = direct(ks_host)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref_out)) and np.array_equal(_bits(lse), _bits(ref_lse))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run(dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, dc.bt, scale=wl.scale, kv_scale=ks_dev,
                 out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gc.collect()   # no earlier graph may be collected during the capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, dc.bt, scale=wl.scale, kv_scale=ks_dev,
                 out=out, lse=lse)
    torch.cuda.synchronize()
    for rep, f in enumerate((1.25, 0.5, 1.0)):
        ks = (ks_host * np.float32(f)).astype(np.float32)
        ks_dev.copy_(torch.from_numpy(ks))           # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = _bits(out), _bits(lse)
        kc_g = dc.k_cache.cpu().numpy().copy()
        ref_out, ref_lse = direct(ks)
        torch.cuda.synchronize()
        # the oracle with the same scales: the new tokens are quantised with them, the cached
        # prefix keeps its codes and is read with them
        ref = oracle_full(dataclasses.replace(wl, kv_scale=(np.float32(ks[0]), np.float32(ks[1]))))
        check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"], "fp8",
                        label=f"device scales replay {rep}")
        assert np.array_equal(kc_g, ref["k_cache"]), f"replay {rep}: appended codes differ from the oracle"
        assert np.array_equal(got_o, _bits(ref_out)), f"replay {rep} (scales x{f}): out differs"
        assert np.array_equal(got_l, _bits(ref_lse)), f"replay {rep} (scales x{f}): lse differs"
        assert np.array_equal(kc_g, dc.k_cache.cpu().numpy()), f"replay {rep}: appended codes differ"
    del g
    gc.collect()
    plan.close()
    say("[ok] device scales: plan runs and graph replays follow the scale buffer bit for bit")
