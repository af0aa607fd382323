"""Caller-owned workspace (vpk_set_workspace) on the GPU.

The binding registers a torch tensor as the workspace of every stream it
calls on; then the library allocates no device memory of its own.  Results
are bitwise those of the library's own workspace, with the work list read
from pinned host memory or uploaded into the workspace, and within the
oracle's tolerances with a workspace too small for the planner's splits.
"""
import numpy as np
import pytest
import torch

import varlen_paged_kv_amd as vpk
from synth import make_custom
from varlen_paged_kv_amd import _lib

from gpu_util import DeviceCall, check_attention, oracle_full, say, to_np_out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    vpk.AUTO_WORKSPACE = True
    vpk.set_option("force_splits", 0)
    vpk.set_option("plan_upload", 0)
    vpk.set_option("plan_reuse", 1)


def _mixed(cache="bf16", seed=71):
    return make_custom(q_lens=[1, 37, 1, 300, 1], new_lens=[1, 37, 1, 300, 1], cache_lens=[500, 40, 1000, 0, 77],
                       Hq=8, Hkv=2, D=128, page_size=16, causal=True, cache_dtype=cache, seed=seed)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _run(dc, stream):
    with torch.cuda.stream(stream):
        out, lse = dc.run(stream=stream)
    stream.synchronize()
    return out, lse


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_torch_workspace_means_no_library_allocation(cache):
    vpk.set_option("force_splits", 3)     # split partials live in the workspace
    wl = _mixed(cache)
    dc = DeviceCall(wl)
    s = torch.cuda.Stream()
    dev0, pin0 = vpk.library_memory()
    say(f"[case] torch workspace {cache}: library memory before {dev0} device / {pin0} pinned bytes")
    out, lse = _run(dc, s)
    dev1, _ = vpk.library_memory()
    assert dev1 == dev0, f"the library allocated {dev1 - dev0} device bytes with a caller workspace"
    ref = oracle_full(wl)
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    "fp8" if cache == "fp8" else "bf16", label=f"torch workspace {cache}")
    say(f"[ok] torch workspace {cache}: no library device memory, within tolerance")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_caller_and_library_workspaces_give_the_same_bits(cache):
    vpk.set_option("force_splits", 3)
    wl = _mixed(cache, seed=72)
    dc = DeviceCall(wl)
    say(f"[case] library workspace vs caller workspace vs uploaded plan, {cache}")
    vpk.AUTO_WORKSPACE = False
    s_lib = torch.cuda.Stream()
    o_lib, l_lib = _run(dc, s_lib)                   # library-owned workspace on a fresh stream
    vpk.AUTO_WORKSPACE = True
    s_user = torch.cuda.Stream()
    o_user, l_user = _run(dc, s_user)                # torch tensor registered by the binding
    vpk.set_option("plan_upload", 1)
    o_up, l_up = _run(dc, s_user)                    # work list uploaded into that workspace
    o_up_lib, l_up_lib = None, None
    vpk.AUTO_WORKSPACE = False
    o_up_lib, l_up_lib = _run(dc, s_lib)             # uploaded into the library's workspace
    for name, o, l in (("caller", o_user, l_user), ("caller+upload", o_up, l_up), ("library+upload", o_up_lib, l_up_lib)):
        assert np.array_equal(_bits(o), _bits(o_lib)), f"{name}: out differs"
        assert np.array_equal(_bits(l), _bits(l_lib)), f"{name}: lse differs"
    ref = oracle_full(wl)
    check_attention(to_np_out(o_lib), l_lib.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    "fp8" if cache == "fp8" else "bf16", label=f"workspaces {cache}")
    say(f"[ok] workspaces {cache}: bitwise equal, within tolerance")


def test_small_workspace_splits_less_and_too_small_is_refused():
    wl = make_custom(q_lens=[1, 1, 2], new_lens=[1, 1, 2], cache_lens=[3000, 2500, 4000], Hq=8, Hkv=2, D=128,
                     page_size=16, causal=True, cache_dtype="bf16", seed=73)
    dc = DeviceCall(wl)
    ref = oracle_full(wl)
    vpk.AUTO_WORKSPACE = False
    s = torch.cuda.Stream()
    dims = _lib.VpkDims(wl.B, wl.Tq, wl.Tn, wl.Hq, wl.Hkv, wl.D, wl.num_pages, wl.block_table.shape[1],
                        _lib.VPK_DTYPE_BF16)
    full = vpk.workspace_bytes_upper_bound(dims)
    # room for the head, the plan and a few hundred partial rows: the planner splits less
    for size in (full, 64 * 1024, 8 * 1024):
        buf = torch.empty(size, dtype=torch.uint8, device="cuda")
        vpk.set_workspace(buf, stream=s)
        say(f"[case] workspace of {size} bytes (bound {full})")
        out, lse = _run(dc, s)
        check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                        label=f"workspace {size} bytes")
        del buf
    # too small for the turned copies of q and k_new of a rope call
    buf = torch.empty(8 * 1024, dtype=torch.uint8, device="cuda")
    vpk.set_workspace(buf, stream=s)
    from synth import rope_tables
    cos, sin = rope_tables(5000, wl.D)
    with pytest.raises(vpk.VpkError) as ei:
        with torch.cuda.stream(s):
            vpk.attn_varlen_paged_rope_fwd(dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt,
                                           dc.cl, wl.page_size, wl.causal, wl.scale, rope_cos=torch.from_numpy(cos).cuda(),
                                           rope_sin=torch.from_numpy(sin).cuda(), host_index=dc.host, stream=s)
    assert ei.value.status == _lib.VPK_ERROR_CAPACITY, ei.value
    vpk.set_workspace(None, stream=s)
    s.synchronize()
    say(f"[ok] small workspaces within tolerance; too small refused: {ei.value.msg}")


def test_repeated_calls_read_the_reused_work_list():
    """Direct calls on one stream with a caller's workspace: from the second call in a row with the same work
    list on, the kernels read its copy at the end of the workspace.  A call with other lengths between, and
    calls whose partials reach the copy (a workspace of exactly the bound, every tile cut into 7 parts), must
    not disturb it: every call gives the bits of the same call with reuse off, in the same workspace."""
    wa = _mixed("bf16", seed=74)
    wb = make_custom(q_lens=[3, 1, 64], new_lens=[3, 1, 64], cache_lens=[100, 2000, 30], Hq=8, Hkv=2, D=128,
                     page_size=16, causal=True, cache_dtype="bf16", seed=75)
    da, db = DeviceCall(wa), DeviceCall(wb)
    vpk.AUTO_WORKSPACE = False
    big = max(int(wl.B) for wl in (wa, wb))
    dims = [_lib.VpkDims(wl.B, wl.Tq, wl.Tn, wl.Hq, wl.Hkv, wl.D, wl.num_pages, wl.block_table.shape[1],
                         _lib.VPK_DTYPE_BF16) for wl in (wa, wb)]
    size = max(vpk.workspace_bytes_upper_bound(d) for d in dims)
    steps = [("a", 0), ("a", 0), ("a", 0), ("b", 0), ("a", 0), ("a", 0), ("a", 7), ("a", 7), ("a", 0), ("a", 0)]
    results = {}
    for reuse in (0, 1):
        vpk.set_option("plan_reuse", reuse)
        s = torch.cuda.Stream()
        buf = torch.empty(size, dtype=torch.uint8, device="cuda")
        vpk.set_workspace(buf, stream=s)
        say(f"[case] plan reuse {reuse}: {len(steps)} calls in a row, workspace {size} bytes (batch {big})")
        outs = []
        with torch.cuda.stream(s):
            for name, splits in steps:
                vpk.set_option("force_splits", splits)
                outs.append((da if name == "a" else db).run(stream=s))
        s.synchronize()
        vpk.set_workspace(None, stream=s)
        results[reuse] = [(_bits(o), _bits(l)) for o, l in outs]
        del buf
    vpk.set_option("force_splits", 0)
    for i, ((o0, l0), (o1, l1)) in enumerate(zip(results[0], results[1])):
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), f"call {i} {steps[i]}: reuse changed the bits"
    ref = oracle_full(wa)
    o, l = outs[-1]
    check_attention(to_np_out(o), l.cpu().numpy().astype(np.float64), ref["out"], ref["lse"], label="plan reuse")
    say("[ok] plan reuse: every call bitwise equal to reuse off, within tolerance")



def test_back_to_back_calls_through_the_plan_ring():
    """Fourteen direct calls without a synchronisation, cycling over three batches with different lengths
    (each call long on the GPU, so the host plans well ahead and wraps the ring of 8 plan buffers, whose
    reuse waits on one event per 4 calls): each result must be bitwise the same call run alone."""
    rng = np.random.default_rng(76)
    wls = []
    for i in range(3):
        ql = rng.integers(128, 512, size=8)
        wls.append(make_custom(q_lens=ql.tolist(), new_lens=ql.tolist(),
                               cache_lens=rng.integers(2000, 6000, size=8).tolist(), Hq=32, Hkv=8, D=128,
                               page_size=16, causal=True, cache_dtype="bf16", seed=77 + i))
    dcs = [DeviceCall(wl) for wl in wls]
    s = torch.cuda.Stream()
    alone = []
    for dc in dcs:
        o, l = _run(dc, s)
        alone.append((_bits(o), _bits(l)))
    order = [i % 3 for i in range(14)]
    say(f"[case] plan ring: {len(order)} calls back to back over 3 batches of 8 sequences")
    with torch.cuda.stream(s):
        outs = [dcs[i].run(stream=s) for i in order]
    s.synchronize()
    for n, (i, (o, l)) in enumerate(zip(order, outs)):
        assert np.array_equal(_bits(o), alone[i][0]) and np.array_equal(_bits(l), alone[i][1]), \
            f"call {n} (batch {i}) differs from the same call alone"
    say("[ok] plan ring: every back-to-back call bitwise equal to the call alone")
