"""Error paths on the GPU, each ending before any kernel could go wrong.

* Direct calls refuse stream capture (VPK_ERROR_NOT_SUPPORTED) before
  anything is enqueued.
* The binding rejects outputs and index arrays of the wrong shape, dtype or
  length before calling the library.
* The kernels' own page-id guard: page ids outside [0, num_pages) that the
  host cannot see (no host block_table) are skipped and flagged.  The caches
  are allocated with spare pages past the declared num_pages, so even a
  broken guard would read and write inside the allocation.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import varlen_paged_kv_amd as vpk
from synth import make_custom
from varlen_paged_kv_amd import _lib

from gpu_util import DeviceCall, check_attention, dev_bf16, dev_i32, dev_u8, say, to_np_out

pytestmark = pytest.mark.gpu


def _small(cache="bf16", seed=61):
    return make_custom(q_lens=[3, 2], new_lens=[3, 2], cache_lens=[40, 20], Hq=4, Hkv=2, D=128, page_size=16,
                       causal=True, cache_dtype=cache, seed=seed)


def _capture_and_call(fn):
    """Run fn() inside a graph capture (next to one ordinary captured op); return the (status, message)
    of the VpkError it raised, or None.

    Only the status and message are kept: the exception's traceback references this frame, and with it
    the graph, so keeping the exception would leave the graph to the cyclic garbage collector, which
    may then destroy it in the middle of a later capture (an abort).  The graph is destroyed here,
    outside any capture."""
    gc.collect()                      # no earlier graph may be collected during this capture
    x = torch.zeros(16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    err = None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            x.add_(1.0)
            try:
                fn(s)
            except vpk.VpkError as e:
                err = (e.status, e.msg)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert float(x[0]) == 1.0
    del g
    gc.collect()
    torch.cuda.synchronize()
    return err


@pytest.mark.parametrize("entry", ["attn", "list", "append"])
def test_direct_calls_refuse_stream_capture(entry):
    wl = _small()
    dc = DeviceCall(wl)
    say(f"[case] capture refusal: {entry}")
    kc0, vc0 = dc.cache_host()

    def call(s):
        if entry == "attn":
            dc.run(stream=s)
        elif entry == "append":
            vpk.kv_cache_append(dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl, wl.page_size,
                                host_index=dc.host, stream=s)
        else:
            cu = wl.cu_seqlens_q.astype(np.int64)
            indptr = np.concatenate([[0], np.cumsum([wl.block_table.shape[1]] * wl.B)]).astype(np.int32)
            vpk.attn_varlen_paged_list_fwd(dc.q, cu[:-1], np.diff(cu), dc.k_new, dc.v_new, wl.cu_seqlens_knew,
                                           dc.k_cache, dc.v_cache, indptr, dc.bt.reshape(-1), wl.cache_seqlens,
                                           wl.page_size, wl.causal, wl.scale, stream=s)

    err = _capture_and_call(call)
    assert err is not None and err[0] == _lib.VPK_ERROR_NOT_SUPPORTED, err
    kc1, vc1 = dc.cache_host()
    assert np.array_equal(kc0, kc1) and np.array_equal(vc0, vc1), "a refused call changed the cache"
    say(f"[ok] capture refusal {entry}: {err[1]}")


def test_binding_rejects_bad_outputs_and_index_lengths():
    wl = _small()
    dc = DeviceCall(wl)
    Tq, Hq, D = wl.Tq, wl.Hq, wl.D
    assert Tq != Hq
    bad = {
        "out too small": dict(out=torch.empty((Tq - 1, Hq, D), dtype=torch.bfloat16, device="cuda")),
        "out fp32": dict(out=torch.empty((Tq, Hq, D), dtype=torch.float32, device="cuda")),
        "out strided": dict(out=torch.empty((Tq, Hq, 2 * D), dtype=torch.bfloat16, device="cuda")[:, :, :D]),
        "lse transposed": dict(lse=torch.empty((Tq, Hq), dtype=torch.float32, device="cuda")),
        "lse bf16": dict(lse=torch.empty((Hq, Tq), dtype=torch.bfloat16, device="cuda")),
    }
    for label, kw in bad.items():
        say(f"[case] binding rejects {label}")
        with pytest.raises(vpk.VpkError):
            vpk.attn_varlen_paged_fwd(dc.q, dc.cu_q, dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt,
                                      dc.cl, wl.page_size, wl.causal, wl.scale, host_index=dc.host, **kw)
    args = dict(q=dc.q, cu_seqlens_q=dc.cu_q, k_new=dc.k_new, v_new=dc.v_new, cu_seqlens_knew=dc.cu_kn,
                k_cache=dc.k_cache, v_cache=dc.v_cache, block_table=dc.bt, cache_seqlens=dc.cl)
    for label, key, val in (("block_table rows", "block_table", dc.bt[:1].contiguous()),
                            ("cache_seqlens length", "cache_seqlens", dc.cl[:1].contiguous()),
                            ("cu_seqlens_knew length", "cu_seqlens_knew", dc.cu_kn[:2].contiguous())):
        say(f"[case] binding rejects {label}")
        with pytest.raises(vpk.VpkError):
            vpk.attn_varlen_paged_fwd(**{**args, key: val}, page_size=wl.page_size, causal=wl.causal,
                                      scale=wl.scale, host_index=dict(cu_seqlens_q=wl.cu_seqlens_q))
    say("[case] binding rejects a host block_table of the wrong size")
    with pytest.raises(vpk.VpkError):
        vpk.attn_varlen_paged_fwd(**args, page_size=wl.page_size, causal=wl.causal, scale=wl.scale,
                                  host_index={**dc.host, "block_table": wl.block_table[:1]})
    torch.cuda.synchronize()
    say("[ok] binding checks")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_device_page_guard(cache):
    """Page ids past num_pages, seen only by the kernels: skipped and flagged, never followed."""
    wl = _small(cache, seed=62)
    S, P = wl.page_size, wl.num_pages
    spare = 4
    # caches with `spare` pages past the declared pool; the call sees the first P pages only
    fill = np.random.default_rng(5)
    if cache == "fp8":
        ext_k = np.concatenate([wl.k_cache, fill.integers(0, 120, (spare,) + wl.k_cache.shape[1:]).astype(np.uint8)])
        ext_v = np.concatenate([wl.v_cache, fill.integers(0, 120, (spare,) + wl.v_cache.shape[1:]).astype(np.uint8)])
        mk = dev_u8
    else:
        ext_k = np.concatenate([wl.k_cache, np.full((spare,) + wl.k_cache.shape[1:], 0x3F80, np.uint16)])
        ext_v = np.concatenate([wl.v_cache, np.full((spare,) + wl.v_cache.shape[1:], 0x4000, np.uint16)])
        mk = dev_bf16
    bt = wl.block_table.copy()
    bt[0, 1] = P + 1   # sequence 0, keys 16..31: all cached
    bt[1, 1] = P + 2   # sequence 1, keys 16..21: 16..19 cached, 20..21 new (appended there)
    kc_d, vc_d = mk(ext_k), mk(ext_v)
    q, kn, vn = dev_bf16(wl.q), dev_bf16(wl.k_new), dev_bf16(wl.v_new)
    say(f"[case] device page guard {cache}: num_pages {P}, ids {P + 1} and {P + 2} in the spare range")
    vpk.device_error()   # clear the flag of this stream's workspace
    out, lse = vpk.attn_varlen_paged_fwd(
        q, dev_i32(wl.cu_seqlens_q), kn, vn, dev_i32(wl.cu_seqlens_knew), kc_d[:P], vc_d[:P], dev_i32(bt),
        dev_i32(wl.cache_seqlens), S, wl.causal, wl.scale, wl.kv_scale,
        host_index=dict(cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_knew=wl.cu_seqlens_knew,
                        cache_seqlens=wl.cache_seqlens))
    torch.cuda.synchronize()
    assert vpk.device_error() == 1, "the device error flag was not raised"
    # expected cache: the oracle's append through the same table, except that nothing lands
    # on the skipped pages (spare pages keep their contents)
    rk, rv = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, ext_k, ext_v, bt, wl.cache_seqlens, S, cache,
                           wl.kv_scale)
    rk[P:], rv[P:] = ext_k[P:], ext_v[P:]
    got_k = kc_d.cpu().numpy() if cache == "fp8" else kc_d.view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = vc_d.cpu().numpy() if cache == "fp8" else vc_d.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, rk) and np.array_equal(got_v, rv), "cache bytes differ"
    # expected attention: keys on a skipped page read as zero (with a bf16 cache the new tokens
    # come from k_new / v_new themselves)
    Q = oracle.bf16_bits_to_f64(wl.q)
    ref_out = np.zeros((wl.Tq, wl.Hq, wl.D))
    ref_lse = np.full((wl.Hq, wl.Tq), -np.inf)
    for b in range(wl.B):
        K, V = oracle.sequence_kv(b, k_new=wl.k_new, v_new=wl.v_new, cu_seqlens_knew=wl.cu_seqlens_knew,
                                  k_cache=rk, v_cache=rv, block_table=bt, cache_seqlens=wl.cache_seqlens,
                                  page_size=S, cache_dtype=cache, kv_scale=wl.kv_scale)
        lc = int(wl.cache_seqlens[b])
        K, V = K.copy(), V.copy()
        for pos in range(16, min(32, K.shape[0])):
            if cache == "bf16" and pos >= lc:
                j = int(wl.cu_seqlens_knew[b]) + pos - lc
                K[pos] = oracle.bf16_bits_to_f64(wl.k_new[j])
                V[pos] = oracle.bf16_bits_to_f64(wl.v_new[j])
            else:
                K[pos] = 0.0
                V[pos] = 0.0
        s0, e0 = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        o, l = oracle.attend(Q[s0:e0], K, V, wl.causal, wl.scale)
        ref_out[s0:e0], ref_lse[:, s0:e0] = o, l
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse,
                    "fp8" if cache == "fp8" else "bf16", label=f"page guard {cache}")
    say(f"[ok] device page guard {cache}: flagged, skipped pages read as zero, their appends dropped")
