"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status codes before it
touches the device (fake, never-dereferenced device pointers are passed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from varlen_paged_kv_amd import _lib
from varlen_paged_kv_amd._lib import VpkDims, VpkHostIndex

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "vpk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    declared = _declared_functions()
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.vpk_abi_version() == 1


FAKE = 1 << 20  # aligned, never dereferenced on the host


def _call(dims, *, q=FAKE, cu_q=FAKE, k_new=FAKE, v_new=FAKE, cu_kn=FAKE, kc=FAKE, vc=FAKE,
          bt=FAKE, cl=FAKE, page_size=16, causal=1, scale=0.1, kv_scale=None, out=FAKE,
          lse=FAKE, host=None):
    lib = _lib.load()
    ks = None if kv_scale is None else (ctypes.c_float * 2)(*kv_scale)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.attn_varlen_paged_fwd(ctypes.byref(dims), vp(q), vp(cu_q), vp(k_new), vp(v_new),
                                   vp(cu_kn), vp(kc), vp(vc), vp(bt), vp(cl), page_size, causal,
                                   scale, ks, vp(out), vp(lse),
                                   None if host is None else ctypes.byref(host), None)
    return st, lib.vpk_last_error().decode()


def _host(cu_q, cu_kn=None, cl=None, bt=None):
    arrs = [None if a is None else np.ascontiguousarray(a, np.int32) for a in (cu_q, cu_kn, cl, bt)]
    hi = VpkHostIndex(*[None if a is None else a.ctypes.data for a in arrs])
    return hi, arrs


def _dims(**kw):
    d = dict(batch=2, total_q=4, total_knew=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
             num_pages=10, max_pages_per_seq=4, kv_cache_dtype=1)
    d.update(kw)
    return VpkDims(**d)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(num_q_heads=6, num_kv_heads=4), 1, "multiple"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(batch=-1), 1, "negative"),
    (dict(num_kv_heads=0), 1, "positive"),
    (dict(kv_cache_dtype=7), 1, "kv_cache_dtype"),
    (dict(num_pages=0), 1, "num_pages"),
])
def test_dims_errors(kw, code, frag):
    hi, keep = _host([0, 2, 4], [0, 2, 4], [3, 5])
    st, msg = _call(_dims(**kw), host=hi)
    assert st == code and frag in msg


def test_argument_errors():
    hi, keep = _host([0, 2, 4], [0, 2, 4], [3, 5])
    d = _dims()
    assert _call(d, host=hi, page_size=0)[0] == 1
    assert _call(d, host=hi, k_new=None)[0] == 1                    # k_new without v_new
    assert _call(d, host=hi, kc=None)[0] == 1                       # k_cache without v_cache
    assert _call(d, host=hi, k_new=None, v_new=None, kc=None, vc=None)[0] == 1
    assert _call(d, host=hi, causal=2)[0] == 1
    assert _call(d, host=hi, scale=float("nan"))[0] == 1
    assert _call(d, host=hi, q=FAKE + 2)[0] == 1                     # misaligned
    assert "aligned" in _call(d, host=hi, out=FAKE + 8)[1]
    assert _call(d, host=hi, bt=None)[0] == 1
    # fp8 without / with bad scales
    d8 = _dims(kv_cache_dtype=2)
    assert "kv_scale" in _call(d8, host=hi)[1]
    assert _call(d8, host=hi, kv_scale=(1.0, 0.0))[0] == 1
    assert _call(d8, host=hi, kv_scale=(1.0, float("inf")))[0] == 1
    # bf16 cache with a scale
    assert _call(d, host=hi, kv_scale=(1.0, 1.0))[0] == 1


def test_index_content_errors():
    d = _dims()
    hi, k = _host([1, 2, 4], [0, 2, 4], [3, 5])
    assert "cu_seqlens_q[0]" in _call(d, host=hi)[1]
    hi, k = _host([0, 3, 2], [0, 2, 4], [3, 5])
    assert "non-decreasing" in _call(d, host=hi)[1]
    hi, k = _host([0, 2, 5], [0, 2, 4], [3, 5])
    assert "total" in _call(d, host=hi)[1]
    hi, k = _host([0, 2, 4], [0, 2, 3], [3, 5])
    assert "cu_seqlens_knew" in _call(d, host=hi)[1]
    hi, k = _host([0, 2, 4], [0, 2, 4], [3, -1])
    assert _call(d, host=hi)[0] == 1
    # capacity: 4 pages of 16 slots hold 64 keys; 63 cached + 2 new do not fit
    hi, k = _host([0, 2, 4], [0, 2, 4], [3, 63])
    st, msg = _call(d, host=hi)
    assert st == 3 and "slots" in msg
    # page ids checked when a host block table is given
    bt = np.array([[0, 1, 2, 3], [4, 5, 10, 7]], np.int32)
    hi, k = _host([0, 2, 4], [0, 2, 4], [3, 40], bt)
    st, msg = _call(d, host=hi)
    assert st == 1 and "block_table[1][2]" in msg
    # entries past ceil(Lk / S) are never read, so -1 padding there is fine
    # (checked through the host-only planner entry, which runs the same checks)
    bt = np.array([[0, -1, -1, -1], [4, 5, 6, 7]], np.int32)
    hi, k = _host([0, 2, 4], [0, 2, 4], [3, 40], bt)
    lib = _lib.load()
    items = (ctypes.c_int32 * 4096)()
    n, nq = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.vpk_plan_debug(ctypes.byref(d), ctypes.byref(hi), 1, 1, 16, 1, 256, items, 512,
                            ctypes.byref(n), ctypes.byref(nq))
    assert st == 0, lib.vpk_last_error()
    bt[0, 0] = -1
    st = lib.vpk_plan_debug(ctypes.byref(d), ctypes.byref(hi), 1, 1, 16, 1, 256, items, 512,
                            ctypes.byref(n), ctypes.byref(nq))
    assert st == 1 and b"block_table[0][0]" in lib.vpk_last_error()


def test_options():
    lib = _lib.load()
    assert lib.vpk_set_option(b"force_splits", 3) == 0
    assert lib.vpk_set_option(b"force_splits", 0) == 0
    assert lib.vpk_set_option(b"persistent", 5) == 1
    assert lib.vpk_set_option(b"nope", 1) == 1
    assert "unknown option" in lib.vpk_last_error().decode()
    assert lib.vpk_timing_read(7, None, None) == 1


def _plan_create(dims, host, has_new=1, has_cache=1, page_size=16, causal=1):
    lib = _lib.load()
    h = ctypes.c_void_p()
    st = lib.vpk_plan_create(ctypes.byref(dims), None if host is None else ctypes.byref(host),
                             has_new, has_cache, page_size, causal, ctypes.byref(h))
    return st, lib.vpk_last_error().decode(), h


def test_plan_create_errors_before_the_device():
    """vpk_plan_create checks everything on the host first: each bad argument
    returns its status with no handle and no device call."""
    d = _dims()
    hi, keep = _host([0, 2, 4], [0, 2, 4], [3, 5])
    st, msg, h = _plan_create(d, None)
    assert st == 1 and "host index" in msg and h.value is None
    hq, keep2 = _host([0, 2, 4])                                     # no cu_seqlens_knew / cache_seqlens
    assert _plan_create(d, hq)[0] == 1
    assert _plan_create(d, hi, has_new=0, has_cache=0)[0] == 1
    assert _plan_create(d, hi, has_new=2)[0] == 1
    assert _plan_create(d, hi, causal=2)[0] == 1
    assert _plan_create(d, hi, page_size=0)[0] == 1
    assert _plan_create(_dims(head_dim=96), hi)[0] == 2
    bad, k3 = _host([0, 3, 2], [0, 2, 4], [3, 5])
    assert "non-decreasing" in _plan_create(d, bad)[1]
    full, k4 = _host([0, 2, 4], [0, 2, 4], [63, 5])                  # 63 + 2 keys > 4 pages of 16
    assert _plan_create(d, full)[0] == 3
    bt = np.array([[0, 1, 2, 3], [4, 99, 6, 7]], np.int32)           # page 99 >= num_pages
    hb, k5 = _host([0, 2, 4], [0, 2, 4], [3, 20], bt)
    st, msg, _ = _plan_create(d, hb)
    assert st == 1 and "outside" in msg
    assert _plan_create(_dims(total_knew=4), hi, has_new=0)[0] == 1   # new tokens counted without new tokens
    lib = _lib.load()
    assert lib.vpk_plan_run(None, None, None, None, None, None, None, 0.1, None, None, None, None) == 1
    assert lib.vpk_plan_destroy(None) == 0


def test_qkv_prob_score_bytes():
    """Room for kept QKV-Prob scores: 128 bytes per (row, 32 keys, kv head) of each sequence of at most 8
    packed rows (head_dim 128 only), plus 256 bytes of alignment; 0 when nothing qualifies."""
    lib = _lib.load()
    d = _dims(batch=4, total_q=12, total_knew=12, num_q_heads=8, num_kv_heads=2)          # g = 4
    hi, keep = _host([0, 1, 3, 11, 12], [0, 1, 3, 11, 12], [100, 31, 0, 5000])
    # rows 4, 8, 32 (too many), 4; keys 101, 33, -, 5001 -> blocks 4, 2, -, 157
    want = (4 * 4 + 8 * 2 + 4 * 157) * 2 * 128 + 256
    assert lib.vpk_qkv_prob_score_bytes(ctypes.byref(d), ctypes.byref(hi)) == want
    only_new, k2 = _host([0, 1, 3, 11, 12], [0, 1, 3, 11, 12])                            # no cache
    assert lib.vpk_qkv_prob_score_bytes(ctypes.byref(d), ctypes.byref(only_new)) == (4 + 8 + 4) * 2 * 128 + 256
    assert lib.vpk_qkv_prob_score_bytes(ctypes.byref(_dims(batch=4, total_q=12, total_knew=12, num_q_heads=8,
                                                           num_kv_heads=2, head_dim=64)), ctypes.byref(hi)) == 0
    assert lib.vpk_qkv_prob_score_bytes(ctypes.byref(d), None) == 0
    assert lib.vpk_set_option(b"keep_scores", 0) == 0
    assert lib.vpk_set_option(b"keep_scores", 1) == 0
    assert lib.vpk_set_option(b"keep_scores", 2) == 1
    assert lib.vpk_set_option(b"plan_reuse", 0) == 0
    assert lib.vpk_set_option(b"plan_reuse", 1) == 0
    assert lib.vpk_set_option(b"plan_reuse", 2) == 1


def test_plan_log(capfd):
    """Option "plan_log" prints one line per planned call on stderr (the plan is
    built before any device call, so the line appears here without a GPU)."""
    lib = _lib.load()
    assert lib.vpk_set_option(b"plan_log", 2) == 1
    hi, keep = _host([0, 2, 4], [0, 2, 4], [3, 5])
    try:
        assert lib.vpk_set_option(b"plan_log", 1) == 0
        assert lib.vpk_set_option(b"num_cus", 256) == 0
        st, msg, h = _plan_create(_dims(), hi)
        if st == 0:
            lib.vpk_plan_destroy(h)
    finally:
        lib.vpk_set_option(b"plan_log", -1)
        lib.vpk_set_option(b"num_cus", 0)
    err = capfd.readouterr().err
    assert "vpk: plan_create batch=2 q_rows=4 new_rows=4 hq=8 hkv=2 D=128" in err
    assert "units pre=0 dec=2" in err        # two sequences of 2 tokens x 4 heads per kv head: decode mode
    assert lib.vpk_set_option(b"plan_log", 0) == 0
    try:
        st, msg, h = _plan_create(_dims(), hi)
        if st == 0:
            lib.vpk_plan_destroy(h)
    finally:
        lib.vpk_set_option(b"plan_log", -1)
    assert "vpk:" not in capfd.readouterr().err


def _list_call(dims, hp, *, q=FAKE, k_new=FAKE, v_new=FAKE, kc=FAKE, vc=FAKE, kvi=FAKE, page_size=16,
               causal=1, scale=0.1, out=FAKE, lse=FAKE):
    lib = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.attn_varlen_paged_list_fwd(ctypes.byref(dims), vp(q), vp(k_new), vp(v_new), vp(kc), vp(vc), vp(kvi),
                                        page_size, causal, scale, None, vp(out), vp(lse),
                                        None if hp is None else ctypes.byref(hp), None)
    return st, lib.vpk_last_error().decode()


def _pages(q_start, q_len, cu_kn=None, cl=None, indptr=None, indices=None):
    arrs = [None if a is None else np.ascontiguousarray(a, np.int32)
            for a in (q_start, q_len, cu_kn, cl, indptr, indices)]
    return _lib.VpkHostPages(*[None if a is None else a.ctypes.data for a in arrs]), arrs


def test_page_list_form_errors_before_the_device():
    """attn_varlen_paged_list_fwd checks its host arrays before any device work."""
    d = _dims(total_q=10)
    ok, k0 = _pages([0, 6], [2, 2], [0, 2, 4], [3, 5], [0, 2, 4], [0, 1, 2, 3])
    assert _list_call(d, None)[0] == 1
    hp, k1 = _pages([0, 1], [2, 2], [0, 2, 4], [3, 5], [0, 2, 4])          # rows 0-1 and 1-2 overlap
    st, msg = _list_call(d, hp)
    assert st == 1 and "share" in msg
    hp, k2 = _pages([0, 9], [2, 2], [0, 2, 4], [3, 5], [0, 2, 4])          # row 10 is past total_q
    assert "outside" in _list_call(d, hp)[1]
    hp, k3 = _pages([0, 6], [2, 2], [0, 2, 4], [3, 5], [0, 2, 1])          # kv_indptr decreases
    assert "non-decreasing" in _list_call(d, hp)[1]
    hp, k4 = _pages([0, 6], [2, 2], [0, 2, 4], [31, 5], [0, 2, 4])         # 31 + 2 keys > 2 pages of 16
    assert _list_call(d, hp)[0] == 3
    hp, k5 = _pages([0, 6], [2, 2], [0, 2, 4], [3, 5], [0, 2, 4], [0, 1, 99, 3])
    st, msg = _list_call(d, hp)
    assert st == 1 and "kv_indices" in msg
    hp, k6 = _pages([0, 6], [2, 2], [0, 2, 4], None, [0, 2, 4])            # cache without cache_seqlens
    assert _list_call(d, hp)[0] == 1
    hp, k7 = _pages([0, 6], [2, 2])                                        # new tokens without cu_seqlens_knew
    assert _list_call(d, hp, kc=None, vc=None, kvi=None)[0] == 1


def test_rope_errors_before_the_device():
    lib = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(dims, rope, host):
        st = lib.attn_varlen_paged_rope_fwd(ctypes.byref(dims), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                            vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 16, 1, 0.1, None,
                                            None if rope is None else ctypes.byref(rope), vp(FAKE), vp(FAKE),
                                            ctypes.byref(host), None)
        return st, lib.vpk_last_error().decode()

    def rope(**kw):
        r = dict(cos=FAKE, sin=FAKE, max_positions=64, rotary_dim=128, interleaved=0)
        r.update(kw)
        return _lib.VpkRope(**r)

    d = _dims()
    hi, k = _host([0, 2, 4], [0, 2, 4], [3, 5])
    assert call(d, None, hi) == (1, "rope is NULL")
    for kw, frag in ((dict(rotary_dim=120), "rotary_dim"), (dict(rotary_dim=144), "rotary_dim"),
                     (dict(rotary_dim=0), "rotary_dim"), (dict(interleaved=2), "interleaved"),
                     (dict(max_positions=0), "max_positions"), (dict(cos=None), "rope->cos"),
                     (dict(sin=FAKE + 4), "rope->sin")):
        st, msg = call(d, rope(**kw), hi)
        assert st == 1 and frag in msg, (kw, msg)
    # positions: sequence 1 reaches Lc + Ln - 1 = 6; with 6 table rows that is past the end
    st, msg = call(d, rope(max_positions=6), hi)
    assert st == 1 and "sequence 1 reaches position 6" in msg
    # a sequence with more query rows than keys has no position for its first rows
    d2 = _dims(total_knew=2)
    hi, k = _host([0, 3, 4], [0, 1, 2], [1, 5])
    st, msg = call(d2, rope(), hi)
    assert st == 1 and "sequence 0" in msg and "query rows than keys" in msg


def test_device_scale_run_errors_before_the_device():
    lib = _lib.load()
    vp = ctypes.c_void_p
    st = lib.vpk_plan_run_device_scale(None, vp(FAKE), None, None, None, None, None, 0.1, vp(FAKE), vp(FAKE),
                                       vp(FAKE), None)
    assert st == 1 and b"plan is NULL" in lib.vpk_last_error()


def test_workspace_bound_host_only():
    lib = _lib.load()
    d = _lib.VpkDims(4, 100, 100, 32, 8, 128, 1000, 64, _lib.VPK_DTYPE_BF16)
    b0 = lib.vpk_workspace_bytes_upper_bound(ctypes.byref(d), 256, 0)
    b1 = lib.vpk_workspace_bytes_upper_bound(ctypes.byref(d), 256, 1)
    # the rope copies of q and k_new in bf16
    assert b1 - b0 >= 2 * (100 * 32 * 128 + 100 * 8 * 128)
    # more rows never need less
    d2 = _lib.VpkDims(4, 1000, 1000, 32, 8, 128, 1000, 64, _lib.VPK_DTYPE_BF16)
    assert lib.vpk_workspace_bytes_upper_bound(ctypes.byref(d2), 256, 0) >= b0 > 512
    bad = _lib.VpkDims(4, 100, 100, 30, 8, 128, 1000, 64, _lib.VPK_DTYPE_BF16)
    assert lib.vpk_workspace_bytes_upper_bound(ctypes.byref(bad), 256, 0) == 0
    assert lib.vpk_workspace_bytes_upper_bound(None, 256, 0) == 0
    st = lib.vpk_set_workspace(None, ctypes.c_void_p(FAKE + 8), 1 << 20)
    assert st == 1 and b"aligned" in lib.vpk_last_error()
    st = lib.vpk_set_workspace(None, ctypes.c_void_p(FAKE), 1024)
    assert st == 1 and b"at least" in lib.vpk_last_error()


def test_qkv_prob_errors_before_the_device():
    lib = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(dims, qp, kv=(0.02, 0.01), cache=FAKE):
        ks = (ctypes.c_float * 2)(*kv)
        qps = None if qp is None else (ctypes.c_float * 2)(*qp)
        st = lib.attn_varlen_paged_qkv_prob_fwd(ctypes.byref(dims), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                                vp(cache), vp(cache), vp(FAKE), vp(FAKE), 16, 1, 0.1, ks, qps, None,
                                                vp(FAKE), vp(FAKE), ctypes.byref(hi), None)
        return st, lib.vpk_last_error().decode()

    hi, keep = _host([0, 2, 4], [0, 2, 4], [3, 5])
    fp8 = _dims(kv_cache_dtype=2)
    st, msg = call(_dims(kv_cache_dtype=1), (0.01, 1 / 448))
    assert st == 1 and "fp8" in msg, msg
    st, msg = call(fp8, (0.01, 1 / 448), cache=None)
    assert st == 1 and "fp8" in msg, msg
    assert call(fp8, None) == (1, "qp_scale is NULL")
    for qp, frag in (((0.0, 1 / 448), "q_scale"), ((float("nan"), 1 / 448), "q_scale"),
                     ((0.01, 1 / 500), "p_scale"), ((0.01, float("inf")), "p_scale")):
        st, msg = call(fp8, qp)
        assert st == 1 and frag in msg, (qp, msg)
