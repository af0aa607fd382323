"""The page-list form (attn_varlen_paged_list_fwd) on the GPU.

With each block_table row turned into that sequence's page list (CSR) and
query rows given by start and length, the call must match the oracle
(attention within tolerance, appended cache bytes exact) and give the dense
call's bits; with the sequences' query rows moved elsewhere in q (other order, gaps
between them), each sequence's output rows and lse columns must move with
them, bit for bit, and rows no sequence names must stay untouched."""
import numpy as np
import pytest
import torch

import varlen_paged_kv_amd as vpk
from synth import make_custom

from gpu_util import DeviceCall, check_attention, oracle_full, say, to_np_out

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _csr(wl):
    """Page lists of the dense block_table: the first ceil(Lk / S) ids of each row,
    after two spare ids at the front (kv_indptr[0] = 2) and with b % 3 spare ids
    after each list (a list may hold more pages than its sequence needs)."""
    S = wl.page_size
    need = (wl.kv_lens() + S - 1) // S
    parts, indptr = [np.array([0, 1], np.int32)], [2]
    for b in range(wl.B):
        parts.append(wl.block_table[b, :need[b]].astype(np.int32))
        parts.append(np.full(b % 3, b % wl.num_pages, np.int32))
        indptr.append(indptr[-1] + int(need[b]) + b % 3)
    return np.array(indptr, np.int32), np.ascontiguousarray(np.concatenate(parts), np.int32)


CASES = {
    "mixed_bf16": lambda: make_custom(q_lens=[1, 37, 1, 300, 1], new_lens=[1, 37, 1, 300, 1],
                                      cache_lens=[500, 40, 1000, 0, 77], Hq=8, Hkv=2, D=128, page_size=16,
                                      causal=True, cache_dtype="bf16", seed=51),
    "mixed_fp8_S5": lambda: make_custom(q_lens=[3, 1, 70], new_lens=[3, 1, 70], cache_lens=[41, 300, 9],
                                        Hq=4, Hkv=1, D=64, page_size=5, causal=True, cache_dtype="fp8", seed=52),
    "no_cache_D64": lambda: make_custom(q_lens=[200, 3, 90], new_lens=[200, 3, 90], cache_lens=[0, 0, 0],
                                        Hq=4, Hkv=4, D=64, page_size=0, causal=True, cache_dtype=None,
                                        seed=54),
    "cache_only": lambda: make_custom(q_lens=[1, 1, 40], new_lens=None, cache_lens=[300, 1200, 64], Hq=8,
                                      Hkv=2, D=128, page_size=64, causal=True, cache_dtype="bf16", seed=53),
}


def _list_call(dc, q, q_start, q_len, out=None, lse=None):
    wl = dc.wl
    has_cache = wl.k_cache is not None
    indptr, indices = _csr(wl) if has_cache else (None, None)
    return vpk.attn_varlen_paged_list_fwd(
        q, q_start, q_len, dc.k_new, dc.v_new, wl.cu_seqlens_knew if dc.with_new else None,
        dc.k_cache, dc.v_cache, indptr, torch.from_numpy(indices).to(q.device) if has_cache else None,
        wl.cache_seqlens if has_cache else None, wl.page_size if has_cache else 0, wl.causal, wl.scale,
        wl.kv_scale if dc.fp8 else None, out=out, lse=lse, kv_indices_host=indices)


@pytest.mark.parametrize("case", sorted(CASES))
def test_page_lists_equal_dense_block_table(case):
    wl = CASES[case]()
    dc = DeviceCall(wl, with_new=wl.k_new is not None)
    say(f"[case] page lists {case}")
    ref_out, ref_lse = dc.run()
    kc0, vc0 = dc.cache_host()
    cu = wl.cu_seqlens_q.astype(np.int64)
    out, lse = _list_call(dc, dc.q, cu[:-1], np.diff(cu))
    torch.cuda.synchronize()
    ref = oracle_full(wl, with_new=dc.with_new)
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    "fp8" if dc.fp8 else "bf16", label=f"page lists {case}")
    if kc0 is not None:
        assert np.array_equal(kc0, ref["k_cache"]) and np.array_equal(vc0, ref["v_cache"]), f"{case}: cache bytes"
    assert np.array_equal(_bits(out), _bits(ref_out)), f"{case}: out differs"
    assert np.array_equal(_bits(lse), _bits(ref_lse)), f"{case}: lse differs"
    kc1, vc1 = dc.cache_host()
    if kc0 is not None:
        assert np.array_equal(kc0, kc1) and np.array_equal(vc0, vc1), f"{case}: cache bytes differ"
    say(f"[ok] page lists {case}: within the oracle tolerances, bitwise equal to the dense call")


@pytest.mark.parametrize("case", sorted(CASES))
def test_query_rows_anywhere(case):
    wl = CASES[case]()
    dc = DeviceCall(wl, with_new=wl.k_new is not None)
    ref_out, ref_lse = dc.run()
    torch.cuda.synchronize()
    cu = wl.cu_seqlens_q.astype(np.int64)
    ql = np.diff(cu)
    # sequences in reverse order with a gap of 3 rows before each
    starts = np.zeros(wl.B, np.int64)
    pos = 0
    for b in reversed(range(wl.B)):
        pos += 3
        starts[b] = pos
        pos += ql[b]
    T2 = int(pos + 2)
    q2 = torch.zeros((T2, wl.Hq, wl.D), dtype=torch.bfloat16, device=dc.q.device)
    for b in range(wl.B):
        q2[starts[b]:starts[b] + ql[b]] = dc.q[cu[b]:cu[b + 1]]
    out2 = torch.full((T2, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=dc.q.device)   # untouched rows keep 7
    lse2 = torch.full((wl.Hq, T2), 5.0, dtype=torch.float32, device=dc.q.device)
    _list_call(dc, q2, starts, ql, out=out2, lse=lse2)
    torch.cuda.synchronize()
    ref = oracle_full(wl, with_new=dc.with_new)
    o2f, l2f = to_np_out(out2), lse2.cpu().numpy().astype(np.float64)
    for b in range(wl.B):
        s2, n = int(starts[b]), int(ql[b])
        check_attention(o2f[s2:s2 + n], l2f[:, s2:s2 + n], ref["out"][cu[b]:cu[b + 1]], ref["lse"][:, cu[b]:cu[b + 1]],
                        "fp8" if dc.fp8 else "bf16", label=f"{case} moved seq {b}")
    o_ref, l_ref, o2, l2 = _bits(ref_out), _bits(ref_lse), _bits(out2), _bits(lse2)
    named = np.zeros(T2, bool)
    for b in range(wl.B):
        s2, n = int(starts[b]), int(ql[b])
        named[s2:s2 + n] = True
        assert np.array_equal(o2[s2:s2 + n], o_ref[cu[b]:cu[b + 1]]), f"{case}: seq {b} out differs"
        assert np.array_equal(l2[:, s2:s2 + n], l_ref[:, cu[b]:cu[b + 1]]), f"{case}: seq {b} lse differs"
    seven = _bits(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]
    five = _bits(torch.full((1,), 5.0, dtype=torch.float32))[0]
    assert np.all(o2[~named] == seven) and np.all(l2[:, ~named] == five), f"{case}: rows no sequence names changed"
    say(f"[ok] query rows anywhere {case}: rows moved bit for bit, others untouched")
