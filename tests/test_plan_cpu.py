"""Host planner checks (no GPU): the work list covers every (sequence, query
head, token) row exactly once, with exactly the keys that row may see, split
parts tile the key range, and the persistent queues partition the items.

The facts checked are independent of the planner's code: visible keys of token
t are j < Lk and, when causal, j <= t + Lk - Lq; packed rows are token * g +
head_in_group."""
import numpy as np
import pytest

import varlen_paged_kv_amd as vpk
from synth import make_custom, make_workload

BLOCK_N = 64


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    vpk.set_option("force_splits", 0)
    vpk.set_option("persistent", -1)
    vpk.set_option("split_min_keys", 256)


def _plan(wl, num_cus=256, causal=None):
    return vpk.plan_debug(batch=wl.B, num_q_heads=wl.Hq, num_kv_heads=wl.Hkv, head_dim=wl.D,
                          cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_knew=wl.cu_seqlens_knew,
                          cache_seqlens=wl.cache_seqlens, block_table=wl.block_table,
                          page_size=wl.page_size if wl.k_cache is not None else 1,
                          causal=wl.causal if causal is None else causal, num_cus=num_cus,
                          has_cache=wl.k_cache is not None, num_pages=wl.num_pages or None,
                          kv_cache_dtype=wl.cache_dtype or "bf16")


def _check_coverage(wl, items, causal, nq=0):
    g = wl.Hq // wl.Hkv
    ql, kl = wl.q_lens(), wl.kv_lens()
    tiles = {}
    for it in items:
        seq, row0, nrows, kvh, kb, ke, part, queue = (int(x) for x in it)
        assert 0 <= seq < wl.B and 0 <= kvh < wl.Hkv
        assert 1 <= nrows <= 256 and 0 <= row0 and row0 + nrows <= ql[seq] * g   # prefill tiles: 256 rows
        assert kb % BLOCK_N == 0 and 0 <= kb and kb <= ke <= kl[seq]
        assert queue == -1 or 0 <= queue < nq
        tiles.setdefault((seq, kvh, row0, nrows), []).append((kb, ke, part))
    # rows: for each (seq, kv head) the tiles partition [0, Lq * g)
    for b in range(wl.B):
        for h in range(wl.Hkv):
            spans = sorted((r0, r0 + n) for (s, kh, r0, n) in tiles if s == b and kh == h)
            cur = 0
            for a, e in spans:
                assert a == cur
                cur = e
            assert cur == ql[b] * g
    # keys: the parts of a tile partition [0, kend) with kend the last row's bound
    for (seq, kvh, row0, nrows), parts in tiles.items():
        t_last = (row0 + nrows - 1) // g
        kend = kl[seq]
        if causal:
            kend = max(0, min(kend, t_last + kl[seq] - ql[seq] + 1))
        parts.sort()
        cur = 0
        for kb, ke, part in parts:
            assert kb == cur or (kb == ke == cur)
            cur = ke
        assert cur == kend
        if len(parts) == 1:
            assert parts[0][2] == -1
        else:
            offs = sorted(p[2] for p in parts)
            assert all(o >= 0 for o in offs)
            assert offs == [offs[0] + s * nrows for s in range(len(parts))]
        if wl.k_cache is not None:
            for kb, ke, _ in parts:
                if ke > kb:
                    assert (ke - 1) // wl.page_size - kb // wl.page_size + 1 <= 1024


@pytest.mark.parametrize("name", ["tiny", "varlen_prefill", "paged_decode", "chunked_prefill", "mixed_fp8"])
def test_workload_plans_cover_every_row_once(name):
    wl = make_workload(name, lengths_only=True)
    items, nq = _plan(wl)
    _check_coverage(wl, items, wl.causal, nq=nq)


def test_decode_is_split_to_fill_the_gpu():
    wl = make_workload("paged_decode", lengths_only=True)
    items, _ = _plan(wl)
    assert len(items) >= 2 * 256 * 2 // 2          # split parts fill the slots
    assert (items[:, 6] >= 0).sum() > 0


@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths(causal):
    # empty q rows, empty KV (zero cache and zero new), q longer than kv, S = 1 and 5
    for S in (1, 5, 16):
        wl = make_custom(q_lens=[0, 3, 7, 1, 130], new_lens=[0, 0, 2, 1, 130],
                         cache_lens=[5, 0, 0, 300, 17], Hq=4, Hkv=2, D=64, page_size=S, seed=3, lengths_only=True)
        items, nq = _plan(wl, causal=causal)
        _check_coverage(wl, items, causal, nq=nq)
        # the sequence with no keys still gets items (they write zeros / -inf)
        assert any(int(it[0]) == 1 for it in items)


@pytest.mark.parametrize("n", [1, 2, 7])
def test_forced_splits(n):
    vpk.set_option("force_splits", n)
    wl = make_custom(q_lens=[1, 40, 3], new_lens=[1, 40, 3], cache_lens=[700, 100, 0], Hq=8, Hkv=2,
                     D=128, page_size=16, seed=4, lengths_only=True)
    items, nq = _plan(wl)
    _check_coverage(wl, items, True, nq=nq)
    for (seq, kvh, row0, nrows) in {tuple(int(x) for x in it[:4]) for it in items}:
        parts = [it for it in items if tuple(int(x) for x in it[:4]) == (seq, kvh, row0, nrows)]
        nblk = -(-int(max(it[5] for it in parts)) // BLOCK_N)
        assert len(parts) == min(n, max(nblk, 1))


def test_long_ranges_are_split_for_the_page_list():
    # page_size 1: one item may not span more than 1024 pages
    wl = make_custom(q_lens=[1], new_lens=[1], cache_lens=[5000], Hq=2, Hkv=1, D=64, page_size=1, seed=5, lengths_only=True)
    items, nq = _plan(wl)
    _check_coverage(wl, items, True, nq=nq)
    assert len(items) >= 5


def test_persistent_queues_partition_items():
    vpk.set_option("persistent", 1)
    wl = make_workload("mixed_fp8", lengths_only=True)
    items, nq = _plan(wl, num_cus=64)
    assert 0 < nq <= 64 + 128                  # queues: one per prefill-mode slot (1 per CU), one per decode-mode slot (2 per CU)
    _check_coverage(wl, items, True, nq=nq)
    q = items[:, 7]
    assert np.all(np.diff(q) >= 0)            # grouped by queue, in queue order
    assert set(q.tolist()) == set(range(nq))
