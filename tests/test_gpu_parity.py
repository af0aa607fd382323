"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

* append and page gather: bit-exact (cache bytes; one-hot gather probe);
* attention values: max-abs 2e-2 (3e-2 with an fp8 cache), mean-abs 2e-3,
  lse max-abs 1e-3, rows without visible keys exactly 0 / -inf;
* full-size workloads in the launch configuration the bench times, checked on
  sampled sequences the oracle computes one by one.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import varlen_paged_kv_amd as vpk
from synth import make_custom, make_workload
from synth.workloads import to_bf16_bits

from gpu_util import (DeviceCall, check_attention, dev_bf16, dev_i32, dev_u8, oracle_full, run_and_check, say,
                      to_np_out)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    vpk.set_option("force_splits", 0)
    vpk.set_option("persistent", -1)
    vpk.set_option("num_cus", 0)
    vpk.set_option("mixed_grid", 1)


_run_and_check = run_and_check


def test_tiny_workload():
    _run_and_check(make_workload("tiny"), "tiny")


SMALL = [
    # label, q_lens, new_lens, cache_lens, Hq, Hkv, D, S, causal, cache
    ("ragged_S16_g4", [1, 37, 200, 129], [1, 37, 200, 129], [0, 65, 300, 1000], 8, 2, 128, 16, True, "bf16"),
    ("noncausal_S5_g1_D64", [3, 70, 1], [3, 70, 1], [10, 0, 257], 4, 4, 64, 5, False, "bf16"),
    ("S1_g8", [2, 9], [2, 9], [130, 5], 8, 1, 128, 1, True, "bf16"),
    ("S64_fp8", [100, 1, 1, 33], [100, 1, 1, 33], [0, 900, 64, 129], 8, 2, 128, 64, True, "fp8"),
    ("fp8_D64_S4_noncausal", [5, 66], [5, 66], [31, 2], 4, 2, 64, 4, False, "fp8"),
    ("no_cache_prefill", [1, 130, 257, 64], [1, 130, 257, 64], [0, 0, 0, 0], 8, 2, 128, 0, True, None),
    ("no_cache_noncausal_D64", [17, 3, 300], [17, 3, 300], [0, 0, 0], 4, 1, 64, 0, False, None),
    ("q_longer_than_kv", [10, 4], [3, 0], [0, 2], 4, 2, 128, 16, True, "bf16"),
    ("empty_sequences", [0, 5, 0, 1], [0, 5, 0, 0], [3, 0, 0, 0], 4, 2, 128, 16, True, "bf16"),
    ("zero_kv_all_rows_dead", [4], [0], [0], 4, 2, 128, 16, True, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    label, ql, nl, cl, hq, hkv, d, s, causal, cache = case
    wl = make_custom(q_lens=ql, new_lens=nl, cache_lens=cl, Hq=hq, Hkv=hkv, D=d, page_size=s,
                     causal=causal, cache_dtype=cache, seed=zlib.crc32(label.encode()) % 1000)
    _run_and_check(wl, label)


def test_cache_only_no_new_tokens():
    wl = make_custom(q_lens=[2, 1, 7], new_lens=None, cache_lens=[5, 300, 64], Hq=8, Hkv=2, D=128,
                     page_size=16, seed=11)
    _run_and_check(wl, "cache_only")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_poisoned_unused_slots(cache):
    wl = make_custom(q_lens=[3, 1, 77], new_lens=[3, 1, 77], cache_lens=[13, 200, 5], Hq=8, Hkv=2,
                     D=128, page_size=16, cache_dtype=cache, seed=12, poison=True)
    _run_and_check(wl, f"poison_{cache}")


def _medium(seed=13, cache="bf16"):
    return make_custom(q_lens=[1, 1, 150, 3], new_lens=[1, 1, 150, 3], cache_lens=[2000, 700, 900, 64],
                       Hq=8, Hkv=2, D=128, page_size=16, cache_dtype=cache, seed=seed)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_split_invariance(cache):
    wl = _medium(cache=cache)
    ref = oracle_full(wl)
    kind = "fp8" if cache == "fp8" else "bf16"
    results = []
    for n in (1, 2, 7):
        vpk.set_option("force_splits", n)
        say(f"[case] split_invariance {cache} force_splits={n}")
        out, lse = DeviceCall(wl).run()
        torch.cuda.synchronize()
        o, l = to_np_out(out), lse.cpu().numpy().astype(np.float64)
        check_attention(o, l, ref["out"], ref["lse"], kind, label=f"splits={n}")
        results.append((o, l))
    for o, l in results[1:]:
        assert np.abs(l - results[0][1]).max() <= 1e-5
        assert np.abs(o - results[0][0]).max() <= 1.6e-2


def test_persistent_schedule_is_bitwise_identical():
    wl = _medium(seed=14)
    outs = []
    for mode in (0, 1):
        vpk.set_option("persistent", mode)
        say(f"[case] persistent={mode}")
        out, lse = DeviceCall(wl).run()
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_long_persistent_queues(cache):
    """One CU assumed: every workgroup's queue spans several chunks of entries
    (the queue metadata is staged through LDS chunk by chunk), with splits."""
    wl = make_custom(q_lens=[1, 40, 300, 3, 1, 77], new_lens=[1, 40, 300, 3, 1, 77],
                     cache_lens=[2000, 700, 900, 64, 5000, 0], Hq=8, Hkv=2, D=128, page_size=16,
                     cache_dtype=cache, seed=17)
    vpk.set_option("num_cus", 1)
    vpk.set_option("force_splits", 7)
    _run_and_check(wl, f"long_queues_{cache}")


def test_deterministic_and_idempotent_append():
    wl = _medium(seed=15)
    dc = DeviceCall(wl)
    say("[case] determinism run 1")
    o1, l1 = dc.run()
    k1, v1 = dc.cache_host()
    say("[case] determinism run 2 (same cache, append repeated)")
    o2, l2 = dc.run()
    k2, v2 = dc.cache_host()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_non_default_stream():
    wl = _medium(seed=16)
    s = torch.cuda.Stream()
    dc = DeviceCall(wl)
    say("[case] non-default stream")
    with torch.cuda.stream(s):
        out, lse = dc.run(stream=s)
    s.synchronize()
    ref = oracle_full(wl)
    check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"], ref["lse"],
                    label="stream")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_append_entry_point_bit_exact(cache):
    wl = make_custom(q_lens=[5, 1, 40], new_lens=[5, 1, 40], cache_lens=[3, 64, 0], Hq=4, Hkv=2,
                     D=128, page_size=16, cache_dtype=cache, seed=17)
    dc = DeviceCall(wl)
    say(f"[case] kv_cache_append {cache}")
    for _ in range(2):   # idempotent
        vpk.kv_cache_append(dc.k_new, dc.v_new, dc.cu_kn, dc.k_cache, dc.v_cache, dc.bt, dc.cl,
                            wl.page_size, wl.kv_scale if cache == "fp8" else None,
                            host_index=dc.host)
        kc, vc = dc.cache_host()
        rk, rv = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, wl.k_cache, wl.v_cache,
                               wl.block_table, wl.cache_seqlens, wl.page_size, cache, wl.kv_scale)
        assert np.array_equal(kc, rk) and np.array_equal(vc, rv)


@pytest.mark.parametrize("scale", [1.0, 0.0137, 37.0, 2.0 ** -12])
def test_fp8_encoder_every_bf16_pattern(scale):
    # all 65536 bf16 bit patterns (NaN and inf included) as 512 new tokens of one
    # sequence with Hkv = 1, D = 128, appended into an fp8 cache
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 1, 128)
    P, S = 32, 16
    k_cache = np.zeros((P, S, 1, 128), np.uint8)
    bt = np.random.default_rng(18).permutation(P).astype(np.int32)[None, :]
    cu = np.array([0, 512], np.int32)
    cl = np.array([0], np.int32)
    ks = (np.float32(scale), np.float32(scale * 3))
    say(f"[case] fp8 encoder all patterns scale={scale}")
    kc_d, vc_d = dev_u8(k_cache), dev_u8(k_cache.copy())
    kn = dev_bf16(bits)
    vn = dev_bf16(bits[::-1].copy())
    vpk.kv_cache_append(kn, vn, dev_i32(cu), kc_d, vc_d, dev_i32(bt), dev_i32(cl), S, ks,
                        host_index=dict(cu_seqlens_knew=cu, cache_seqlens=cl, block_table=bt))
    rk, rv = oracle.append(bits, bits[::-1].copy(), cu, k_cache, k_cache.copy(), bt, cl, S, "fp8", ks)
    assert np.array_equal(kc_d.cpu().numpy(), rk)
    assert np.array_equal(vc_d.cpu().numpy(), rv)


def _one_hot_case(S, cache, seed, all_codes_v=False):
    """Keys orthogonal (40 * e_code), each query aimed at one visible key: out must be that V row.

    all_codes_v (fp8): the V rows of each sequence and kv head run through every finite
    non-zero e4m3fn code (subnormals, negatives and the largest magnitudes included), so
    the widening of every such code reaches an output bit for bit."""
    rng = np.random.default_rng(seed)
    D, Hq, Hkv = 128, 8, 2
    g = Hq // Hkv
    lens = [(3, 90), (5, 0), (1, 127), (20, 20)]          # (q_len, cache_len); new = q_len
    B = len(lens)
    ql = np.array([a for a, _ in lens]); cl = np.array([c for _, c in lens])
    lk = ql + cl
    wl = make_custom(q_lens=ql, new_lens=ql, cache_lens=cl, Hq=Hq, Hkv=Hkv, D=D, page_size=S,
                     causal=True, cache_dtype=cache, seed=seed)
    fp8 = cache == "fp8"
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    all_codes = []
    K = np.zeros((int(lk.sum()), Hkv, D), np.float32)
    V = np.zeros_like(K)
    for b in range(B):
        codes = rng.permutation(D)[: lk[b]]
        for h in range(Hkv):
            for j in range(lk[b]):
                K[cu_k[b] + j, h, codes[j]] = 40.0
                if fp8 and all_codes_v:
                    # codes 1..126 and 129..254 (0x7F / 0xFF are NaN, 0x80 is -0, whose
                    # sum with +0 products is +0), in turn over keys and elements
                    finite = np.concatenate([np.arange(1, 127), np.arange(129, 255)])
                    V[cu_k[b] + j, h] = oracle.e4m3fn_decode(
                        finite[(np.arange(D) + (j * 2 + h) * D) % len(finite)].astype(np.uint8))
                elif fp8:   # distinct e4m3 values per key: code pattern
                    V[cu_k[b] + j, h] = oracle.e4m3fn_decode(((np.arange(D) * 3 + j * 5 + h) % 100 + 8).astype(np.uint8))
                else:
                    V[cu_k[b] + j, h] = rng.standard_normal(D).astype(np.float32)
        all_codes.append(codes)
    Vb = to_bf16_bits(V)
    Q = np.zeros((int(ql.sum()), Hq, D), np.float32)
    target = np.zeros((int(ql.sum()), Hq), np.int64)
    for b in range(B):
        codes = all_codes[b]
        for i in range(ql[b]):
            t = wl.cu_seqlens_q[b] + i
            for h in range(Hq):
                last = i + lk[b] - ql[b]             # last visible key (end-aligned causal)
                j = int(rng.integers(0, last + 1))
                target[t, h] = cu_k[b] + j
                Q[t, h, codes[j]] = 40.0
    wl.q = to_bf16_bits(Q)
    new_idx = np.concatenate([np.arange(cu_k[b] + cl[b], cu_k[b + 1]) for b in range(B)])
    Kb = to_bf16_bits(K)
    wl.k_new, wl.v_new = Kb[new_idx], Vb[new_idx]
    if fp8:
        wl.kv_scale = (np.float32(1.0), np.float32(1.0))
    for b in range(B):
        for j in range(cl[b]):
            page, slot = wl.block_table[b, j // S], j % S
            if fp8:
                wl.k_cache[page, slot] = oracle.e4m3fn_encode(K[cu_k[b] + j])
                wl.v_cache[page, slot] = oracle.e4m3fn_encode(V[cu_k[b] + j])
            else:
                wl.k_cache[page, slot] = Kb[cu_k[b] + j]
                wl.v_cache[page, slot] = Vb[cu_k[b] + j]
    expect = np.zeros((int(ql.sum()), Hq, D), np.uint16)
    for t in range(int(ql.sum())):
        for h in range(Hq):
            expect[t, h] = Vb[target[t, h], h // g]
    return wl, expect


@pytest.mark.parametrize("S", [1, 4, 16, 64])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_one_hot_gather_probe_bit_exact(S, cache):
    wl, expect = _one_hot_case(S, cache, seed=S * 10 + (cache == "fp8"))
    say(f"[case] one-hot probe S={S} cache={cache}")
    out, _ = DeviceCall(wl).run()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"first mismatches at {bad[:5].tolist()}"


@pytest.mark.parametrize("S", [16, 64])
def test_one_hot_probe_every_e4m3_code(S):
    """The fp8 widening in the attention kernels (decode-mode and prefill-mode rows) is exact
    on every finite non-zero e4m3fn code: each output row is its V row's decoded codes."""
    wl, expect = _one_hot_case(S, "fp8", seed=77 + S, all_codes_v=True)
    # the targeted rows reach every finite non-zero code (checked on the host)
    vals = (expect.astype(np.uint32) << 16).view(np.float32)
    reached = set(np.unique(oracle.e4m3fn_encode(vals.reshape(-1))).tolist())
    assert set(range(1, 127)) | set(range(129, 255)) <= reached
    say(f"[case] one-hot probe over every e4m3 code S={S}")
    out, _ = DeviceCall(wl).run()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"first mismatches at {bad[:5].tolist()}"


FULL = ["varlen_prefill", "paged_decode", "chunked_prefill", "mixed_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads(name):
    """The four full-size workloads in the launch configuration the bench times: every
    sequence's attention against the oracle's whole call, every appended byte exact."""
    wl = make_workload(name)
    say(f"[case] full size {name}: Tq={wl.Tq} Tn={wl.Tn} pages={wl.num_pages}")
    dc = DeviceCall(wl)
    out, lse = dc.run()
    torch.cuda.synchronize()
    o_all = to_np_out(out)
    l_all = lse.cpu().numpy().astype(np.float64)
    kc, vc = dc.cache_host()
    say(f"[step] {name}: GPU call done, running the oracle on all {wl.B} sequences")
    ref = oracle_full(wl)
    if kc is not None:
        assert np.array_equal(kc, ref["k_cache"]) and np.array_equal(vc, ref["v_cache"]), f"{name}: cache bytes"
    kind = "fp8" if wl.cache_dtype == "fp8" else "bf16"
    errs = check_attention(o_all, l_all, ref["out"], ref["lse"], kind, label=f"{name} (all sequences)")
    # per sequence too, so that a bad sequence is not averaged away in mean-abs
    for b in range(wl.B):
        s, e = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
        if e > s:
            check_attention(o_all[s:e], l_all[:, s:e], ref["out"][s:e], ref["lse"][:, s:e], kind,
                            label=f"{name} seq {b}")
    say(f"[ok] {name}: all {wl.B} sequences; max {errs[0]:.2e} mean {errs[1]:.2e} lse {errs[2]:.2e}")


MIXED_CASES = [
    # label, q_lens, cache_lens, Hq, Hkv, D, S, cache
    ("bf16_D128", [1, 300, 1, 1, 40, 1], [3000, 100, 700, 0, 50, 5000], 8, 2, 128, 16, "bf16"),
    ("fp8_D128_S64", [2, 1, 513, 1, 1], [900, 4000, 0, 64, 2500], 8, 2, 128, 64, "fp8"),
    ("bf16_D64_g8", [1, 1, 130, 1], [2000, 33, 70, 1000], 16, 2, 64, 16, "bf16"),
    ("fp8_D64_S5", [3, 90, 1, 1], [77, 10, 900, 3], 4, 1, 64, 5, "fp8"),
]


@pytest.mark.parametrize("persistent", [0, 1])
@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("case", MIXED_CASES, ids=[c[0] for c in MIXED_CASES])
def test_mixed_batches_one_launch_and_two_grids(case, grid, persistent):
    """A batch with both decode-mode and prefill-mode items: in one launch (the mixed grid, decode
    items on eight waves) and in two grids, with and without persistent queues, against the oracle."""
    label, ql, cl, hq, hkv, d, s, cache = case
    vpk.set_option("mixed_grid", grid)
    vpk.set_option("persistent", persistent)
    try:
        wl = make_custom(q_lens=ql, new_lens=ql, cache_lens=cl, Hq=hq, Hkv=hkv, D=d, page_size=s, causal=True,
                         cache_dtype=cache, seed=zlib.crc32(label.encode()) % 1000)
        _run_and_check(wl, f"mixed {label} grid={grid} persistent={persistent}")
    finally:
        vpk.set_option("mixed_grid", 1)
