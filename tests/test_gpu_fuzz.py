"""Seeded fuzz tier: 200 random small batches through the C ABI against the oracle.

Each case draws its own shape from a seeded generator: batch 1..8, lengths
0..300 (empty sequences, rows that see no key, q longer than kv), page sizes
1, 4, 5, 16, 64, head_dim 64 / 128, 1, 4 or 8 query heads per kv head,
causal or not, no cache / bf16 cache / fp8 cache, calls with and without new
tokens.  Some cases pin a decode-mode item of exactly 32 packed rows and a
prefill-mode item of 33..36 rows, the boundary between the two kernels.
Attention must be within the tolerances, appended cache bytes exact.
"""
import numpy as np
import pytest

import varlen_paged_kv_amd as vpk
from synth import make_custom

from gpu_util import run_and_check

N_CASES = 200


def fuzz_case(i: int):
    """Shape and lengths of fuzz case i (pure function of i)."""
    rng = np.random.default_rng(9000 + i)
    D = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    cache = [None, "bf16", "fp8"][int(rng.integers(0, 3))]
    S = int(rng.choice([1, 4, 5, 16, 64])) if cache else 0
    causal = bool(rng.integers(0, 2))
    B = int(rng.integers(1, 9))
    with_new = cache is None or bool(rng.random() < 0.85)

    def length():
        r = rng.random()
        if r < 0.15:
            return 0
        if r < 0.35:
            return 1
        if r < 0.5:
            return int(rng.integers(2, 16))
        return int(rng.integers(16, 301))

    ql = [length() for _ in range(B)]
    nl = [q if rng.random() < 0.7 else length() for q in ql] if with_new else None
    cl = [length() for _ in range(B)] if cache else [0] * B
    if i % 5 == 0:
        # a decode-mode item of exactly 32 packed rows next to a prefill-mode
        # one just above the boundary
        ql[0] = 32 // g
        ql[-1] = 32 // g + 1 if B > 1 else ql[-1]
        if with_new:
            nl[0] = ql[0]
            if B > 1:
                nl[-1] = ql[-1]
    if cache is None and sum(nl) == 0:
        nl[0] = ql[0] = max(ql[0], 1)
    return dict(q_lens=ql, new_lens=nl, cache_lens=cl, Hq=g * Hkv, Hkv=Hkv, D=D, page_size=S,
                causal=causal, cache_dtype=cache, seed=9000 + i)


def test_fuzz_cases_cover_the_boundaries():
    """Host-side check that the drawn cases reach the regimes the tier is for."""
    cases = [fuzz_case(i) for i in range(N_CASES)]
    assert {c["cache_dtype"] for c in cases} == {None, "bf16", "fp8"}
    assert {c["D"] for c in cases} == {64, 128}
    assert {c["Hq"] // c["Hkv"] for c in cases} == {1, 4, 8}
    assert {c["page_size"] for c in cases if c["cache_dtype"]} == {1, 4, 5, 16, 64}
    assert any(c["new_lens"] is None for c in cases)
    assert any(0 in c["q_lens"] for c in cases)
    rows = [q * (c["Hq"] // c["Hkv"]) for c in cases for q in c["q_lens"]]
    assert 32 in rows and any(32 < r <= 40 for r in rows)
    assert {c["causal"] for c in cases} == {True, False}


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz(i):
    spec = fuzz_case(i)
    wl = make_custom(**spec)
    run_and_check(wl, f"fuzz {i} q={spec['q_lens']} new={spec['new_lens']} cache={spec['cache_lens']}",
                  with_new=spec["new_lens"] is not None)


N_SPLIT_CASES = 100


@pytest.fixture
def _planner_knobs():
    yield
    vpk.set_option("force_splits", 0)
    vpk.set_option("split_min_keys", 256)
    vpk.set_option("persistent", -1)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_SPLIT_CASES))
def test_fuzz_split_and_persistent(i, _planner_knobs):
    """The same draws with every tile cut into 2, 3 or 7 key parts (64-key minimum, so short ranges split
    too; the LSE merge then combines them) and persistent queues forced on or off."""
    spec = fuzz_case(i)
    splits = (2, 3, 7)[i % 3]
    persistent = (i // 3) % 2
    vpk.set_option("force_splits", splits)
    vpk.set_option("split_min_keys", 64)
    vpk.set_option("persistent", persistent)
    wl = make_custom(**spec)
    run_and_check(wl, f"fuzz {i} splits {splits} persistent {persistent}", with_new=spec["new_lens"] is not None)
