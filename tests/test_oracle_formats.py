"""Pins for the oracle's number formats (CPU only).

e4m3fn decode/encode are pinned against torch's float8_e4m3fn type (a library
implementation of the same OCP format) and against hand-written definitional
values in tests/golden/e4m3fn_codes.txt; the bf16 widening is pinned against
torch's bfloat16.
"""
import os

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_every_code():
    ours = e4m3fn_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # sign of zero kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_golden_values():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 15
    for code_hex, val in rows:
        got = e4m3fn_decode(np.array([int(code_hex, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code_hex
        else:
            want = float(val)
            assert got == want and np.signbit(got) == np.signbit(want), (code_hex, got, want)


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3fn_encode(vals), codes)


@pytest.mark.parametrize("scale", [1.0, 4.53125 / 448.0, 0.0137, 37.0, 2.0 ** -12])
def test_encode_all_bf16_patterns_against_torch(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (x32 * inv).astype(np.float32)
    ours = e4m3fn_encode(prod)
    t = torch.from_numpy(prod.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a = np.abs(prod.astype(np.float64))
    nan = np.isnan(prod)
    # torch's cast is finite-preserving below 464 (it rounds to nearest even there)
    ok = (~nan) & (a < 464.0)
    assert np.array_equal(ours[ok], t[ok])
    # beyond: saturate to +-448 with the sign kept
    sat = (~nan) & (a >= 464.0)
    want = np.where(np.signbit(prod[sat]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(ours[sat], want)
    # NaN stays NaN, sign kept
    assert np.all((ours[nan] & 0x7F) == 0x7F)
    assert np.array_equal(ours[nan] >> 7, np.signbit(prod[nan]).astype(np.uint8))


def test_encode_ties_go_to_even_code():
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> 0x38; between 1.125 and 1.25 -> 0x3A
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, -464.0, 1e30, -np.inf, np.inf],
                 np.float32)
    got = e4m3fn_encode(x)
    assert got.tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xFE, 0x7E, 0xFE, 0x7E]


def test_bf16_widening_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
