"""Pins of the oracle's number formats against definitions it does not share.

* e4m3 decode  -> torch.float8_e4m3fn (a library decoder) and known points of
                  the OCP E4M3FN definition.
* e4m3 encode  -> an independent nearest-value table search (ties to the even
                  mantissa, saturating), torch's float32 -> float8_e4m3fn cast
                  in its non-overflowing range, and the round-trip identity on
                  every finite code.
* e8m0 decode  -> torch.float8_e8m0fnu.
* bf16 round   -> torch's float32 -> bfloat16 cast.

The structured input sets hit every rounding decision: all sign/exponent/top
mantissa-bit combinations with the sticky bits empty, single-bit and full,
plus random float32 bit patterns.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F


def _structured_f32():
    """float32 bit patterns covering every (sign, exponent, top 8 mantissa
    bits) combination with several low-bit (sticky) patterns."""
    hi = np.arange(1 << 17, dtype=np.uint64) << 15          # sign|exp|top-8 mantissa
    lows = np.array([0, 1, 0x3FFF, 0x4000, 0x4001, 0x7FFF], dtype=np.uint64)
    bits = (hi[:, None] | lows[None, :]).reshape(-1).astype(np.uint32)
    rnd = np.random.default_rng(7).integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([bits, rnd]).view(np.float32)


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


# ---------------------------------------------------------------- e4m3 ----
def test_e4m3_decode_matches_torch_all_codes():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(F.e4m3_decode(c), ref)


def test_e4m3_decode_known_points():
    d = lambda b: float(F.e4m3_decode(np.array([b], np.uint8))[0])
    assert d(0x7E) == 448.0                 # largest finite value
    assert d(0x08) == 2.0 ** -6             # smallest normal
    assert d(0x01) == 2.0 ** -9             # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9         # largest subnormal
    assert d(0x38) == 1.0
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0xFE) == -448.0


def test_e4m3_finite_values_strictly_increasing():
    v = F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert v.size == 127


def test_e4m3_round_trip_identity_every_finite_code():
    c = _finite_codes()
    assert c.size == 254                    # 253 distinct values, +0 and -0
    np.testing.assert_array_equal(F.e4m3_encode(F.e4m3_decode(c)), c)


def _table_search_encode(x32):
    """Independent encoder: nearest finite e4m3 value by search over the
    sorted value table; on a tie the code with the even mantissa wins; beyond
    448 saturate; the sign is copied."""
    pos_codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = F.e4m3_decode(pos_codes)
    x = np.asarray(x32, np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, vals.size - 1)
    lo = np.clip(hi - 1, 0, vals.size - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((pos_codes[hi] & 1) == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo])
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def test_e4m3_encode_matches_table_search():
    x = _structured_f32()
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(F.e4m3_encode(x), _table_search_encode(x))


def test_e4m3_encode_matches_torch_in_range():
    x = _structured_f32()
    x = x[np.isfinite(x) & (np.abs(x) <= 464.0)]   # torch does not saturate above
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e4m3_encode(x), ref)


def test_e4m3_encode_saturates_and_keeps_nan():
    x = np.array([448.0, 463.9, 464.0, 464.1, 1e30, np.inf, -500.0, -np.inf, np.nan], np.float32)
    got = F.e4m3_encode(x)
    np.testing.assert_array_equal(got[:8], [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert got[8] & 0x7F == 0x7F


def test_e4m3_ties_go_to_even():
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> 0x38; between 1.125 and 1.25 -> 0x3A
    np.testing.assert_array_equal(F.e4m3_encode(np.array([1.0625, 1.1875], np.float32)), [0x38, 0x3A])
    # half the smallest subnormal rounds to zero, a hair above rounds up
    np.testing.assert_array_equal(
        F.e4m3_encode(np.array([2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1))], np.float32)),
        [0x00, 0x01])


# ---------------------------------------------------------------- e8m0 ----
def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).double().numpy()
    got = F.e8m0_decode(b)
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


# ---------------------------------------------------------------- bf16 ----
def test_bf16_round_matches_torch():
    x = _structured_f32()
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_round(x)
    fin = np.isfinite(x)
    np.testing.assert_array_equal(got[fin], ref[fin])
    nan = np.isnan(x)
    assert np.all(np.isnan(F.bf16_decode(got[nan])))


def test_bf16_decode_exact():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(F.bf16_decode(b), ref)


@pytest.mark.parametrize("v,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (1.00390625, 0x3F80),
                                    (1.01171875, 0x3F82), (3.0e38, 0x7F62)])
def test_bf16_known_points(v, bits):
    assert int(F.bf16_round(np.array([v], np.float32))[0]) == bits
