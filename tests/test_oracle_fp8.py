"""Pins of the oracle's FP8 E4M3FN codec against things other than itself.

* the format's defining special values (largest finite, smallest subnormal and
  normal, NaN codes, signed zero);
* PyTorch's ``float8_e4m3fn`` CPU conversion (an independent library
  implementation of the same OCP format) for decode of all 256 codes and for
  encode of many values up to the saturation bound;
* an exhaustive nearest-value search (brute force) with the even-mantissa tie
  rule, on values that include every midpoint between adjacent codes.
"""

import math

import numpy as np
import pytest
import torch

from oracle import decode_table, fp8_decode, fp8_encode, FP8_MAX


def test_special_values():
    t = decode_table()
    assert t[0x00] == 0.0 and not math.copysign(1, t[0x00]) < 0
    assert t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and FP8_MAX == 448.0
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)      # codes 0..0x7E are increasing


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(mine[~nan]))


def _all_finite_magnitudes():
    t = decode_table()[:0x7F]
    return t


def _brute_encode(x: float) -> int:
    """Nearest finite code by exhaustive search; ties -> even mantissa."""
    if abs(x) >= 448.0:
        return 0x7E | (0x80 if math.copysign(1, x) < 0 else 0)
    mags = _all_finite_magnitudes()
    a = abs(x)
    best = None
    for c in range(0x7F):
        err = abs(mags[c] - a)
        if best is None or err < best[0] or (err == best[0] and (c & 1) == 0):
            best = (err, c)
    c = best[1]
    return c | (0x80 if math.copysign(1, x) < 0 else 0)


def test_encode_matches_brute_force_on_midpoints():
    mags = _all_finite_magnitudes()
    mids = (mags[:-1] + mags[1:]) / 2.0
    vals = np.concatenate([mags, mids, mids * (1 + 1e-12), mids * (1 - 1e-12),
                           [447.9, 448.0, 455.9, 1e6, 2.0 ** -10, 2.0 ** -11]])
    vals = np.concatenate([vals, -vals])
    mine = fp8_encode(vals)
    for v, c in zip(vals, mine):
        assert int(c) == _brute_encode(float(v)), (v, c)


def test_encode_known_ties():
    # 1.0625 lies half way between 1.0 (m=0) and 1.125 (m=1): even -> 1.0
    # 1.1875 lies half way between 1.125 (m=1) and 1.25 (m=2): even -> 1.25
    assert fp8_decode(fp8_encode([1.0625, 1.1875])).tolist() == [1.0, 1.25]
    # subnormal tie 1.5 * 2**-9 -> 2 * 2**-9 (even)
    assert fp8_decode(fp8_encode([1.5 * 2.0 ** -9]))[0] == 2 * 2.0 ** -9


def test_encode_matches_torch_random():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000) * 4,
        rng.standard_normal(20000) * 2.0 ** -7,     # subnormal range
        rng.uniform(-464, 464, 20000),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_encode(x), ref)


def test_encode_saturates_and_rejects_nan():
    assert fp8_encode([1e30, -1e30, 449.0, 470.0]).tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    with pytest.raises(ValueError):
        fp8_encode([float("nan")])


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8_encode(fp8_decode(codes)), codes)
