"""Pins for the oracle's number formats: e4m3 decode/encode and BF16 rounding.

Pinned against: the OCP E4M3 definition (golden table), exhaustive
round-trips, the ties-to-even rule at every midpoint, and torch's own CPU
casts (a library routine) for in-range values.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16_round, e4m3_decode, e4m3_encode, f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    # signs of zero
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def test_golden_special_values():
    doc = json.load(open(os.path.join(GOLDEN, "e4m3_special_values.json")))
    for d in doc["decode"]:
        assert e4m3_decode([int(d["code"], 16)])[0] == d["value"], d
    for c in doc["nan_codes"]:
        assert np.isnan(e4m3_decode([int(c, 16)])[0])
    for d in doc["encode"]:
        assert int(e4m3_encode([d["value"]])[0]) == int(d["code"], 16), d


def test_roundtrip_every_finite_code():
    vals = e4m3_decode(FINITE)
    assert np.array_equal(e4m3_encode(vals), np.array(FINITE, np.uint8))


def test_midpoints_round_to_even():
    # Every midpoint between neighbouring non-negative codes goes to the code
    # with the even mantissa; just above / below goes to the nearer code.
    pos = list(range(0, 0x7F))
    for lo, hi in zip(pos[:-1], pos[1:]):
        a, b = e4m3_decode([lo, hi])
        mid = (a + b) / 2
        want = lo if lo % 2 == 0 else hi
        assert int(e4m3_encode([mid])[0]) == want, (lo, hi)
        assert int(e4m3_encode([-mid])[0]) == want | 0x80
        eps = (b - a) * 2.0**-10
        assert int(e4m3_encode([mid - eps])[0]) == lo
        assert int(e4m3_encode([mid + eps])[0]) == hi


def test_saturation():
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e30])
    assert np.all(e4m3_encode(big) == 0x7E)
    assert np.all(e4m3_encode(-big) == 0xFE)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), size=200_000))
    v = f32(mag * np.where(rng.integers(0, 2, mag.size) == 0, -1, 1))
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), ref)


def test_encode_nearest_bruteforce():
    # Nearest representable value by exhaustive search over all finite codes.
    rng = np.random.default_rng(2)
    v = f32(rng.uniform(-460, 460, size=5000))
    grid = e4m3_decode(FINITE)
    got = e4m3_decode(e4m3_encode(v))
    best = np.min(np.abs(v[:, None] - grid[None, :]), axis=1)
    assert np.all(np.abs(v - got) == best)


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(100_000) * 10.0 ** rng.uniform(-20, 20, 100_000),
        # exact ties: 8 significant bits plus a trailing half
        np.ldexp(rng.integers(128, 256, 1000) * 2 + 1, rng.integers(-30, 30, 1000)),
    ])
    v = f32(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(v), ref)


def test_f32_rounding():
    assert f32(1.0 + 2.0**-24) == 1.0          # tie to even
    assert f32(1.0 + 3 * 2.0**-24) == 1.0 + 2.0**-22
    assert f32(0.1) == np.float32(0.1)


@pytest.mark.parametrize("mutant", ["no_ties_even", "no_saturation"])
def test_codec_pins_catch_planted_mistakes(mutant, monkeypatch):
    """A plausible mistake planted in the oracle's encoder fails a pin."""
    import oracle.codecs as codecs

    real = codecs.e4m3_encode

    def ties_away(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        out = real(v)
        lo = real(a)
        nxt = np.minimum(lo.astype(np.int64) + 1, 0x7E)
        mid = (e4m3_decode(lo) + e4m3_decode(nxt)) / 2
        up = (a == mid) & (lo % 2 == 0) & (a > e4m3_decode(lo))
        return np.where(up, nxt | np.where(np.signbit(v), 0x80, 0), out).astype(np.uint8)

    def no_sat(v):
        out = real(v)
        return np.where(np.abs(np.asarray(v)) > 464.0, 0x7F, out).astype(np.uint8)

    bad = {"no_ties_even": ties_away, "no_saturation": no_sat}[mutant]
    monkeypatch.setattr(codecs, "e4m3_encode", bad)
    monkeypatch.setitem(globals(), "e4m3_encode", bad)
    with pytest.raises(AssertionError):
        test_golden_special_values()
