"""Pins of the boundary-step oracle (oracle/boundary.py): MXFP8 quantisation
of the latent and the reduce + RMSNorm of the combine ("kimi_k3 ... ep.comm"
page, EpDispatch, EpCombine, rms_rstd; the MX scale rule read from the OCP
MX v1.0 definition), against closed forms, brute force and invariants."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import boundary
from oracle.codecs import E4M3_VALUES, bf16_round, e4m3_decode

RNG = np.random.default_rng(7)


def bf16_rows(shape, scale=1.0, rng=RNG):
    return bf16_round(rng.standard_normal(shape) * scale)


# ---- E8M0 ------------------------------------------------------------------

def test_e8m0_closed_form():
    v = boundary.e8m0_decode([0, 1, 126, 127, 128, 254, 255])
    assert v[0] == 2.0**-127 and v[1] == 2.0**-126 and v[2] == 0.5 and v[3] == 1.0
    assert v[4] == 2.0 and v[5] == 2.0**127 and np.isnan(v[6])


# ---- MXFP8 -----------------------------------------------------------------

def brute_e4m3(v):
    """Nearest finite e4m3 value by search over all codes, ties to the even
    code (lowest mantissa bit clear), saturating at 448."""
    finite = np.isfinite(E4M3_VALUES)
    vals, codes = E4M3_VALUES[finite], np.arange(256)[finite]
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(v):
        x = min(max(x, -448.0), 448.0)
        d = np.abs(vals - x)
        best = np.nonzero(d == d.min())[0]
        pick = [c for c in codes[best] if (c & 1) == 0] or list(codes[best])
        # +0 and -0 tie at zero: keep the sign of x
        if len(pick) > 1:
            pick = [c for c in pick if ((c & 0x80) != 0) == (x < 0 or (x == 0 and np.signbit(x)))] or pick
        out[i] = pick[0]
    return out


def test_mxfp8_brute_force_small():
    """Every element is the e4m3 nearest to v / 2^shared with shared =
    floor(log2(block max)) - 8, found by search; the scale byte is shared +
    127."""
    x = bf16_rows((3, 64), scale=5.0)
    q, sf = boundary.mxfp8_quantize(x)
    for t in range(3):
        for b in range(2):
            blk = x[t, 32 * b:32 * b + 32]
            m = np.abs(blk).max()
            k = int(np.floor(np.log2(m)))
            assert sf[t, b] == k - 8 + 127
            want = brute_e4m3(blk / 2.0**(k - 8))
            got = q[t, 32 * b:32 * b + 32]
            same = (got == want) | ((e4m3_decode(got) == 0) & (e4m3_decode(want) == 0))
            assert same.all(), (t, b, got[~same], want[~same])


def test_mxfp8_power_of_two_max_is_identity_on_grid():
    """A block of e4m3 grid values whose max magnitude is 256 (= 2^8) has
    shared exponent 0 (byte 127) and codes equal to the values' own."""
    grid = E4M3_VALUES[np.isfinite(E4M3_VALUES) & (np.abs(E4M3_VALUES) <= 256)]
    blk = RNG.choice(grid, size=32)
    blk[5] = -256.0
    q, sf = boundary.mxfp8_quantize(blk[None, :])
    assert sf[0, 0] == 127
    assert np.array_equal(e4m3_decode(q[0]), blk)


@pytest.mark.parametrize("top,byte,code", [(448.0, 127, 0x7E), (480.0, 127, 0x7E), (496.0, 127, 0x7E),
                                           (512.0, 128, 0x78), (256.0, 127, 0x78), (255.0, 126, 0x7E),
                                           (192.0, 126, 0x7C)])
def test_mxfp8_block_max_band(top, byte, code):
    """The block max after scaling lies in [256, 512): a max of 448..511
    stays (shared exponent 0) and saturates to 448 (0x7E); 512 scales by 1/2
    to 256 (0x78); 255 scales by 2 to 510 and saturates; 192 scales by 2 to
    384 (0x7C). All tops are BF16 values."""
    blk = np.zeros(32)
    blk[3] = top
    blk[7] = 1.0
    q, sf = boundary.mxfp8_quantize(bf16_round(blk)[None, :])
    assert sf[0, 0] == byte and q[0, 3] == code


def test_mxfp8_scaling_invariance():
    """Multiplying a row by 2^k leaves the codes and adds k to every scale
    byte."""
    x = bf16_rows((2, 96), scale=3.0)
    q0, s0 = boundary.mxfp8_quantize(x)
    for k in (-20, -1, 1, 30):
        q, s = boundary.mxfp8_quantize(x * 2.0**k)
        assert np.array_equal(q, q0) and np.array_equal(s.astype(int), s0.astype(int) + k)


def test_mxfp8_zero_block_and_bounds():
    x = bf16_rows((2, 64))
    x[1, 32:] = 0.0
    q, sf = boundary.mxfp8_quantize(x)
    assert sf[1, 1] == 0 and not q[1, 32:].any()
    deq = e4m3_decode(q).reshape(2, 2, 32) * boundary.e8m0_decode(sf)[..., None]
    blk = x.reshape(2, 2, 32)
    # nonzero blocks: the scaled max lies in [256, 512), and every element is within half an e4m3 step
    m = (np.abs(blk).max(axis=2) / boundary.e8m0_decode(sf))
    assert np.all((m[sf > 0] >= 256) & (m[sf > 0] < 512))
    assert np.all(np.abs(deq - blk) <= np.abs(blk) * 2.0**-4 + boundary.e8m0_decode(sf)[..., None] * 2.0**-10)


# ---- reduce + RMSNorm -------------------------------------------------------

def test_reduce_latent_single_partial_is_identity():
    p = bf16_rows((3, 1, 64))
    assert np.array_equal(boundary.reduce_latent(p), p[:, 0])


def test_reduce_latent_exact_sum_rounded_once():
    """Partials whose sum needs more than BF16's 8 bits: the latent is the
    exact sum rounded once (not rounded after every addition)."""
    p = np.zeros((1, 3, 4))
    p[0, :, 0] = [1.0, 2.0**-8, 2.0**-8]       # 1 + 2^-7: exact in BF16
    p[0, :, 1] = [1.0, 2.0**-9, 2.0**-9]       # 1 + 2^-8: a tie, to even -> 1
    p[0, :, 2] = [256.0, 1.0, 0.5]             # 257.5 -> 258 (BF16 step 2 here)
    p[0, :, 3] = [1.0, -1.0, 2.0**-30]         # cancellation keeps the small term
    got = boundary.reduce_latent(p)[0]
    assert list(got) == [1.0 + 2.0**-7, 1.0, 258.0, 2.0**-30]


def test_rms_norm_closed_forms():
    D = 64
    # constant row c with eps = 0: every output is sign(c) * gamma
    x = np.full((1, D), -3.0)
    g = bf16_round(np.linspace(0.5, 2.0, D))
    assert np.array_equal(boundary.rms_norm(x, g, 0.0)[0], -g)
    # rows of +-2^k: rstd = 2^-k exactly
    x = np.where(RNG.integers(0, 2, (2, D)) == 0, -8.0, 8.0)
    assert np.array_equal(boundary.rms_norm(x, np.ones(D), 0.0), x / 8.0)
    # eps inside the root: a zero row stays zero, and a row of 1s with eps = 3 gives 1/2
    assert not boundary.rms_norm(np.zeros((1, D)), g, 1e-5).any()
    assert np.array_equal(boundary.rms_norm(np.ones((1, D)), np.ones(D), 3.0)[0], np.full(D, 0.5))


def test_rms_norm_scale_invariance():
    """With eps = 0 the norm ignores a power-of-two scale of its input."""
    x = bf16_rows((3, 128))
    g = bf16_rows((128,))
    assert np.array_equal(boundary.rms_norm(x * 2.0**9, g, 0.0), boundary.rms_norm(x, g, 0.0))


# ---- planted mistakes fail a pin -------------------------------------------

def test_planted_mistakes_fail_a_pin(monkeypatch):
    # an element exponent off by one (a scaled block max in [128, 256))
    orig = boundary.E4M3_EMAX
    monkeypatch.setattr(boundary, "E4M3_EMAX", orig - 1)
    with pytest.raises(AssertionError):
        test_mxfp8_block_max_band(448.0, 127, 0x7E)
    monkeypatch.setattr(boundary, "E4M3_EMAX", orig)
    # forgetting the mean (sum instead of sum / D)
    real = boundary.rms_norm

    def no_mean(latent, gamma, eps):
        x = np.asarray(latent, dtype=np.float64)
        return bf16_round(x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps) * gamma)

    monkeypatch.setattr(boundary, "rms_norm", no_mean)
    with pytest.raises(AssertionError):
        test_rms_norm_closed_forms()
    monkeypatch.setattr(boundary, "rms_norm", real)
