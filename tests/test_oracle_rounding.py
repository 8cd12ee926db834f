"""Pins for the rounding points the pages fix, checked by exact arithmetic.

The oracle evaluates in float64 and rounds to binary32 where the pages do.
These tests evaluate the same steps in exact rational arithmetic (Python
Fractions, the exponential from the decimal module at 60 digits) and round
each step to binary32 with a rounding routine written here, so they share
nothing with the oracle's float64 route. E4M3 codes come from torch's CPU
float8_e4m3fn cast (a library routine). Points are chosen where the pages'
rounding points change the result, and planted mistakes must fail:

* the routed SwiGLU ("mega_moe" page, hidden_block): exp, 1 + e, the divide
  and the product with up each rounded to FP32 in that order; a SiLU rounded
  once from float64 must fail;
* the hidden requant ("mega_moe" page, hidden_block): q = e4m3(act / s), a
  divide; the reciprocal multiply must fail;
* the activation quant ("mega_moe" page, epilogue): q = e4m3(v * FP32(1/s));
  the divide must fail;
* UE8M0 scale bytes ("shared_expert" page, block_scales): the scale is the
  binary32 with bit pattern byte << 23, so byte 0 is +0.0 and byte 255 +inf.
"""

import struct
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.moe


# --------------------------------------------------------------------------
# Exact helpers (independent of the oracle)
# --------------------------------------------------------------------------

def rn32(q: Fraction) -> Fraction:
    """Nearest binary32 to the rational q, ties to the even significand
    (normal and subnormal range; no overflow handling is needed here)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # e = floor(log2 a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def exp_exact(x: Fraction) -> Fraction:
    """exp(x) to 60 significant digits, as a rational."""
    with localcontext() as ctx:
        ctx.prec = 60
        d = Decimal(x.numerator) / Decimal(x.denominator)
        return Fraction(d.exp())


def as_f32(values):
    return np.asarray(values, dtype=np.float32)


def e4m3_codes(values_f32) -> np.ndarray:
    """torch's e4m3fn byte of each binary32 value (all |v| <= 448 here)."""
    t = torch.from_numpy(np.ascontiguousarray(as_f32(values_f32)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def f32_bits_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


# --------------------------------------------------------------------------
# Routed SwiGLU: FP32 steps
# --------------------------------------------------------------------------

def _silu_points():
    rng = np.random.default_rng(2024)
    gate = np.concatenate([rng.uniform(-16.0, 7.0, 600), rng.uniform(-2.0, 2.0, 600)])
    up = rng.uniform(-7.0, 7.0, gate.size)
    return as_f32(gate), as_f32(up)


def _act_steps(g: float, u: float) -> float:
    """act = (g / (1 + exp(-g))) * u, every operation rounded to binary32."""
    G, U = Fraction(float(g)), Fraction(float(u))
    e = rn32(exp_exact(-G))
    d = rn32(1 + e)
    s = rn32(G / d)
    return float(rn32(s * U))


def _act_once(g: float, u: float) -> float:
    """The same value rounded once from its exact value (a plausible mistake)."""
    G, U = Fraction(float(g)), Fraction(float(u))
    return float(rn32(G / (1 + exp_exact(-G)) * U))


@pytest.fixture(scope="module")
def silu_cases():
    gate, up = _silu_points()
    steps = np.array([_act_steps(g, u) for g, u in zip(gate, up)])
    once = np.array([_act_once(g, u) for g, u in zip(gate, up)])
    return gate, up, steps, once


def test_swiglu_rounds_each_step_to_fp32(silu_cases):
    gate, up, steps, once = silu_cases
    # the points discriminate: step-wise and once-rounded results differ on many
    assert np.count_nonzero(steps != once) >= 100
    h1 = np.stack([up.astype(np.float64), gate.astype(np.float64)], axis=1)  # I = 1: [up | gate]
    got = oracle.swiglu(h1, 1, 7.0)[:, 0]
    bad = np.nonzero(got != steps)[0]
    assert bad.size == 0, f"{bad.size} points differ, first gate={gate[bad[0]]!r} up={up[bad[0]]!r}"


def test_silu_steps_pin_catches_single_rounding(monkeypatch, silu_cases):
    def silu_once(g):
        g = np.asarray(g, dtype=np.float64)
        with np.errstate(over="ignore"):
            return oracle.f32(g / (1.0 + np.exp(-g)))

    monkeypatch.setattr(oracle.moe, "silu_f32", silu_once)
    with pytest.raises(AssertionError):
        test_swiglu_rounds_each_step_to_fp32(silu_cases)


def test_silu_steps_pin_catches_product_rounded_once(monkeypatch, silu_cases):
    def swiglu_once(h1, inter, limit):
        h1 = np.asarray(h1, dtype=np.float64)
        up = np.clip(h1[:, :inter], -limit, limit)
        g = np.minimum(h1[:, inter:], limit)
        with np.errstate(over="ignore"):
            return oracle.f32(g / (1.0 + np.exp(-g)) * up)

    monkeypatch.setattr(oracle, "swiglu", swiglu_once)
    with pytest.raises(AssertionError):
        test_swiglu_rounds_each_step_to_fp32(silu_cases)


# --------------------------------------------------------------------------
# FP8 quantisers: divide (hidden) versus reciprocal multiply (activation)
# --------------------------------------------------------------------------

def _e4m3_midpoints() -> np.ndarray:
    """Midpoints between consecutive positive finite e4m3 values."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0**-9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    vals = np.array(sorted(vals))
    return (vals[:-1] + vals[1:]) / 2


def _disagreeing(values, s):
    """Values whose e4m3 codes differ between v / s and v * FP32(1/s)."""
    v = as_f32(values)
    s32 = np.float32(s)
    by_div = v / s32
    by_inv = v * (np.float32(1.0) / s32)
    return v[e4m3_codes(by_div) != e4m3_codes(by_inv)]


def _exact_block_codes(block, reciprocal: bool):
    """Codes and scale of one 128-value block, from exact arithmetic."""
    amax = max(Fraction(float(abs(v))) for v in block)
    s = rn32(max(amax, Fraction(float(np.float32(1e-10)))) / 448)
    if reciprocal:
        inv = rn32(1 / s)
        q = [rn32(Fraction(float(v)) * inv) for v in block]
    else:
        q = [rn32(Fraction(float(v)) / s) for v in block]
    return e4m3_codes([float(x) for x in q]), float(s)


def _blocks_from(candidates_by_amax):
    rows = []
    for amax, cands in candidates_by_amax:
        cands = cands[np.abs(cands) <= amax][:127]
        row = np.zeros(128, np.float32)
        row[0] = amax
        row[1:1 + cands.size] = cands
        rows.append(row)
    return np.stack(rows)


@pytest.fixture(scope="module")
def hidden_blocks():
    """FP32 activation blocks with many values whose code depends on the
    divide: near e4m3 midpoints, a few FP32 steps either side."""
    mids = _e4m3_midpoints()
    out = []
    for amax in as_f32([3.7, 0.0123, 1000.3, 5.1, 6.9999]):
        s = np.float32(np.float32(amax) / np.float32(448.0))
        base = as_f32(mids * np.float64(s))
        # the FP32 values up to three steps either side of each midpoint * s
        near = np.concatenate([(base.view(np.int32) + d).view(np.float32) for d in range(-3, 4)])
        near = np.concatenate([near, -near])
        out.append((np.float32(amax), _disagreeing(near, s)))
    return _blocks_from(out)


def test_hidden_requant_divides(hidden_blocks):
    blocks = hidden_blocks
    n_disc = sum(_disagreeing(r[1:], np.float32(r[0]) / np.float32(448.0)).size for r in blocks)
    assert n_disc >= 50, "too few discriminating values"
    q, s = oracle.requantize_hidden(blocks.astype(np.float64))
    for i, row in enumerate(blocks):
        want_q, want_s = _exact_block_codes(row, reciprocal=False)
        assert s[i, 0] == want_s
        assert np.array_equal(q[i], want_q), f"block {i}: {np.count_nonzero(q[i] != want_q)} codes differ"


def test_hidden_divide_pin_catches_reciprocal(monkeypatch, hidden_blocks):
    real = oracle.quantize_blocks
    monkeypatch.setattr(oracle, "requantize_hidden",
                        lambda act: real(act, ue8m0=False, reciprocal=True))
    with pytest.raises(AssertionError):
        test_hidden_requant_divides(hidden_blocks)


@pytest.fixture(scope="module")
def bf16_blocks():
    """BF16 activation blocks (x is BF16) whose codes depend on multiplying
    by FP32(1/s) rather than dividing: every positive BF16 value up to amax
    is tried, for amax values drawn from BF16."""
    rng = np.random.default_rng(7)
    all_bf16 = (np.arange(0x3000, 0x4700, dtype=np.uint32) << 16).view(np.float32)  # 2**-31 .. 2**15
    out = []
    found = 0
    for raw in rng.integers(0x3C00, 0x4200, size=400):       # amax in [2**-7, 32)
        amax = np.float32((np.uint32(raw) << 16).view(np.float32))
        s = np.float32(amax / np.float32(448.0))
        cands = all_bf16[(all_bf16 <= amax) & (all_bf16 >= amax * np.float32(2.0**-10))]
        d = _disagreeing(cands, s)
        if d.size:
            out.append((amax, np.concatenate([d, -d])))
            found += d.size
        if found >= 40:
            break
    return _blocks_from(out)


def test_activation_quant_multiplies_by_reciprocal(bf16_blocks):
    blocks = bf16_blocks
    assert blocks.shape[0] >= 3
    q, s = oracle.quantize_blocks(blocks.astype(np.float64), ue8m0=False, reciprocal=True)
    n_disc = 0
    for i, row in enumerate(blocks):
        want_q, want_s = _exact_block_codes(row, reciprocal=True)
        div_q, _ = _exact_block_codes(row, reciprocal=False)
        n_disc += np.count_nonzero(want_q != div_q)
        assert s[i, 0] == want_s
        assert np.array_equal(q[i], want_q), f"block {i}: {np.count_nonzero(q[i] != want_q)} codes differ"
    assert n_disc >= 20


def test_activation_reciprocal_pin_catches_divide(monkeypatch, bf16_blocks):
    real = oracle.quantize_blocks
    monkeypatch.setattr(oracle, "quantize_blocks",
                        lambda v, ue8m0, reciprocal: real(v, ue8m0, reciprocal=False))
    with pytest.raises(AssertionError):
        test_activation_quant_multiplies_by_reciprocal(bf16_blocks)


def test_layer_uses_the_page_quantisers(monkeypatch):
    """moe_decode reaches the quantisers pinned above: x through the
    reciprocal form, the hidden through requantize_hidden."""
    import synth
    from tests.helpers import oracle_layer

    calls = []
    real_q, real_h = oracle.moe.quantize_blocks, oracle.moe.requantize_hidden

    def spy_q(v, ue8m0, reciprocal):
        calls.append(("quantize_blocks", bool(reciprocal)))
        return real_q(v, ue8m0, reciprocal)

    def spy_h(act):
        calls.append(("requantize_hidden", None))
        return real_h(act)

    monkeypatch.setattr(oracle.moe, "quantize_blocks", spy_q)
    monkeypatch.setattr(oracle.moe, "requantize_hidden", spy_h)
    oracle_layer(synth.make_inputs(synth.CONFIGS["tiny"], seed=0))
    assert ("quantize_blocks", True) in calls
    assert ("requantize_hidden", None) in calls


# --------------------------------------------------------------------------
# UE8M0 scale bytes
# --------------------------------------------------------------------------

def _packed_all_bytes():
    """Packed words for n = 128 rows and K = 256 * 128: K block b carries
    exponent byte b (0..255) on every row."""
    nblocks = 256
    words = np.zeros((128, nblocks // 4), np.int64)
    for b in range(nblocks):
        words[:, b // 4] |= b << (8 * (b % 4))
    return (words.astype(np.uint32)).view(np.int32), 128, nblocks * 128


def test_ue8m0_bytes_are_the_exponent_field():
    packed, n, k = _packed_all_bytes()
    got = oracle.unpack_ue8m0(packed, n, k)
    assert got.shape == (1, 256)
    want = np.array([f32_bits_value(b << 23) for b in range(256)])
    assert np.array_equal(got[0], want)
    assert got[0, 0] == 0.0 and not np.signbit(got[0, 0])
    assert np.isposinf(got[0, 255])
    assert got[0, 127] == 1.0 and got[0, 1] == 2.0**-126 and got[0, 254] == 2.0**127


def test_ue8m0_pin_catches_power_of_two_decode(monkeypatch):
    def ldexp_form(packed, n, k):
        words = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
        b = np.arange(k // 128)
        byte = (words[::128][:, b // 4] >> (8 * (b % 4))) & 0xFF
        return np.ldexp(1.0, byte - 127)

    monkeypatch.setattr(oracle, "unpack_ue8m0", ldexp_form)
    with pytest.raises(AssertionError):
        test_ue8m0_bytes_are_the_exponent_field()
